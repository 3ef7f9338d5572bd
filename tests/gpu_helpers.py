"""Helpers for GPU parity tests: host copies for the oracle, sampling of large caches."""

from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np
import torch

import oracle.paged_attention as O
from tolerance import assert_close


def say(msg: str):
    """Name the case before a GPU step, flushed, so a failing run still says what ran."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def host_caches(w):
    """Float64 host copies of a workload's K and V caches; 8-bit caches are
    dequantized by the oracle (codes times their page's scale)."""
    if w.kv is None:
        return host(w.k_cache), host(w.v_cache)
    return tuple(O.dequantize_cache(c.view(torch.uint8).cpu().numpy(), sc.cpu().numpy(), w.kv)
                 for c, sc in ((w.k_cache, w.k_scale), (w.v_cache, w.v_scale)))


class HostPages:
    """The pages of a device cache that a set of block-table rows references,
    copied to host and indexed by physical page id (what the oracle's gather
    needs: ``cache[page_id]`` and ``cache.shape``).  With ``scales`` and
    ``kind`` the pages hold 8-bit codes and are dequantized by the oracle."""

    def __init__(self, cache: torch.Tensor, page_ids, scales=None, kind=None):
        ids = sorted({int(x) for x in page_ids})
        idx = torch.tensor(ids, dtype=torch.long, device=cache.device)
        if kind is None:
            pages = cache.index_select(0, idx).float().cpu().numpy()
        else:
            codes = cache.view(torch.uint8).index_select(0, idx).cpu().numpy()
            pages = O.dequantize_cache(codes, scales.index_select(0, idx).cpu().numpy(), kind)
        self._map = {pid: pages[i] for i, pid in enumerate(ids)}
        self.shape = tuple(cache.shape)

    def __getitem__(self, pid):
        return self._map[int(pid)]


def referenced_pages(table_host: torch.Tensor, seq_lens, batch_ids, page_size):
    ids = []
    for b in batch_ids:
        n = -(-int(seq_lens[b]) // page_size)
        ids.extend(table_host[b, :n].tolist())
    return ids


def oracle_full(w, causal=None):
    """Oracle (out, lse) for every sequence of a small workload."""
    causal = w.causal if causal is None else causal
    k, v = host_caches(w)
    return O.attention(host(w.q), k, v, w.table_host.numpy(), np.array(w.seq_lens_host), w.scale,
                       causal)


def oracle_splits(w, splits, causal=None):
    causal = w.causal if causal is None else causal
    k, v = host_caches(w)
    return O.split_partials(host(w.q), k, v, w.table_host.numpy(), np.array(w.seq_lens_host),
                            w.scale, causal, splits)


def oracle_workers() -> int:
    """Threads for the oracle: the host cores this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def compare_every_sequence(w, out, lse, chunk=32, rows_per_task=128):
    """Every output element and LSE of a large workload against the oracle.

    Sequences are taken ``chunk`` at a time: the pages they reference are
    copied to host (8-bit codes dequantized by the oracle), then the oracle
    runs over every (sequence, block of ``rows_per_task`` query rows) on a
    thread pool.  A causal block of rows starting at row ``i0`` is the oracle's
    prefix-causal attention with offset ``L - Sq + i0``, which is bottom-right
    causal masking for those rows.  Returns the largest |out error|."""
    from threadpoolctl import threadpool_limits

    out_h = out.float().cpu().numpy()
    lse_h = lse.float().cpu().numpy()
    q = host(w.q)
    batch, seq_q = q.shape[0], q.shape[1]
    ps = w.k_cache.shape[1]
    worst = 0.0
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(max_workers=oracle_workers()) as ex:
        for c0 in range(0, batch, chunk):
            ids = list(range(c0, min(c0 + chunk, batch)))
            pages = referenced_pages(w.table_host, w.seq_lens_host, ids, ps)
            kp = HostPages(w.k_cache, pages, w.k_scale, w.kv)
            vp = HostPages(w.v_cache, pages, w.v_scale, w.kv)
            tasks = [(b, i0, min(i0 + rows_per_task, seq_q)) for b in ids
                     for i0 in range(0, seq_q, rows_per_task)]

            def one(task):
                b, i0, i1 = task
                length = w.seq_lens_host[b]
                prefix = [length - seq_q + i0] if w.causal else None
                return O.attention(q[b:b + 1, i0:i1], kp, vp, w.table_host[b:b + 1].numpy(),
                                   np.array([length]), w.scale, w.causal, prefix_offset=prefix)

            for (b, i0, i1), (xo, xl) in zip(tasks, ex.map(one, tasks)):
                err = assert_close(out_h[b, i0:i1], xo[0], w.q.dtype,
                                   f"out, sequence {b} rows {i0}..{i1 - 1}")
                assert_close(lse_h[b, i0:i1], xl[0], torch.float32,
                             f"lse, sequence {b} rows {i0}..{i1 - 1}")
                worst = max(worst, err)
            del kp, vp
    return worst
