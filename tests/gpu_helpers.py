"""Helpers for GPU parity tests: host copies for the oracle, sampling of large caches."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle.paged_attention as O


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


def oracle_sampled(w, batch_ids):
    """Oracle (out, lse) for the sequences ``batch_ids`` of a large workload,
    reading only the pages those sequences reference."""
    ps = w.k_cache.shape[1]
    ids = referenced_pages(w.table_host, w.seq_lens_host, batch_ids, ps)
    kp = HostPages(w.k_cache, ids, w.k_scale, w.kv)
    vp = HostPages(w.v_cache, ids, w.v_scale, w.kv)
    q = host(w.q[list(batch_ids)])
    table = w.table_host[list(batch_ids)].numpy()
    lens = np.array([w.seq_lens_host[b] for b in batch_ids])
    return O.attention(q, kp, vp, table, lens, w.scale, w.causal)
