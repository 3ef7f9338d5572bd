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


class HostPages:
    """The pages of a device cache that a set of block-table rows references,
    copied to host and indexed by physical page id (what the oracle's gather
    needs: ``cache[page_id]`` and ``cache.shape``)."""

    def __init__(self, cache: torch.Tensor, page_ids):
        ids = sorted({int(x) for x in page_ids})
        idx = torch.tensor(ids, dtype=torch.long, device=cache.device)
        pages = cache.index_select(0, idx).float().cpu().numpy()
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
    return O.attention(host(w.q), host(w.k_cache), host(w.v_cache), w.table_host.numpy(),
                       np.array(w.seq_lens_host), w.scale, causal)


def oracle_splits(w, splits, causal=None):
    causal = w.causal if causal is None else causal
    return O.split_partials(host(w.q), host(w.k_cache), host(w.v_cache), w.table_host.numpy(),
                            np.array(w.seq_lens_host), w.scale, causal, splits)


def oracle_sampled(w, batch_ids):
    """Oracle (out, lse) for the sequences ``batch_ids`` of a large workload,
    reading only the pages those sequences reference."""
    ps = w.k_cache.shape[1]
    ids = referenced_pages(w.table_host, w.seq_lens_host, batch_ids, ps)
    kp = HostPages(w.k_cache, ids)
    vp = HostPages(w.v_cache, ids)
    q = host(w.q[list(batch_ids)])
    table = w.table_host[list(batch_ids)].numpy()
    lens = np.array([w.seq_lens_host[b] for b in batch_ids])
    return O.attention(q, kp, vp, table, lens, w.scale, w.causal)
