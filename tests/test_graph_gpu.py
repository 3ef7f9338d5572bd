"""Decode and prefill captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay, with new query values written eagerly and the device
synchronised between replays, must equal an eager call on the same inputs
bit for bit and meet the parity bar against the oracle.  The captured decode
splits (S > 1), so the graph holds the attention kernel and the combine."""

import numpy as np
import pytest
import torch

import paged_kv_cache_195_amd as pa
from gpu_helpers import oracle_full, say
from paged_kv_cache_195_amd.workloads import make_custom
from tolerance import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_graph_replays_match_eager(kind):
    if kind == "decode":
        w = make_custom("bf16", [37, 500, 0, 1000], 32, 8, 128, 16, seed=61, device=DEV)
        fn_api, causal = pa.decode, False
    else:
        w = make_custom("bf16", [100, 64, 300], 32, 8, 128, 16, seq_q=64, causal=True,
                        seed=62, device=DEV)
        fn_api, causal = pa.prefill, True
    shape = pa.make_shape(w.q, w.k_cache, w.v_cache, w.block_table)
    splits = pa.resolve_num_splits(shape, 0)
    say(f"graph {kind}: automatic S={splits}")
    if kind == "decode":
        assert splits > 1
    work = torch.empty(max(pa.workspace_bytes(shape, 0), 1), dtype=torch.uint8, device=DEV)
    out = torch.empty((w.q.shape[0], w.q.shape[1], w.q.shape[2], w.v_cache.shape[3]),
                      dtype=w.q.dtype, device=DEV)
    lse = torch.empty(out.shape[:3], dtype=torch.float32, device=DEV)

    def step():
        fn_api(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale, causal=causal,
               out=out, lse=lse, workspace=work)

    g = _capture(step)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(63)
    for r in range(4):
        # eager work between replays: new queries, then a full synchronisation
        w.q.copy_(torch.randn(w.q.shape, generator=gen, device=DEV).to(w.q.dtype))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = fn_api(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale,
                                  causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: out differs from the eager call"
        assert torch.equal(lse.nan_to_num(), ref_lse.nan_to_num()), f"replay {r}: lse differs"
        assert torch.equal(torch.isinf(lse), torch.isinf(ref_lse))
        if r in (0, 3):
            xo, xl = oracle_full(w, causal)
            assert_close(out, xo, torch.bfloat16, f"replay {r} out")
            assert_close(lse, xl, torch.float32, f"replay {r} lse")
