"""The end of the matrix-core decode kernels: the waves that share a kv head
merge their partial softmax states through LDS, with the number of waves per
head (1, 2, 4 or 8) a compile-time parameter chosen at run time from the
plan.  Each case first asks the planner for the (kernel, waves per workgroup,
kv heads per workgroup) it is meant to reach, so every waves-per-head variant
of both kernels and both workgroup widths runs with the automatic plan (one
split here: outputs written by the element pass); the same shapes with three
splits (16-byte partial stores, then the combine), and an output that is only
2-byte aligned (element stores instead of 8-byte ones).  Against the f64 oracle."""

import numpy as np
import pytest
import torch

import oracle.paged_attention as O
import paged_kv_cache_195_amd as pa
from gpu_helpers import host, host_caches, say
from paged_kv_cache_195_amd.workloads import make_custom
from tolerance import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (batch, Hq, Hkv, q dtype, kernel, waves per workgroup, kv heads per workgroup)
CASES = [
    (256, 32, 8, "bf16", "mfma", 8, 8),             # one wave per kv head
    (128, 32, 8, "f16", "mfma", 8, 4),              # two
    (64, 32, 8, "bf16", "mfma", 8, 2),              # four
    (32, 32, 8, "bf16", "mfma", 8, 1),              # eight
    (256, 64, 4, "bf16", "mfma", 4, 4),             # 4-wave workgroups: one wave per head
    (128, 64, 4, "f16", "mfma", 4, 2),              # two
    (64, 64, 4, "bf16", "mfma", 4, 1),              # four
    (256, 32, 1, "bf16", "mfma_two_blocks", 8, 1),  # two row blocks per wave: eight waves per head
    (256, 64, 2, "f16", "mfma_two_blocks", 8, 2),   # four
    (256, 96, 4, "bf16", "mfma_two_blocks", 8, 4),  # two
    (256, 160, 8, "bf16", "mfma_two_blocks", 8, 8), # one, G = 20: 12 padding rows per block pair
]


def _run(case, splits, unaligned):
    batch, hq, hkv, dtype, kernel, waves, kpw = case
    rng = np.random.default_rng(batch * 7 + hq)
    lens = rng.integers(0, 161, size=batch).tolist()
    lens[0], lens[-1] = 160, 0
    say(f"wave merge: B={batch} Hq={hq} Hkv={hkv} {dtype} S={splits} unaligned={unaligned}")
    w = make_custom(dtype, lens, hq, hkv, 128, 16, seed=91, device=DEV)
    shape = pa.make_shape(w.q, w.k_cache, w.v_cache, w.block_table)
    plan = pa.describe_plan(shape, splits)
    assert (plan["kernel"], plan["waves"]) == (kernel, waves)
    if splits == 0:  # with three splits the grid is wider and the planner may keep more heads
        assert plan["kv_heads_per_workgroup"] == kpw
    out = None
    if unaligned:  # a view one element into its buffer: 2-byte aligned, not 8-byte
        buf = torch.empty(w.q.numel() + 1, dtype=w.q.dtype, device=DEV)
        out = buf[1:].view(w.q.shape)
    o, lse = pa.decode(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale,
                       num_splits=splits, out=out, num_pages=w.num_pages_arg)
    torch.cuda.synchronize()
    k, v = host_caches(w)
    xo, xl = O.attention(host(w.q), k, v, w.table_host.numpy(), np.array(lens), w.scale, False)
    assert_close(o, xo, w.q.dtype, "out")
    assert_close(lse, xl, torch.float32, "lse")


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[4]}-W{c[5]}-kpw{c[6]}-{c[3]}")
@pytest.mark.parametrize("splits", [0, 3])
def test_wave_merge(case, splits):
    _run(case, splits, unaligned=False)


@pytest.mark.parametrize("case", [CASES[3], CASES[6], CASES[7]],
                         ids=lambda c: f"{c[4]}-W{c[5]}-kpw{c[6]}-{c[3]}")
def test_wave_merge_unaligned_output(case):
    _run(case, 0, unaligned=True)
