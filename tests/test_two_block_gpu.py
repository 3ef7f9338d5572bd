"""The matrix-core kernel with two 16-row blocks per wave (17 to 32 query rows
per kv head share each staged K/V tile), used over batches of at least 128
(sequence, kv head) pairs: decode at group sizes 17..32, and 8-bit caches with
17 to 63 rows; plus a small 8-bit batch that keeps one block per wave.  Against
the f64 oracle, with the split partials for S > 1."""

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

# (q dtype, kv codes, D, page, Hq, Hkv, batch, Sq)
CASES = [
    ("bf16", None, 128, 16, 24, 1, 128, 1),          # G = 24, 4-wave workgroups
    ("f16", None, 64, 32, 160, 8, 16, 1),            # G = 20, 8-wave workgroups
    ("bf16", None, 128, 16, 256, 8, 16, 1),          # G = 32: one full row group
    ("bf16", None, 32, 16, 17, 1, 130, 1),           # G = 17, D = 32
    ("bf16", "int8", 128, 16, 48, 2, 64, 1),         # 8-bit, G = 24
    ("f16", "fp8_e4m3", 64, 16, 80, 2, 64, 1),       # 8-bit, G = 40: two row groups of 32
    ("bf16", "int8", 128, 16, 32, 8, 16, 6),         # 8-bit chunk of 6 queries: 24 rows
    ("bf16", "int8", 128, 16, 48, 2, 4, 1),          # small batch: one row block per wave
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-D{c[2]}-G{c[4] // c[5]}-B{c[6]}-Sq{c[7]}")
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_two_row_blocks_per_wave(case, splits):
    dtype, kv, d, ps, hq, hkv, batch, sq = case
    rng = np.random.default_rng(hq * 131 + batch)
    lens = rng.integers(0, 301, size=batch).tolist()
    lens[0], lens[-1] = 300, 0
    causal = sq > 1
    say(f"two row blocks: {dtype} kv={kv} D={d} ps={ps} Hq={hq} Hkv={hkv} B={batch} Sq={sq} "
        f"S={splits}")
    w = make_custom(dtype, lens, hq, hkv, d, ps, seq_q=sq, causal=causal, seed=71, device=DEV,
                    kv=kv)
    shape = pa.make_shape(w.q, w.k_cache, w.v_cache, w.block_table)
    s = pa.resolve_num_splits(shape, splits)
    fn = pa.decode if sq == 1 else pa.prefill
    out, lse, ws = fn(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale,
                      causal=causal, num_splits=splits, num_pages=w.num_pages_arg,
                      return_workspace=True, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    k, v = host_caches(w)
    args = (host(w.q), k, v, w.table_host.numpy(), np.array(lens), w.scale, causal)
    xo, xl = O.attention(*args)
    assert_close(out, xo, w.q.dtype, "out")
    assert_close(lse, xl, torch.float32, "lse")
    if s > 1:
        rows = w.q.shape[0] * w.q.shape[1] * w.q.shape[2]
        po, pl = pa.split_views(ws, rows, s, w.v_cache.shape[3])
        xo, xl = O.split_partials(*args, s)
        assert_close(po, xo.reshape(rows, s, -1), w.q.dtype, "part_out")
        assert_close(pl, xl.reshape(rows, s), w.q.dtype, "part_lse")
