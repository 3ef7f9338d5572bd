"""Seeded random sweep of the supported envelope against the f64 oracle.

Each case draws every knob at once -- query dtype, 8-bit K/V codes, head dim,
page size, kv heads and group size (odd ones included), batch, decode or
prefill with up to 100 query rows, ragged lengths (empty ones included),
causal masking, prefix offsets, the split count (automatic, 1, or 2..9), table
slack and row stride -- so that combinations no targeted test names (8-bit
prefill, prefix offsets across splits, odd groups under the automatic plan)
still meet the parity bar.  A second set draws wide batches (at least 128
sequence-kv-head pairs) with 17 to 63 query rows per kv head, the envelope of
the two-block kernel, and checks with the planner that they take it.  The
draws depend only on the case index.
"""

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
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
N_CASES = 256
N_WIDE_CASES = 32


def draw(i):
    rng = np.random.default_rng(7000 + i)
    dtype = str(rng.choice(["f32", "f16", "bf16"], p=[0.2, 0.35, 0.45]))
    kv = None
    if dtype != "f32" and rng.random() < 0.3:
        kv = str(rng.choice(["int8", "fp8_e4m3"]))
    d = int(rng.choice([64, 128] if kv else [32, 64, 128]))
    ps = int(rng.choice([16, 32]))
    hkv = int(rng.choice([1, 2, 3, 4, 5, 8]))
    g = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    batch = int(rng.integers(1, 7))
    prefill = rng.random() < 0.4
    seq_q = int(rng.integers(2, 101)) if prefill else 1
    lens = rng.integers(0, 601, size=batch)
    if rng.random() < 0.3:
        lens[int(rng.integers(batch))] = 0
    lens = [int(x) for x in lens]
    causal = bool(rng.random() < (0.85 if prefill else 0.3))
    prefix = None
    if rng.random() < 0.2:
        prefix = [int(rng.integers(-20, L + 21)) for L in lens]
    r = rng.random()
    splits = 0 if r < 0.4 else (1 if r < 0.7 else int(rng.integers(2, 10)))
    n_max = max([-(-L // ps) for L in lens] + [1])
    width = n_max + int(rng.integers(0, 4))
    stride = width + int(rng.integers(0, 3))
    return dict(dtype=dtype, kv=kv, d=d, ps=ps, hkv=hkv, hq=hkv * g, batch=batch, seq_q=seq_q,
                lens=lens, causal=causal, prefix=prefix, splits=splits, width=width,
                stride=stride)


def draw_wide(i):
    """Batches of at least 128 (sequence, kv head) pairs at small lengths with
    17 to 32 query rows per kv head (16-bit decode, 16-bit chunks of several
    queries at D = 32) or 17 to 63 (8-bit caches): the two-block kernel."""
    rng = np.random.default_rng(9100 + i)
    kv = [None, None, "int8", "fp8_e4m3"][int(rng.integers(4))]
    dtype = str(rng.choice(["f16", "bf16"]))
    d = int(rng.choice([64, 128] if kv else [32, 64, 128]))
    ps = int(rng.choice([16, 32]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    max_rows = 63 if kv else 32
    if (kv or d == 32) and rng.random() < 0.4:
        seq_q = int(rng.integers(2, 9))
        g = int(rng.integers(-(-17 // seq_q), max_rows // seq_q + 1))
    else:
        seq_q = 1
        g = int(rng.integers(17, max_rows + 1))
    batch = -(-128 // hkv) + int(rng.integers(0, 24))
    lens = [int(x) for x in rng.integers(0, 161, size=batch)]
    lens[int(rng.integers(batch))] = 0
    causal = bool(seq_q > 1 and rng.random() < 0.8)
    prefix = None
    if rng.random() < 0.25:
        prefix = [int(rng.integers(-10, L + 11)) for L in lens]
    r = rng.random()
    splits = 0 if r < 0.4 else (1 if r < 0.7 else int(rng.integers(2, 7)))
    n_max = max([-(-L // ps) for L in lens] + [1])
    width = n_max + int(rng.integers(0, 4))
    stride = width + int(rng.integers(0, 3))
    return dict(dtype=dtype, kv=kv, d=d, ps=ps, hkv=hkv, hq=hkv * g, batch=batch, seq_q=seq_q,
                lens=lens, causal=causal, prefix=prefix, splits=splits, width=width,
                stride=stride)


def run_case(c, seed, want_kernel=None):
    w = make_custom(c["dtype"], c["lens"], c["hq"], c["hkv"], c["d"], c["ps"], seq_q=c["seq_q"],
                    causal=c["causal"], width=c["width"], table_stride=c["stride"],
                    seed=seed, device=DEV, kv=c["kv"])
    if want_kernel is not None:
        shape = pa.make_shape(w.q, w.k_cache, w.v_cache, w.block_table)
        assert pa.describe_plan(shape, c["splits"])["kernel"] == want_kernel
    fn = pa.decode if c["seq_q"] == 1 else pa.prefill
    po = None if c["prefix"] is None else torch.tensor(c["prefix"], dtype=torch.int32, device=DEV)
    out, lse = fn(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale,
                  causal=c["causal"], num_splits=c["splits"], num_pages=w.num_pages_arg,
                  prefix_offset=po, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    k, v = host_caches(w)
    xo, xl = O.attention(host(w.q), k, v, w.table_host.numpy(), np.array(w.seq_lens_host),
                         w.scale, c["causal"], prefix_offset=c["prefix"])
    assert_close(out, xo, TDT[c["dtype"]], "out")
    assert_close(lse, xl, torch.float32, "lse")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_envelope_case(i):
    c = draw(i)
    say(f"sweep case {i}: {c}")
    run_case(c, 500 + i)


@pytest.mark.parametrize("i", range(N_WIDE_CASES))
def test_random_wide_batch_case(i):
    c = draw_wide(i)
    say(f"wide-batch sweep case {i}: {c}")
    run_case(c, 900 + i, want_kernel="mfma_two_blocks")
