"""GPU parity of the optional inputs (pa_decode_ex / pa_prefill_ex): prefix
offsets and the page-id range check, against the f64 oracle.

Out-of-range page ids are made by telling the library fewer pages than the
caches hold, and rows given out-of-range lengths have valid ids in every slot
of their storage, so an id that slipped through the check would still name
allocated memory: a failure shows up as a wrong value, never as a fault.
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


def oracle(w, causal, prefix=None, lens=None, splits=None):
    lens = np.array(w.seq_lens_host if lens is None else lens)
    k, v = host_caches(w)
    args = (host(w.q), k, v, w.table_host.numpy(), lens, w.scale, causal)
    if splits is None:
        return O.attention(*args, prefix_offset=prefix)
    return O.split_partials(*args, splits, prefix_offset=prefix)


def call(w, causal, splits=0, prefix=None, page_check=None, num_pages=None, decode=None):
    decode = w.q.shape[1] == 1 if decode is None else decode
    fn = pa.decode if decode else pa.prefill
    po = None if prefix is None else torch.tensor(prefix, dtype=torch.int32, device=DEV)
    res = fn(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale, causal=causal,
             num_splits=splits, num_pages=w.num_pages_arg if num_pages is None else num_pages,
             return_workspace=True, prefix_offset=po, page_check=page_check, k_scale=w.k_scale,
             v_scale=w.v_scale)
    torch.cuda.synchronize()
    return res


def check_split_partials(w, splits, ws, causal, prefix=None, lens=None):
    rows = w.q.shape[0] * w.q.shape[1] * w.q.shape[2]
    dv = w.v_cache.shape[3]
    po, pl = pa.split_views(ws, rows, splits, dv)
    xo, xl = oracle(w, causal, prefix, lens, splits)
    # the tolerance of the problem's dtype applies to its float32 partials too
    assert_close(po, xo.reshape(rows, splits, dv), w.q.dtype, "part_out")
    assert_close(pl, xl.reshape(rows, splits), w.q.dtype, "part_lse")


# (dtype, D, page, Hq, Hkv, Sq, lens, prefix): the three kernels (the vector-ALU one
# for f32, the matrix-core decode kernel for 16-bit caches, the shared-tile prefill
# kernel from 64 rows per kv head) with offsets before the first key, inside, at
# L - Sq and past the end.
PREFIX_CASES = [
    ("f32", 64, 16, 4, 2, 3, [37, 200, 90], [-5, 120, 87]),
    ("bf16", 128, 16, 8, 2, 2, [100, 300, 17], [50, -1, 15]),
    ("f16", 128, 32, 16, 2, 5, [64, 500, 33], [10, 495, 40]),
    ("bf16", 64, 16, 32, 8, 3, [260, 77], [100, 3]),
    ("bf16", 128, 16, 32, 8, 40, [300, 41, 1000], [250, -30, 500]),
    ("f16", 64, 32, 4, 1, 96, [96, 400], [0, 1000]),
]


@pytest.mark.parametrize("case", PREFIX_CASES, ids=lambda c: f"{c[0]}-G{c[3] // c[4]}-Sq{c[5]}")
@pytest.mark.parametrize("splits", [1, 3])
def test_prefix_offset(case, splits):
    dtype, d, ps, hq, hkv, sq, lens, prefix = case
    say(f"prefix offset {dtype} D={d} ps={ps} Hq={hq} Hkv={hkv} Sq={sq} lens={lens} "
        f"prefix={prefix} S={splits}")
    w = make_custom(dtype, lens, hq, hkv, d, ps, seq_q=sq, seed=31, device=DEV)
    # causal=False on purpose: a prefix offset turns prefix-causal masking on
    out, lse, ws = call(w, False, splits, prefix=prefix, decode=False)
    xo, xl = oracle(w, False, prefix)
    assert_close(out, xo, TDT[dtype], "out")
    assert_close(lse, xl, torch.float32, "lse")
    if splits > 1:
        check_split_partials(w, splits, ws, False, prefix)


def test_prefix_offset_decode():
    """Decode (Sq = 1) with offsets: the new token sees keys 0..offset."""
    lens = [700, 33, 1000, 16, 250]
    prefix = [699, 10, -1, 15, 100]
    say(f"prefix offset decode bf16 lens={lens} prefix={prefix}")
    w = make_custom("bf16", lens, 32, 8, 128, 16, seed=32, device=DEV)
    for splits in (1, 4):
        out, lse, ws = call(w, False, splits, prefix=prefix, decode=True)
        xo, xl = oracle(w, False, prefix)
        assert_close(out, xo, torch.bfloat16, "out")
        assert_close(lse, xl, torch.float32, "lse")
        if splits > 1:
            check_split_partials(w, splits, ws, False, prefix)


@pytest.mark.parametrize("hq,sq", [(8, 3), (32, 4), (32, 64)])
def test_prefix_bottom_right_bit_identical(hq, sq):
    """prefix_offset = L - Sq reproduces causal masking bit for bit, in every kernel."""
    lens = [300, 130, 64]
    say(f"prefix = L - Sq vs causal, bf16 Hq={hq} Hkv=8 Sq={sq}")
    w = make_custom("bf16", lens, hq, 8, 128, 16, seq_q=sq, seed=33, device=DEV)
    a_out, a_lse, _ = call(w, True, 2, decode=False)
    b_out, b_lse, _ = call(w, False, 2, prefix=[x - sq for x in lens], decode=False)
    assert torch.equal(a_out, b_out) and torch.equal(a_lse, b_lse)


def test_page_check_all_pass_is_identical():
    lens = [0, 17, 300, 999]
    say(f"page check, all valid, lens={lens}")
    w = make_custom("bf16", lens, 32, 8, 128, 16, width=63, seed=34, device=DEV)
    res = torch.full((len(lens) + 1,), 12345, dtype=torch.int32, device=DEV)
    for splits in (1, 5):
        a_out, a_lse, _ = call(w, False, splits)
        b_out, b_lse, _ = call(w, False, splits, page_check=res)
        assert res.tolist() == [-1] + lens
        assert torch.equal(a_out, b_out) and torch.equal(a_lse, b_lse)


@pytest.mark.parametrize("splits", [1, 3])
def test_page_check_out_of_range_ids(splits):
    """Ids at or past the stated page count fail their sequence: it is attended
    as empty, and page_check names the first failing sequence."""
    lens = [200, 513, 90, 16, 0, 777, 45, 300]
    w = make_custom("bf16", lens, 32, 8, 128, 16, width=63, extra_pages=0, seed=35, device=DEV)
    phys = w.notes["true_num_pages"]
    table = w.table_host.numpy()
    # state fewer pages than exist: ids >= stated are out of range (still
    # allocated).  The median of the sequences' largest ids splits them into
    # passing and failing ones.
    top = sorted(max(table[b, : -(-x // 16)]) for b, x in enumerate(lens) if x > 0)
    stated = int(top[len(top) // 2])
    first_bad, att = O.check_pages(table, w.seq_lens_host, 16, stated, table.shape[1])
    assert 0 <= first_bad and 0 < sum(a != x for a, x in zip(att, lens)) < len(lens)
    assert stated < phys
    say(f"page check ids: stated {stated} of {phys} pages, expect first_bad={first_bad} "
        f"lens={att} S={splits}")
    res = torch.zeros(len(lens) + 1, dtype=torch.int32, device=DEV)
    out, lse, ws = call(w, False, splits, page_check=res, num_pages=stated)
    assert res.tolist() == [first_bad] + att
    xo, xl = oracle(w, False, lens=att)
    assert_close(out, xo, torch.bfloat16, "out")
    assert_close(lse, xl, torch.float32, "lse")
    if splits > 1:
        check_split_partials(w, splits, ws, False, lens=att)


def test_page_check_lengths_and_prefill():
    """Lengths outside [0, W * page_size] fail unread; prefill with prefix
    offsets and the check together."""
    lens = [64, 130, 40, 96]
    width = 9
    w = make_custom("f16", lens, 16, 2, 64, 16, seq_q=24, width=width, table_stride=width + 1,
                    seed=36, device=DEV)
    storage = w.notes["table_storage"]
    rows = storage[: len(lens) * (width + 1)].view(len(lens), width + 1)
    # rows 1 and 2 get bad lengths; every slot of their storage rows names a real page
    rows[1, :] = rows[1, 0]
    rows[2, :] = rows[2, 0]
    torch.cuda.synchronize()
    w.table_host = w.block_table.cpu()
    bad_lens = [64, width * 16 + 1, -3, 96]
    w.seq_lens = torch.tensor(bad_lens, dtype=torch.int32, device=DEV)
    w.seq_lens_host = bad_lens
    first_bad, att = O.check_pages(w.table_host.numpy(), bad_lens, 16, w.num_pages_arg, width)
    assert (first_bad, att) == (1, [64, 0, 0, 96])
    prefix = [50, 0, 0, 60]
    say(f"page check lengths {bad_lens} + prefix {prefix}, f16 Sq=24 G=8")
    for splits in (1, 2):
        res = torch.zeros(len(lens) + 1, dtype=torch.int32, device=DEV)
        out, lse, ws = call(w, False, splits, prefix=prefix, page_check=res, decode=False)
        assert res.tolist() == [first_bad] + att
        xo, xl = oracle(w, False, prefix, lens=att)
        assert_close(out, xo, torch.float16, "out")
        assert_close(lse, xl, torch.float32, "lse")
        if splits > 1:
            check_split_partials(w, splits, ws, False, prefix, lens=att)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_variable_length_queries_by_padding(dtype):
    """Sequences with their own query counts, padded to one Sq: with
    prefix_offset[b] = L_b - q_b the first q_b rows of sequence b equal a causal
    prefill of just those q_b queries (the padding rows are computed and
    ignored)."""
    lens = [300, 64, 150, 1000]
    qlens = [5, 64, 20, 37]
    sq = 64
    say(f"variable-length queries by padding, {dtype}, lens={lens} q={qlens}")
    w = make_custom(dtype, lens, 32, 8, 128, 16, seq_q=sq, seed=37, device=DEV)
    prefix = [x - q for x, q in zip(lens, qlens)]
    k, v = host_caches(w)
    qh = host(w.q)
    table = w.table_host.numpy()
    for splits in (1, 3):
        out, lse, _ = call(w, False, splits, prefix=prefix, decode=False)
        for b, (length, q) in enumerate(zip(lens, qlens)):
            xo, xl = O.attention(qh[b:b + 1, :q], k, v, table[b:b + 1], np.array([length]),
                                 w.scale, True)
            assert_close(out[b:b + 1, :q], xo, TDT[dtype], f"out b={b}")
            assert_close(lse[b:b + 1, :q], xl, torch.float32, f"lse b={b}")
