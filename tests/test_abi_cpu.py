"""libpa.so loads, exports every declared symbol, and rejects bad arguments on the
host before launching anything (no GPU needed: every call here fails validation)."""

import ctypes
import math
import os
import re

import pytest

import paged_kv_cache_195_amd as pa
from paged_kv_cache_195_amd.api import PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PaShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = pa.load_library()
    names = declared_functions()
    assert names == sorted(pa.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def shape(**kw):
    s = PaShape()
    s.dtype, s.batch, s.seq_q, s.num_q_heads, s.num_kv_heads = 2, 256, 1, 32, 8
    s.head_dim_qk = s.head_dim_v = 128
    s.page_size, s.num_pages, s.max_pages_per_seq, s.block_table_stride = 16, 65536, 256, 256
    for k, v in kw.items():
        setattr(s, k, v)
    return s


FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: every call below fails validation


def call_decode(s, scale=0.1, splits=0, ptrs=None, workspace=None, ws_bytes=0, fn="pa_decode"):
    lib = pa.load_library()
    p = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, out=FAKE)
    if ptrs:
        p.update(ptrs)
    return getattr(lib, fn)(ctypes.byref(s) if s is not None else None, p["q"], p["k"], p["v"],
                            p["bt"], p["sl"], ctypes.c_float(scale), 0, splits, p["out"], None,
                            workspace, ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), PA_EINVAL),
    (dict(num_q_heads=-1), PA_EINVAL),
    (dict(num_kv_heads=0), PA_EINVAL),
    (dict(num_q_heads=30), PA_EINVAL),                 # Hq % Hkv != 0
    (dict(block_table_stride=255), PA_EINVAL),         # stride < W
    (dict(seq_q=2), PA_EINVAL),                        # decode needs Sq == 1
    (dict(dtype=7), PA_EINVAL),
    (dict(page_size=0), PA_EINVAL),
    (dict(num_pages=0), PA_EINVAL),
    (dict(max_pages_per_seq=2 ** 30, block_table_stride=2 ** 30), PA_EINVAL),  # W*ps overflow
    (dict(head_dim_qk=96, head_dim_v=96), PA_EUNSUPPORTED),
    (dict(head_dim_v=64), PA_EUNSUPPORTED),
    (dict(page_size=64), PA_EUNSUPPORTED),
    (dict(batch=70000, max_pages_per_seq=1, block_table_stride=1), PA_EUNSUPPORTED),
])
def test_shape_validation(kw, code):
    assert call_decode(shape(**kw)) == code


def test_null_shape_and_pointers():
    assert call_decode(None) == PA_EINVAL
    for name in ("q", "k", "v", "bt", "sl", "out"):
        assert call_decode(shape(), ptrs={name: None}) == PA_EINVAL, name


def test_misaligned_and_scale_and_splits():
    assert call_decode(shape(), ptrs={"q": ctypes.c_void_p(0x100008)}) == PA_EINVAL
    assert call_decode(shape(), ptrs={"k": ctypes.c_void_p(0x100004)}) == PA_EINVAL
    assert call_decode(shape(), scale=math.nan) == PA_EINVAL
    assert call_decode(shape(), scale=math.inf) == PA_EINVAL
    assert call_decode(shape(), splits=-1) == PA_EINVAL
    assert call_decode(shape(), splits=257) == PA_EINVAL


def test_workspace_required_for_splits():
    s = shape()
    assert call_decode(s, splits=4) == PA_EWORKSPACE
    need = pa.workspace_bytes(s, 4)
    rows = 256 * 32
    assert need == (rows * 4 * 128 * 4 + 255) // 256 * 256 + rows * 4 * 4
    assert call_decode(s, splits=4, workspace=FAKE, ws_bytes=need - 1) == PA_EWORKSPACE
    assert call_decode(shape(seq_q=4), splits=4, workspace=FAKE, ws_bytes=need,
                       fn="pa_prefill") == PA_EWORKSPACE


def test_split_resolution():
    """Automatic S: at least 256 workgroups (one per compute unit), at most 64
    and at most one split per 8 table slots (rounded up); matrix-core decode
    first lowers the kv heads per workgroup to two, then to one where that
    gives S = 1 or where the splits sit at the table-width cap."""
    # Llama-3-8B decode shape: 256 workgroups of 16 waves (8 kv heads each) fill the GPU
    assert pa.resolve_num_splits(shape(), 0) == 1
    assert pa.workspace_bytes(shape(), 0) == 0
    assert pa.resolve_num_splits(shape(), 5) == 5
    # small batches split so the grid has enough workgroups, capped by the table width
    # (the ragged batch's 63-slot table: at two kv heads per workgroup S = 8 would
    # hit the one-split-per-8-slots cap, so one head per workgroup and S = 4)
    s3 = shape(batch=8, max_pages_per_seq=63, block_table_stride=63)
    assert pa.resolve_num_splits(s3, 0) == 4
    assert pa.resolve_num_splits(shape(batch=8, max_pages_per_seq=8, block_table_stride=8), 0) == 1
    assert pa.resolve_num_splits(shape(batch=8, max_pages_per_seq=9, block_table_stride=9), 0) == 2
    # mid-size batches: kv heads per workgroup drop to two before the splits grow
    # (B * Hkv / 2 * S = 256); to one where that gives S = 1 (B = 32)
    assert pa.resolve_num_splits(shape(batch=8), 0) == 8
    assert pa.resolve_num_splits(shape(batch=16), 0) == 4
    assert pa.resolve_num_splits(shape(batch=32), 0) == 1
    assert pa.resolve_num_splits(shape(batch=64), 0) == 1
    assert pa.resolve_num_splits(shape(batch=128), 0) == 1
    # one sequence: one kv head per workgroup and S = W / 8 = 32 splits
    assert pa.resolve_num_splits(shape(batch=1), 0) == 32
    # Qwen3-235B decode shape (G = 16, matrix-core kernel, 4 kv heads per workgroup)
    s5 = shape(num_q_heads=64, num_kv_heads=4, max_pages_per_seq=512, block_table_stride=512,
               num_pages=131072)
    assert pa.resolve_num_splits(s5, 0) == 1
    s1 = shape(dtype=0, batch=2, num_q_heads=4, num_kv_heads=2, head_dim_qk=64, head_dim_v=64,
               max_pages_per_seq=16, block_table_stride=16, num_pages=30)
    assert pa.resolve_num_splits(s1, 0) == 2
    assert pa.resolve_num_splits(shape(batch=0), 0) == PA_EINVAL
    assert pa.resolve_num_splits(shape(), -3) == PA_EINVAL


def test_split_resolution_prefill():
    """Automatic S for prefill shapes: the shared-tile kernel's 128-row
    workgroups already fill the GPU at the benchmark shapes; small ones split."""
    # B=4, Sq=L=1024, GQA 32/8: 32 row groups x 8 kv heads x 4 sequences = 1024 workgroups
    s = shape(batch=4, seq_q=1024, max_pages_per_seq=64, block_table_stride=64, num_pages=256)
    assert pa.resolve_num_splits(s, 0) == 1 and pa.workspace_bytes(s, 0) == 0
    # B=1, Sq=L=4096, GQA 64/8: 256 row groups x 8 kv heads = 2048 workgroups
    s = shape(batch=1, seq_q=4096, num_q_heads=64, max_pages_per_seq=256, block_table_stride=256,
              num_pages=256)
    assert pa.resolve_num_splits(s, 0) == 1
    # B=1, Sq=64, GQA 32/8: 2 row groups x 8 kv heads = 16 workgroups; 16 splits would
    # fill the GPU but the 64-slot table caps S at 8
    s = shape(batch=1, seq_q=64, max_pages_per_seq=64, block_table_stride=64, num_pages=64)
    assert pa.resolve_num_splits(s, 0) == 8
    rows = 64 * 32
    assert pa.workspace_bytes(s, 0) == rows * 8 * 128 * 4 + rows * 8 * 4
    # f16, D=32, one head, Sq=1024 (the 16-row matrix-core kernel): 64 workgroups, S=4
    s = shape(dtype=1, batch=1, seq_q=1024, num_q_heads=1, num_kv_heads=1, head_dim_qk=32,
              head_dim_v=32, page_size=32, max_pages_per_seq=32, block_table_stride=32,
              num_pages=32)
    assert pa.resolve_num_splits(s, 0) == 4


def test_describe_plan():
    """The planner query names the kernel family each shape takes (host only)."""
    from paged_kv_cache_195_amd.api import PA_FP8_E4M3, PA_I8

    def plan(s, splits=0):
        return pa.describe_plan(s, splits)

    # Llama-3-8B decode: one 16-row block per wave, 8 waves, 8 kv heads per workgroup, S = 1
    p = plan(shape())
    assert p == {"kernel": "mfma", "num_splits": 1, "rows_per_workgroup": 16, "row_groups": 1,
                 "waves": 8, "kv_heads_per_workgroup": 8}
    # Qwen3-235B decode (Hkv = 4): 4-wave workgroups
    p = plan(shape(num_q_heads=64, num_kv_heads=4, max_pages_per_seq=512,
                   block_table_stride=512))
    assert (p["kernel"], p["waves"], p["kv_heads_per_workgroup"]) == ("mfma", 4, 4)
    # 17..32 rows per kv head over >= 128 (sequence, kv head) pairs: two blocks per wave
    for hq, hkv, batch in ((24, 1, 128), (256, 8, 16), (17, 1, 130)):
        p = plan(shape(num_q_heads=hq, num_kv_heads=hkv, batch=batch))
        assert (p["kernel"], p["rows_per_workgroup"], p["waves"]) == ("mfma_two_blocks", 32, 8)
    # ... but not below 128 pairs (shared-tile kernel at D = 128)
    assert plan(shape(num_q_heads=24, num_kv_heads=1, batch=127))["kernel"] == "shared_tile_teams"
    # 16-bit D = 32 chunks of several queries take the two-block kernel (no shared-tile
    # kernel at D = 32)
    p = plan(shape(dtype=1, seq_q=6, num_q_heads=8, num_kv_heads=2, head_dim_qk=32,
                   head_dim_v=32, batch=64))
    assert p["kernel"] == "mfma_two_blocks"
    # 8-bit caches: two blocks up to 63 rows, the shared-tile kernel (one team) from 64
    assert plan(shape(kv_dtype=PA_I8, num_q_heads=48, num_kv_heads=1, batch=128))["kernel"] == \
        "mfma_two_blocks"
    p = plan(shape(kv_dtype=PA_FP8_E4M3, seq_q=16, batch=4, max_pages_per_seq=64,
                   block_table_stride=64))
    assert (p["kernel"], p["waves"], p["rows_per_workgroup"]) == ("shared_tile", 4, 128)
    # prefill, 16-bit: D = 128 two teams, D = 64 one team
    s = shape(batch=4, seq_q=1024, max_pages_per_seq=64, block_table_stride=64)
    assert plan(s)["kernel"] == "shared_tile_teams"
    s = shape(batch=4, seq_q=1024, head_dim_qk=64, head_dim_v=64, max_pages_per_seq=64,
              block_table_stride=64)
    assert plan(s)["kernel"] == "shared_tile"
    # f32 caches: the vector-ALU kernel
    assert plan(shape(dtype=0))["kernel"] == "valu"
    # the split count agrees with pa_resolve_num_splits
    for s in (shape(batch=8), shape(batch=1), shape(batch=8, max_pages_per_seq=63,
                                                      block_table_stride=63)):
        assert plan(s)["num_splits"] == pa.resolve_num_splits(s, 0)
    assert plan(shape(), 7)["num_splits"] == 7
    # errors
    lib = pa.load_library()
    assert lib.pa_describe_plan(ctypes.byref(shape()), 0, None) == PA_EINVAL
    assert lib.pa_describe_plan(ctypes.byref(shape(batch=0)), 0,
                                ctypes.byref(pa.api.PaPlanInfo())) == PA_EINVAL
    assert lib.pa_describe_plan(ctypes.byref(shape()), -1,
                                ctypes.byref(pa.api.PaPlanInfo())) == PA_EINVAL


def test_combine_validation():
    lib = pa.load_library()
    assert lib.pa_combine(9, 4, 2, 128, FAKE, FAKE, FAKE, None, None) == PA_EINVAL
    assert lib.pa_combine(2, 0, 2, 128, FAKE, FAKE, FAKE, None, None) == PA_EINVAL
    assert lib.pa_combine(2, 4, 0, 128, FAKE, FAKE, FAKE, None, None) == PA_EINVAL
    assert lib.pa_combine(2, 4, 2, 128, None, FAKE, FAKE, None, None) == PA_EINVAL
    assert lib.pa_combine(2, 4, 2, 128, FAKE, FAKE, None, None, None) == PA_EINVAL
    # misaligned pointers: partials and lse need 4 bytes, a bf16 out 2, an f32 out 4
    odd = ctypes.c_void_p(FAKE.value + 2)
    assert lib.pa_combine(2, 4, 2, 128, odd, FAKE, FAKE, None, None) == PA_EINVAL
    assert lib.pa_combine(2, 4, 2, 128, FAKE, odd, FAKE, None, None) == PA_EINVAL
    assert lib.pa_combine(2, 4, 2, 128, FAKE, FAKE, FAKE, odd, None) == PA_EINVAL
    assert lib.pa_combine(0, 4, 2, 128, FAKE, FAKE, odd, None, None) == PA_EINVAL
    assert lib.pa_combine(2, 4, 2, 128, FAKE, FAKE, ctypes.c_void_p(FAKE.value + 1), None,
                          None) == PA_EINVAL


def test_strerror():
    for code in (0, -1, -2, -3, -4, -5):
        assert pa.strerror(code) and pa.strerror(code) != pa.strerror(99)


def test_noalloc_host_checks():
    """pa_decode_noalloc rejects, on the host and before any HIP call, split
    partials past its static array (PA_ESCRATCH) and invalid shapes."""
    from paged_kv_cache_195_amd.api import NOALLOC_SCRATCH_BYTES, PA_ESCRATCH

    lib = pa.load_library()

    def call(s, splits):
        return lib.pa_decode_noalloc(ctypes.byref(s), None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     ctypes.c_float(0.1), 0, splits, FAKE, None, None)

    s = shape()   # B=256, Hq=32, Dv=128: S=3 fits 16 MiB, S=4 does not
    assert pa.workspace_bytes(s, 3) <= NOALLOC_SCRATCH_BYTES < pa.workspace_bytes(s, 4)
    assert call(s, 4) == PA_ESCRATCH and call(s, 200) == PA_ESCRATCH
    assert call(shape(batch=0), 0) == PA_EINVAL
    assert call(shape(seq_q=2), 0) == PA_EINVAL          # decode needs Sq == 1
    assert call(shape(), -1) == PA_EINVAL
    assert call(shape(), 300) == PA_EINVAL               # past the 256-split limit
    assert call(shape(head_dim_qk=96, head_dim_v=96), 0) == PA_EUNSUPPORTED


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 1, 32)
    with pytest.raises(ValueError):
        pa.decode(q, torch.zeros(2, 16, 1, 32), torch.zeros(2, 16, 1, 32),
                  torch.zeros(1, 2, dtype=torch.int32), torch.zeros(1, dtype=torch.int32), 0.1)


def call_decode_ex(s, opts, ptrs=None):
    lib = pa.load_library()
    p = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, out=FAKE)
    if ptrs:
        p.update(ptrs)
    return lib.pa_decode_ex(ctypes.byref(s), None if opts is None else ctypes.byref(opts),
                            p["q"], p["k"], p["v"], p["bt"], p["sl"], ctypes.c_float(0.1), 0, 0,
                            p["out"], None, None, ctypes.c_size_t(0), None)


def test_options_validation():
    """The _ex entry points run the same checks, plus 4-byte alignment of the
    optional arrays, before anything is launched."""
    from paged_kv_cache_195_amd.api import PaOptions
    assert call_decode_ex(shape(batch=0), None) == PA_EINVAL
    assert call_decode_ex(shape(head_dim_qk=96, head_dim_v=96), PaOptions()) == PA_EUNSUPPORTED
    assert call_decode_ex(shape(), PaOptions(prefix_offset=0x100002)) == PA_EINVAL
    assert call_decode_ex(shape(), PaOptions(page_check=0x100001)) == PA_EINVAL
    assert call_decode_ex(shape(), PaOptions(), ptrs={"bt": ctypes.c_void_p(0x100002)}) == PA_EINVAL
    assert call_decode_ex(shape(), PaOptions(), ptrs={"sl": ctypes.c_void_p(0x100003)}) == PA_EINVAL
    assert call_decode_ex(shape(seq_q=2), PaOptions(prefix_offset=0x100000)) == PA_EINVAL


def test_eight_bit_cache_validation():
    """kv_dtype: codes only with 16-bit queries, D in {64, 128}, and scales
    exactly when the caches hold codes."""
    from paged_kv_cache_195_amd.api import PA_FP8_E4M3, PA_I8, PaOptions
    scales = PaOptions(k_scale=0x200000, v_scale=0x300000)
    assert call_decode_ex(shape(kv_dtype=7), scales) == PA_EINVAL
    assert call_decode_ex(shape(kv_dtype=PA_I8, dtype=0), scales) == PA_EUNSUPPORTED
    assert call_decode_ex(shape(kv_dtype=PA_FP8_E4M3, head_dim_qk=32, head_dim_v=32),
                          scales) == PA_EUNSUPPORTED
    # codes without scales (the plain entry point has none), scales without codes
    assert call_decode(shape(kv_dtype=PA_I8)) == PA_EINVAL
    assert call_decode_ex(shape(kv_dtype=PA_I8), PaOptions(k_scale=0x200000)) == PA_EINVAL
    assert call_decode_ex(shape(), scales) == PA_EINVAL
    assert call_decode_ex(shape(kv_dtype=PA_I8), PaOptions(k_scale=0x200002,
                                                           v_scale=0x300000)) == PA_EINVAL
    # 8-bit caches take the matrix-core kernel: 8 kv heads per workgroup at the
    # Llama-3-8B decode shape, 256 workgroups, so no split
    assert pa.resolve_num_splits(shape(kv_dtype=PA_I8), 0) == 1
    # ... and the same plan as 16-bit caches at the ragged batch's shape
    assert pa.resolve_num_splits(shape(kv_dtype=PA_FP8_E4M3, batch=8, max_pages_per_seq=63,
                                       block_table_stride=63), 0) == 4
