"""Seeded synthetic inputs for paged attention.

This module builds tensors only: query, paged K/V caches, block tables and
sequence lengths, at the shapes of the decode and prefill workloads the pages
measure.  It contains no attention arithmetic, so both the CPU oracle and the
HIP path can be fed from it without sharing any of the method's code.

Recipe (the same for every workload):

* ``torch.Generator(device).manual_seed(seed)`` drives the page permutation,
  then ``q``, ``k_cache`` and ``v_cache`` as standard normals drawn in float32
  and rounded to the workload's dtype; the oracle reads the rounded values.
  Ragged lengths come from a CPU generator with the same seed, so the layout
  is the same whatever the device.
* Physical pages are assigned by a seeded random permutation, so logical and
  physical order differ.
* Block-table slots a sequence does not use hold the unmapped id
  ``0x7FFFFFFF``; pages no sequence references, and the token slots of a last
  page past a sequence's length, are filled with NaN so that any stray read
  shows up in the result.

Workloads (``WORKLOADS``):

``tiny_f32``        B=2, Hq=4, Hkv=2, D=64, page 16, lengths {37, 200}, 16
                    slots per row over 30 physical pages, splits {1, 3}.
``prefill_f16``     one batch-head, Sq = L = 1024, D=32, page 32 (1024
                    elements), 32 shuffled pages, causal, splits {1, 4}.
``ragged_bf16``     B=8, Hq=32, Hkv=8, D=128, page 16, lengths uniform in
                    [17, 1000], table 63 slots wide read through a view whose
                    tail holds the unmapped id, cache page count overstated
                    (65,538), splits 1..8.
``llama3_8b_decode`` B=256, Hq=32, Hkv=8, D=128, page 16, L=4096, K and V
                    caches of exactly 2 GiB (65,536 pages of 32 KiB), table a
                    seeded permutation of all pages, splits auto.
``qwen3_235b_decode`` B=256, Hq=64, Hkv=4, D=128, page 16, L=8192, 2 GiB per
                    cache (131,072 pages of 16 KiB); variant ``straddle`` with
                    131,328 pages (2 GiB + 4 MiB) so used pages lie on both
                    sides of byte offset 2^31.
``llama3_70b_decode`` B=256, Hq=64, Hkv=8, D=128, page 16, L=4096, 2 GiB per
                    cache (65,536 pages of 32 KiB).
``decode_b64_s8192_g8`` B=64, Hq=64, Hkv=8, D=128, page 16, L=8192, 1 GiB per
                    cache (32,768 pages of 32 KiB).
``prefill_b4_s1024``  causal prefill bf16, B=4, Sq=L=1024, Hq=32, Hkv=8, D=128,
                    page 16.
``prefill_b1_s4096``  causal prefill bf16, B=1, Sq=L=4096, Hq=64, Hkv=8, D=128,
                    page 16.
``llama3_8b_decode_int8`` / ``llama3_8b_decode_fp8``  the Llama-3-8B decode
                    shape with 8-bit K/V codes (1 GiB per cache).
``decode_past_4gib`` B=32, Hq=32, Hkv=8, D=128, page 16, L=4096 over caches of
                    131,200 pages of 32 KiB (4 GiB + 4 MiB each): every page
                    that starts at or past byte 2^32 (ids 131,072..131,199),
                    and the page that ends there (131,071), is referenced, the
                    rest of the 8,192 referenced pages drawn at random below;
                    unreferenced pages hold NaN.

8-bit caches (``kv="int8"`` or ``kv="fp8_e4m3"``): K and V hold codes drawn
from the same seeded normals -- int8 as round(32 x) clamped to [-127, 127],
fp8 as torch's float8_e4m3fn conversion of x -- with one float32 scale per
(page, kv head) drawn uniform in [0.5, 1.5) (divided by 32 for int8).
Unreferenced pages get NaN scales and poison codes (fp8: the NaN code; int8:
-128, which the generator never produces), last-page tails poison codes.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

UNMAPPED_PAGE = 0x7FFFFFFF

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    dtype: str
    batch: int
    seq_q: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    causal: bool
    splits: tuple
    seed: int
    description: str
    kv: Optional[str] = None      # None, "int8" or "fp8_e4m3": 8-bit K/V codes


WORKLOADS = {
    "tiny_f32": WorkloadSpec("tiny_f32", "f32", 2, 1, 4, 2, 64, 16, False, (1, 3), 0,
                             "tiny paged GQA decode f32 B=2 Hq=4 Hkv=2 D=64 page16 L={37,200}"),
    "prefill_f16": WorkloadSpec("prefill_f16", "f16", 1, 1024, 1, 1, 32, 32, True, (1, 4), 1,
                                "paged causal prefill f16 Sq=L=1024 H=1 D=32 page32, 32 pages"),
    "ragged_bf16": WorkloadSpec("ragged_bf16", "bf16", 8, 1, 32, 8, 128, 16, False,
                                tuple(range(1, 9)), 2,
                                "ragged paged decode bf16 B=8 Hq=32 Hkv=8 D=128 page16 L~U[17,1000]"),
    "llama3_8b_decode": WorkloadSpec("llama3_8b_decode", "bf16", 256, 1, 32, 8, 128, 16, False,
                                     (0,), 3,
                                     "Llama-3-8B decode bf16 B=256 Hq=32 Hkv=8 D=128 page16 Skv=4096"),
    "qwen3_235b_decode": WorkloadSpec("qwen3_235b_decode", "bf16", 256, 1, 64, 4, 128, 16, False,
                                      (0,), 4,
                                      "Qwen3-235B-A22B decode bf16 B=256 Hq=64 Hkv=4 D=128 page16 Skv=8192"),
    "llama3_70b_decode": WorkloadSpec("llama3_70b_decode", "bf16", 256, 1, 64, 8, 128, 16, False,
                                      (0,), 5,
                                      "Llama-3-70B decode bf16 B=256 Hq=64 Hkv=8 D=128 page16 Skv=4096"),
    "decode_b64_s8192_g8": WorkloadSpec("decode_b64_s8192_g8", "bf16", 64, 1, 64, 8, 128, 16, False,
                                        (0,), 6,
                                        "decode bf16 B=64 Hq=64 Hkv=8 D=128 page16 Skv=8192"),
    "prefill_b4_s1024": WorkloadSpec("prefill_b4_s1024", "bf16", 4, 1024, 32, 8, 128, 16, True,
                                     (0,), 7,
                                     "causal prefill bf16 B=4 Sq=L=1024 Hq=32 Hkv=8 D=128 page16"),
    "prefill_b1_s4096": WorkloadSpec("prefill_b1_s4096", "bf16", 1, 4096, 64, 8, 128, 16, True,
                                     (0,), 8,
                                     "causal prefill bf16 B=1 Sq=L=4096 Hq=64 Hkv=8 D=128 page16"),
    "llama3_8b_decode_int8": WorkloadSpec("llama3_8b_decode_int8", "bf16", 256, 1, 32, 8, 128, 16,
                                          False, (0,), 9,
                                          "Llama-3-8B decode, int8 K/V codes, bf16 q/out B=256 "
                                          "Hq=32 Hkv=8 D=128 page16 Skv=4096", "int8"),
    "llama3_8b_decode_fp8": WorkloadSpec("llama3_8b_decode_fp8", "bf16", 256, 1, 32, 8, 128, 16,
                                         False, (0,), 10,
                                         "Llama-3-8B decode, fp8 E4M3 K/V codes, bf16 q/out B=256 "
                                         "Hq=32 Hkv=8 D=128 page16 Skv=4096", "fp8_e4m3"),
    "decode_g32_b256": WorkloadSpec("decode_g32_b256", "bf16", 256, 1, 32, 1, 128, 16, False,
                                    (0,), 12,
                                    "decode bf16 B=256 Hq=32 Hkv=1 D=128 page16 Skv=4096 "
                                    "(group of 32 query heads per kv head)"),
    "decode_past_4gib": WorkloadSpec("decode_past_4gib", "bf16", 32, 1, 32, 8, 128, 16, False,
                                     (0,), 13,
                                     "decode bf16 B=32 Hq=32 Hkv=8 D=128 page16 Skv=4096 over "
                                     "4 GiB + 4 MiB caches, pages past byte 2^32 referenced"),
    "prefill_b4_s1024_int8": WorkloadSpec("prefill_b4_s1024_int8", "bf16", 4, 1024, 32, 8, 128,
                                          16, True, (0,), 11,
                                          "causal prefill, int8 K/V codes, bf16 q/out B=4 "
                                          "Sq=L=1024 Hq=32 Hkv=8 D=128 page16", "int8"),
}

KV_KINDS = ("int8", "fp8_e4m3")

# Pages per cache of ``decode_past_4gib``: 4 GiB + 4 MiB of 32 KiB pages.
PAST_4GIB_PAGES = 131200

WORKLOAD_ORDER = ["tiny_f32", "prefill_f16", "ragged_bf16", "llama3_8b_decode", "qwen3_235b_decode"]


@dataclass
class PagedInputs:
    """One batch of paged-attention inputs (all tensors on ``device``)."""

    spec: WorkloadSpec
    q: torch.Tensor              # [B, Sq, Hq, D]
    k_cache: torch.Tensor        # [num_pages, page_size, Hkv, D]
    v_cache: torch.Tensor        # [num_pages, page_size, Hkv, D]
    block_table: torch.Tensor    # int32 [B, W], possibly a strided view
    seq_lens: torch.Tensor       # int32 [B]
    scale: float
    causal: bool
    num_pages_arg: int           # page count handed to the library (may be overstated)
    seq_lens_host: List[int] = field(default_factory=list)
    table_host: Optional[torch.Tensor] = None   # CPU int32 copy of block_table
    notes: dict = field(default_factory=dict)
    kv: Optional[str] = None                    # 8-bit code kind of the caches, or None
    k_scale: Optional[torch.Tensor] = None      # [num_pages, Hkv] float32 (8-bit caches)
    v_scale: Optional[torch.Tensor] = None

    @property
    def batch(self) -> int:
        return self.q.shape[0]


def past_4gib_pages(gen, perm: torch.Tensor, total_used: int, page_bytes: int) -> torch.Tensor:
    """``total_used`` distinct page ids in a seeded order: every page from the
    one that ends at byte 2^32 to the last of the ``perm.numel()`` pages, the
    rest taken from ``perm`` (a permutation of all ids) below that page."""
    first_high = (1 << 32) // page_bytes - 1
    high = torch.arange(first_high, perm.numel(), dtype=perm.dtype, device=perm.device)
    low = perm[perm < first_high][: total_used - high.numel()]
    both = torch.cat([high, low])
    return both[torch.randperm(both.numel(), generator=gen, device=perm.device)]


def _normal(gen, shape, dtype, device):
    return torch.randn(shape, generator=gen, dtype=torch.float32, device=device).to(dtype)


def _codes(gen, shape, kind, device):
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    if kind == "int8":
        return torch.clamp(torch.round(x * 32.0), -127.0, 127.0).to(torch.int8)
    if kind == "fp8_e4m3":
        return x.to(torch.float8_e4m3fn)
    raise ValueError(kind)


def _scales(gen, shape, kind, device):
    u = torch.rand(shape, generator=gen, dtype=torch.float32, device=device) + 0.5
    return u / 32.0 if kind == "int8" else u


POISON_CODE = {"int8": 0x80, "fp8_e4m3": 0x7F}


def _poison_codes(codes: torch.Tensor, scales: torch.Tensor, kind: str, used_pages: torch.Tensor,
                  lens: List[int], table: torch.Tensor, page_size: int):
    """Poison codes and NaN scales in unreferenced pages; poison codes past each
    sequence's end."""
    raw = codes.view(torch.uint8)
    mask = torch.ones(codes.shape[0], dtype=torch.bool, device=codes.device)
    mask[used_pages.long()] = False
    raw[mask] = POISON_CODE[kind]
    scales[mask] = float("nan")
    for b, seq_len in enumerate(lens):
        n = -(-seq_len // page_size)
        tail = n * page_size - seq_len
        if n and tail:
            raw[int(table[b, n - 1])][page_size - tail:] = POISON_CODE[kind]


def _quantize_inputs(inputs, gen, kind, used, lens, table, poison):
    """Replace the float caches of ``inputs`` by 8-bit codes and scales."""
    phys, ps, hkv, d = inputs.k_cache.shape
    device = inputs.k_cache.device
    inputs.k_cache = _codes(gen, (phys, ps, hkv, d), kind, device)
    inputs.v_cache = _codes(gen, (phys, ps, hkv, d), kind, device)
    inputs.k_scale = _scales(gen, (phys, hkv), kind, device)
    inputs.v_scale = _scales(gen, (phys, hkv), kind, device)
    inputs.kv = kind
    if poison:
        _poison_codes(inputs.k_cache, inputs.k_scale, kind, used, lens, table, ps)
        _poison_codes(inputs.v_cache, inputs.v_scale, kind, used, lens, table, ps)


def _poison_unused(cache: torch.Tensor, used_pages: torch.Tensor, lens: List[int],
                   table: torch.Tensor, page_size: int):
    """NaN into unreferenced pages and into the slots past each sequence's end."""
    if not cache.dtype.is_floating_point:
        return
    mask = torch.ones(cache.shape[0], dtype=torch.bool, device=cache.device)
    mask[used_pages.long()] = False
    cache[mask] = float("nan")
    for b, seq_len in enumerate(lens):
        n = -(-seq_len // page_size)
        tail = n * page_size - seq_len
        if n and tail:
            cache[int(table[b, n - 1])][page_size - tail:] = float("nan")


def make_workload(name: str, device="cpu", seed: Optional[int] = None, variant: Optional[str] = None,
                  seq_lens: Optional[List[int]] = None, batch: Optional[int] = None,
                  table_stride: Optional[int] = None, kv: Optional[str] = None) -> PagedInputs:
    """Build the named workload on ``device``.

    ``seed`` defaults to the workload's own.  ``variant`` selects a variant
    (``"straddle"`` for the Qwen3 shape; ``"contiguous"`` for an identity page
    order on the two large decode shapes).  ``seq_lens``/``batch`` override the
    lengths (tests use this for edge cases on the small workloads).
    ``table_stride`` reads the block table through a row stride larger than
    its width.  ``kv`` ("int8" or "fp8_e4m3") stores K and V as 8-bit codes
    (the ``*_int8`` / ``*_fp8`` workloads set it themselves).
    """
    spec = WORKLOADS[name]
    kv = spec.kv if kv is None else kv
    if spec.kv is not None:
        name = name.rsplit("_", 1)[0]
    seed = spec.seed if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dtype = DTYPES[spec.dtype]
    ps, hkv, d, hq = spec.page_size, spec.num_kv_heads, spec.head_dim, spec.num_q_heads

    if name == "tiny_f32":
        lens = list(seq_lens) if seq_lens is not None else [37, 200]
        width, phys = 16, 30
    elif name == "prefill_f16":
        lens = list(seq_lens) if seq_lens is not None else [1024]
        width, phys = 32, 32
    elif name == "ragged_bf16":
        b = batch if batch is not None else spec.batch
        width = 63
        if seq_lens is not None:
            lens = list(seq_lens)
        else:
            lens = torch.randint(17, 1001, (b,), generator=torch.Generator().manual_seed(seed)).tolist()
        phys = sum(-(-x // ps) for x in lens) + 8   # a little slack, poisoned
    elif name == "llama3_8b_decode":
        b = batch if batch is not None else spec.batch
        lens = list(seq_lens) if seq_lens is not None else [4096] * b
        width, phys = 256, 65536 if batch is None else max(1, b * 256)
    elif name == "qwen3_235b_decode":
        b = batch if batch is not None else spec.batch
        lens = list(seq_lens) if seq_lens is not None else [8192] * b
        width = 512
        phys = 131328 if variant == "straddle" else (131072 if batch is None else max(1, b * 512))
    elif name == "llama3_70b_decode":
        b = batch if batch is not None else spec.batch
        lens = list(seq_lens) if seq_lens is not None else [4096] * b
        width, phys = 256, b * 256
    elif name == "decode_g32_b256":
        b = batch if batch is not None else spec.batch
        lens = list(seq_lens) if seq_lens is not None else [4096] * b
        width, phys = 256, b * 256
    elif name == "decode_b64_s8192_g8":
        b = batch if batch is not None else spec.batch
        lens = list(seq_lens) if seq_lens is not None else [8192] * b
        width, phys = 512, b * 512
    elif name == "decode_past_4gib":
        b = batch if batch is not None else spec.batch
        lens = list(seq_lens) if seq_lens is not None else [4096] * b
        width, phys = 256, PAST_4GIB_PAGES
    elif name in ("prefill_b4_s1024", "prefill_b1_s4096"):
        b = batch if batch is not None else spec.batch
        lens = list(seq_lens) if seq_lens is not None else [spec.seq_q] * b
        width = -(-spec.seq_q // ps)
        phys = b * width
    else:
        raise KeyError(name)

    bsz = len(lens)
    n_per = [-(-x // ps) for x in lens]
    if max(n_per, default=0) > width:
        raise ValueError("sequence longer than the block table allows")
    total_used = sum(n_per)
    if total_used > phys:
        raise ValueError("not enough physical pages")

    # --- page assignment -------------------------------------------------------
    if variant == "contiguous":
        perm = torch.arange(phys, dtype=torch.int64, device=device)
    else:
        perm = torch.randperm(phys, generator=gen, device=device)
    if name == "decode_past_4gib":
        page_bytes = ps * hkv * d * torch.empty((), dtype=dtype).element_size()
        perm = past_4gib_pages(gen, perm, total_used, page_bytes)
    stride = width if table_stride is None else int(table_stride)
    if stride < width:
        raise ValueError("table stride smaller than its width")
    # storage: rows of `stride` slots plus a 64-entry tail, all unmapped first
    storage = torch.full((bsz * stride + 64,), UNMAPPED_PAGE, dtype=torch.int32, device=device)
    used = perm[:total_used].to(torch.int32)
    rows = storage[: bsz * stride].view(bsz, stride)
    pos = 0
    for b, n in enumerate(n_per):
        rows[b, :n] = used[pos:pos + n]
        pos += n
    table = rows[:, :width]   # view; row stride `stride`, the storage tail is unmapped

    # --- values -----------------------------------------------------------------
    q = _normal(gen, (bsz, spec.seq_q, hq, d), dtype, device)
    k_cache = _normal(gen, (phys, ps, hkv, d), dtype, device)
    v_cache = _normal(gen, (phys, ps, hkv, d), dtype, device)
    if name in ("tiny_f32", "ragged_bf16", "prefill_f16", "decode_past_4gib"):
        _poison_unused(k_cache, used, lens, table, ps)
        _poison_unused(v_cache, used, lens, table, ps)

    num_pages_arg = 65538 if name == "ragged_bf16" else phys
    seq_lens_t = torch.tensor(lens, dtype=torch.int32, device=device)
    inputs = PagedInputs(spec=spec, q=q, k_cache=k_cache, v_cache=v_cache, block_table=table,
                         seq_lens=seq_lens_t, scale=1.0 / math.sqrt(d), causal=spec.causal,
                         num_pages_arg=num_pages_arg, seq_lens_host=list(lens),
                         table_host=table.cpu())
    if kv is not None:
        del k_cache, v_cache
        inputs.k_cache = inputs.v_cache = None
        inputs.k_cache = torch.empty((phys, ps, hkv, d), dtype=torch.int8, device=device)
        _quantize_inputs(inputs, gen, kv, used, lens, table,
                         poison=name in ("tiny_f32", "ragged_bf16", "prefill_f16"))
    inputs.notes["true_num_pages"] = phys
    inputs.notes["table_storage"] = storage
    inputs.notes["variant"] = variant
    if variant == "straddle" or name == "decode_past_4gib":
        page_bytes = ps * hkv * d * k_cache.element_size()
        inputs.notes["max_used_page_start_bytes"] = int(used.max()) * page_bytes
    return inputs


def attention_flops(inputs: PagedInputs) -> int:
    """Algorithmic FLOPs of one call: 2 per multiply-add of q.k and of p.v over
    the keys each query row may see (causal rows see a prefix)."""
    spec = inputs.spec
    sq, hq, d = inputs.q.shape[1], inputs.q.shape[2], inputs.q.shape[3]
    total = 0
    for seq_len in inputs.seq_lens_host:
        for i in range(sq):
            seen = seq_len if not inputs.causal else max(0, min(seq_len, seq_len - sq + i + 1))
            total += seen
    return 4 * d * hq * total


def kv_bytes(inputs: PagedInputs) -> int:
    """Algorithmic K+V bytes one decode step reads: every element of the first
    L tokens of each sequence, once, for K and for V."""
    spec = inputs.spec
    per_token = spec.num_kv_heads * spec.head_dim * inputs.k_cache.element_size()
    total = 2 * per_token * sum(inputs.seq_lens_host)
    if inputs.kv is not None:   # one K and one V float32 scale per (page, kv head) read
        ps = inputs.k_cache.shape[1]
        total += 2 * 4 * spec.num_kv_heads * sum(-(-x // ps) for x in inputs.seq_lens_host)
    return total


def make_custom(dtype: str, seq_lens: List[int], num_q_heads: int, num_kv_heads: int,
                head_dim: int, page_size: int, seq_q: int = 1, causal: bool = False,
                width: Optional[int] = None, extra_pages: int = 5, seed: int = 0,
                device="cpu", table_stride: Optional[int] = None,
                kv: Optional[str] = None) -> PagedInputs:
    """Any shape, same recipe as the named workloads (shuffled pages, unmapped
    unused slots, NaN in unreferenced pages and in last-page tails); ``kv``
    stores K and V as 8-bit codes with per-(page, kv head) scales."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    tdtype = DTYPES[dtype]
    ps = page_size
    n_per = [-(-x // ps) for x in seq_lens]
    width = max(max(n_per, default=0), 1) if width is None else width
    if max(n_per, default=0) > width:
        raise ValueError("sequence longer than the block table allows")
    bsz = len(seq_lens)
    total_used = sum(n_per)
    phys = total_used + extra_pages
    perm = torch.randperm(phys, generator=gen, device=device)
    stride = width if table_stride is None else int(table_stride)
    storage = torch.full((bsz * stride + 64,), UNMAPPED_PAGE, dtype=torch.int32, device=device)
    used = perm[:total_used].to(torch.int32)
    rows = storage[: bsz * stride].view(bsz, stride)
    pos = 0
    for b, n in enumerate(n_per):
        rows[b, :n] = used[pos:pos + n]
        pos += n
    table = rows[:, :width]
    q = _normal(gen, (bsz, seq_q, num_q_heads, head_dim), tdtype, device)
    k_cache = _normal(gen, (phys, ps, num_kv_heads, head_dim), tdtype, device)
    v_cache = _normal(gen, (phys, ps, num_kv_heads, head_dim), tdtype, device)
    _poison_unused(k_cache, used, list(seq_lens), table, ps)
    _poison_unused(v_cache, used, list(seq_lens), table, ps)
    spec = WorkloadSpec("custom", dtype, bsz, seq_q, num_q_heads, num_kv_heads, head_dim, ps,
                        causal, (1,), seed, "custom")
    inputs = PagedInputs(spec=spec, q=q, k_cache=k_cache, v_cache=v_cache, block_table=table,
                         seq_lens=torch.tensor(list(seq_lens), dtype=torch.int32, device=device),
                         scale=1.0 / math.sqrt(head_dim), causal=causal, num_pages_arg=phys,
                         seq_lens_host=list(seq_lens), table_host=table.cpu())
    inputs.notes["true_num_pages"] = phys
    inputs.notes["table_storage"] = storage
    if kv is not None:
        _quantize_inputs(inputs, gen, kv, used, list(seq_lens), table, poison=True)
    return inputs
