"""Plain, slow f64 CPU oracle for paged attention over a block-table K/V cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library (the HIP kernels, the C ABI and its Python binding) never imports it,
and this module imports nothing from the library: the two share no code.

What it computes, and where that is defined:

* Attention is exact softmax attention, ``softmax(scale * q K^T) V``, over the
  *logical* key sequence of each batch entry.  The paged cache is only a
  storage form: the rocMLIR "Paged Attention: rocmlir-gen changes" page
  (Technical Details, "CPU Validation") validates on the regular K/V tensors
  of the logical-order cache, and the "migraphx & highlevel pipeline" page
  (Technical Details, item 1 and the note on ``rock.deref``) describes the
  paged input as a lazy view whose dereference is the gathered sequence.
* A page holds ``page_size`` tokens of every kv head: ``cache[page, token,
  kv_head, dim]``.  The rocm-libraries "one K/V resource per page" page
  (Motivation; Coverage, the in-page offset that must keep its kv-head term)
  fixes that a page holds all kv heads; token-major order inside the page is
  the reading taken here.
* Block table entries at slot ``s < ceil(L / page_size)`` are physical page
  ids; later slots are never read (same page, Coverage: ragged lengths with an
  unmapped id in the table's tail).
* Query head ``h`` reads kv head ``h // G`` with ``G = Hq / Hkv`` (grouped
  query attention; contiguous groups is the reading taken here).
* Causal masking is bottom-right aligned: query row ``i`` of ``Sq`` sits at key
  position ``L - Sq + i`` and sees keys ``j <= L - Sq + i``.  The rocMLIR
  "Fix split-kv attention masking" page (Technical Details, host reference:
  causal valid-split masking) defines validity per query row from that row's
  effective key length, including a prefix offset when one is given, and
  treats prefix-causal masking as causal.  With a per-sequence prefix offset
  ``P_b`` (the reading taken here), row ``i`` sits at key position
  ``P_b + i`` instead, whatever the causal flag says.
* Page-id range check (optional): the rocm-libraries "one K/V resource per
  page" page (Not in this PR; review, LOW findings) notes that page ids are
  bounded by slot index only, not checked against the cache's page count.
  ``check_pages`` is that check: a sequence any of whose first
  ``ceil(L / page_size)`` ids lies outside ``[0, num_pages)``, or whose length
  lies outside ``[0, W * page_size]`` (the same bound on slot indices), is not attended
  (the reading taken here: it counts as empty, so its rows give ``(0, -inf)``),
  and the smallest such batch index is reported.
* Split-KV: the key pages of a sequence are cut into ``S`` ranges of
  ``ceil(n / S)`` pages each, the last ranges clamped to ``n`` and possibly
  empty (same page, Technical Details: ceil-division of the iterations per
  split, then clamping the end).  Each split yields its own normalised output
  and natural-log LSE; a split without a valid key yields output 0 and LSE
  ``-inf`` (same page: the ``-inf - (-inf)`` guard and the 0/0 guard in
  ``scaleFinalOutput``).  The combine weights each split by
  ``exp(lse_s - max lse)`` (same page, host reference: f32 combine for narrow
  floats; here in f64).

* Quantized pages (optional): K and V may be stored as 8-bit codes, each
  (page, kv head) slice with one float32 scale, the element being
  ``scale[page, kv_head] * value(code)``.  The pages name int8 paged attention
  (rocMLIR "Paged Attention: rocmlir-gen changes", the file list's int8 e2e
  test) and i8 split-KV attention (split-kv masking page, Motivation), and fp8
  K/V loaders (per-page resource page, review MEDIUM findings); the scale
  granularity and the fp8 variant (OCP E4M3: 4 exponent bits with bias 7, 3
  mantissa bits, subnormals, no infinities, S.1111.111 is NaN) are this
  build's reading.  ``code_value`` decodes one code from those definitions and
  ``dequantize_cache`` forms the exact float64 cache the attention then reads.

Every function works in float64 on NumPy arrays; inputs are widened exactly.
There is no blocking, fusion or reordering beyond the definitions above.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "pages_for",
    "kv_head_of",
    "key_limit",
    "gather_logical",
    "attend",
    "attention",
    "split_page_ranges",
    "split_partials",
    "combine",
    "check_pages",
    "code_value",
    "dequantize_cache",
]


def pages_for(seq_len: int, page_size: int) -> int:
    """Number of pages holding ``seq_len`` tokens: ``ceil(seq_len / page_size)``."""
    return -(-int(seq_len) // int(page_size))


def kv_head_of(q_head: int, group: int) -> int:
    """KV head read by query head ``q_head`` when ``group`` query heads share one."""
    return q_head // group


def key_limit(seq_len: int, seq_q: int, row: int, causal: bool, prefix=None) -> int:
    """Number of leading keys query row ``row`` may see.

    Non-causal without a prefix offset: all ``seq_len`` keys.  Otherwise the
    row sits at key position ``pos`` and sees keys up to and including it,
    clamped to ``[0, seq_len]``: ``pos = prefix + row`` when a prefix offset is
    given (prefix-causal), else ``pos = seq_len - seq_q + row`` (causal,
    bottom-right aligned).
    """
    if prefix is not None:
        pos = int(prefix) + int(row)
    elif causal:
        pos = int(seq_len) - int(seq_q) + int(row)
    else:
        return int(seq_len)
    return max(0, min(int(seq_len), pos + 1))


def gather_logical(cache, table_row, seq_len: int) -> np.ndarray:
    """Logical-order cache of one sequence: ``[seq_len, H, D]`` float64.

    ``cache`` is ``[num_pages, page_size, H, D]``; slot ``s`` of ``table_row``
    names the physical page that holds tokens ``[s*page_size, (s+1)*page_size)``.
    Only the first ``ceil(seq_len / page_size)`` slots are read.
    """
    page_size = cache.shape[1]
    n = pages_for(seq_len, page_size)
    if n == 0:
        return np.zeros((0,) + tuple(cache.shape[2:]), dtype=np.float64)
    pages = [np.asarray(cache[int(table_row[s])], dtype=np.float64) for s in range(n)]
    return np.concatenate(pages, axis=0)[: int(seq_len)]


def attend(q_row: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Softmax attention of one query row.

    ``q_row [D]``, ``keys [n, D]``, ``values [n, Dv]``.  Returns ``(o [Dv], lse)``
    with ``lse`` the natural log of the softmax denominator.  With no key
    (``n == 0``) the result is ``(0, -inf)``.
    """
    dv = values.shape[1]
    if keys.shape[0] == 0:
        return np.zeros(dv, dtype=np.float64), -math.inf
    s = scale * (keys @ q_row)
    m = s.max()
    p = np.exp(s - m)
    denom = p.sum()
    return (p @ values) / denom, float(m + np.log(denom))


def attention(q, k_cache, v_cache, block_table, seq_lens, scale: float, causal: bool = False,
              prefix_offset=None):
    """Exact paged attention, unsplit.

    ``q [B, Sq, Hq, D]``, ``k_cache [P, page_size, Hkv, D]``,
    ``v_cache [P, page_size, Hkv, Dv]``, ``block_table [B, >=W]`` (int),
    ``seq_lens [B]``, ``prefix_offset [B]`` or None.  Returns
    ``out [B, Sq, Hq, Dv]`` and ``lse [B, Sq, Hq]``.
    """
    q = np.asarray(q, dtype=np.float64)
    batch, seq_q, hq, _ = q.shape
    hkv = k_cache.shape[2]
    dv = v_cache.shape[3]
    group = hq // hkv
    out = np.zeros((batch, seq_q, hq, dv), dtype=np.float64)
    lse = np.full((batch, seq_q, hq), -math.inf, dtype=np.float64)
    for b in range(batch):
        seq_len = int(seq_lens[b])
        keys = gather_logical(k_cache, block_table[b], seq_len)
        values = gather_logical(v_cache, block_table[b], seq_len)
        prefix = None if prefix_offset is None else int(prefix_offset[b])
        for i in range(seq_q):
            lim = key_limit(seq_len, seq_q, i, causal, prefix)
            for h in range(hq):
                kvh = kv_head_of(h, group)
                out[b, i, h], lse[b, i, h] = attend(
                    q[b, i, h], keys[:lim, kvh], values[:lim, kvh], scale
                )
    return out, lse


def split_page_ranges(n_pages: int, num_splits: int):
    """Page ranges ``[(first, end), ...]`` of the ``num_splits`` splits.

    Each split takes ``ceil(n_pages / num_splits)`` pages; starts and ends are
    clamped to ``n_pages``, so trailing splits may be empty.
    """
    per = -(-int(n_pages) // int(num_splits))
    return [
        (min(s * per, n_pages), min((s + 1) * per, n_pages)) for s in range(int(num_splits))
    ]


def split_partials(q, k_cache, v_cache, block_table, seq_lens, scale: float, causal: bool,
                   num_splits: int, prefix_offset=None):
    """Per-split normalised outputs and LSEs.

    Returns ``part_out [B, Sq, Hq, S, Dv]`` and ``part_lse [B, Sq, Hq, S]``.
    Split ``k`` attends over the keys of its page range that the row may see;
    with none it yields ``(0, -inf)``.
    """
    q = np.asarray(q, dtype=np.float64)
    batch, seq_q, hq, _ = q.shape
    page_size = k_cache.shape[1]
    hkv = k_cache.shape[2]
    dv = v_cache.shape[3]
    group = hq // hkv
    part_out = np.zeros((batch, seq_q, hq, num_splits, dv), dtype=np.float64)
    part_lse = np.full((batch, seq_q, hq, num_splits), -math.inf, dtype=np.float64)
    for b in range(batch):
        seq_len = int(seq_lens[b])
        keys = gather_logical(k_cache, block_table[b], seq_len)
        values = gather_logical(v_cache, block_table[b], seq_len)
        ranges = split_page_ranges(pages_for(seq_len, page_size), num_splits)
        prefix = None if prefix_offset is None else int(prefix_offset[b])
        for i in range(seq_q):
            lim = key_limit(seq_len, seq_q, i, causal, prefix)
            for k, (first, end) in enumerate(ranges):
                lo = first * page_size
                hi = min(end * page_size, lim)
                for h in range(hq):
                    kvh = kv_head_of(h, group)
                    if hi <= lo:
                        continue  # empty split: (0, -inf) already stored
                    part_out[b, i, h, k], part_lse[b, i, h, k] = attend(
                        q[b, i, h], keys[lo:hi, kvh], values[lo:hi, kvh], scale
                    )
    return part_out, part_lse


def combine(part_out, part_lse):
    """Log-sum-exp merge of split partials.

    ``part_out [..., S, Dv]`` and ``part_lse [..., S]`` give ``out [..., Dv]``
    and ``lse [...]``.  Per row: ``M = max_s lse_s``; if ``M = -inf`` the row
    has no valid key anywhere and yields ``(0, -inf)``; else
    ``w_s = exp(lse_s - M)``, ``out = sum_s w_s o_s / sum_s w_s`` and
    ``lse = M + ln sum_s w_s``.
    """
    part_out = np.asarray(part_out, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    lead = part_lse.shape[:-1]
    dv = part_out.shape[-1]
    flat_o = part_out.reshape(-1, part_out.shape[-2], dv)
    flat_l = part_lse.reshape(-1, part_lse.shape[-1])
    out = np.zeros((flat_l.shape[0], dv), dtype=np.float64)
    lse = np.full(flat_l.shape[0], -math.inf, dtype=np.float64)
    for r in range(flat_l.shape[0]):
        m = flat_l[r].max()
        if m == -math.inf:
            continue
        w = np.exp(flat_l[r] - m)  # exp(-inf) = 0 for empty splits
        total = w.sum()
        out[r] = (w @ flat_o[r]) / total
        lse[r] = m + math.log(total)
    return out.reshape(lead + (dv,)), lse.reshape(lead)


def check_pages(block_table, seq_lens, page_size: int, num_pages: int, width=None):
    """Page-id range check over the slots each sequence reads.

    Sequence ``b`` reads slots ``[0, ceil(L_b / page_size))`` of its table row;
    it passes when its length lies in ``[0, width * page_size]`` (``width`` =
    the table width, the row's length when None) and every id in those slots
    lies in ``[0, num_pages)``.  Returns ``(first_bad, lens)``: the smallest
    failing batch index (-1 when none fails) and the lengths as attended,
    ``L_b`` for a passing sequence and 0 for a failing one.  Slots past a
    sequence's pages are never looked at, nor any slot of a sequence whose
    length is out of range.
    """
    first_bad = -1
    lens = []
    for b in range(len(seq_lens)):
        seq_len = int(seq_lens[b])
        w = len(block_table[b]) if width is None else int(width)
        ok = 0 <= seq_len <= w * int(page_size)
        if ok:
            for s in range(pages_for(seq_len, page_size)):
                page = int(block_table[b][s])
                if page < 0 or page >= int(num_pages):
                    ok = False
        if not ok and first_bad < 0:
            first_bad = b
        lens.append(seq_len if ok else 0)
    return first_bad, lens


def code_value(code: int, kind: str) -> float:
    """Real value of one 8-bit code.

    ``kind == "int8"``: the two's-complement integer of the byte.
    ``kind == "fp8_e4m3"``: sign bit, then a 4-bit exponent field ``e`` with
    bias 7, then a 3-bit mantissa field ``m``.  ``e == 0`` is subnormal,
    ``m / 8 * 2**-6``; otherwise ``(1 + m / 8) * 2**(e - 7)``; ``e == 15`` with
    ``m == 7`` is NaN (there is no infinity).
    """
    code = int(code) & 0xFF
    if kind == "int8":
        return float(code - 256 if code >= 128 else code)
    if kind != "fp8_e4m3":
        raise ValueError(kind)
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def dequantize_cache(codes, scales, kind: str) -> np.ndarray:
    """Exact float64 cache of quantized pages.

    ``codes [P, page_size, H, D]`` (8-bit patterns, any integer dtype) and
    ``scales [P, H]``: element ``[p, t, h, d]`` is
    ``scales[p, h] * code_value(codes[p, t, h, d])``.
    """
    codes = np.asarray(codes).astype(np.int64) & 0xFF
    table = np.array([code_value(c, kind) for c in range(256)], dtype=np.float64)
    values = table[codes]
    scales = np.asarray(scales, dtype=np.float64)
    return values * scales[:, None, :, None]
