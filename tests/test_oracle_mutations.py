"""Plants plausible mistakes in the oracle (on the CPU) and requires the pins to catch each."""

import math

import numpy as np
import pytest

import oracle.paged_attention as O
import oracle_pins

_orig_attend = O.attend
_orig_key_limit = O.key_limit
_orig_gather = O.gather_logical
_orig_check_pages = O.check_pages
_orig_code_value = O.code_value
_orig_dequantize = O.dequantize_cache


def code_value_fp8_bias8(code, kind):
    v = _orig_code_value(code, kind)
    return v / 2.0 if kind == "fp8_e4m3" else v


def code_value_fp8_subnormal(code, kind):
    if kind == "fp8_e4m3" and (int(code) >> 3) & 0xF == 0:
        return _orig_code_value(code, kind) / 2.0
    return _orig_code_value(code, kind)


def code_value_int8_unsigned(code, kind):
    return float(int(code) & 0xFF) if kind == "int8" else _orig_code_value(code, kind)


def dequantize_no_scale(codes, scales, kind):
    return _orig_dequantize(codes, np.ones_like(np.asarray(scales, dtype=np.float64)), kind)


def dequantize_heads_reversed(codes, scales, kind):
    return _orig_dequantize(codes, np.asarray(scales)[:, ::-1], kind)


def dequantize_pages_reversed(codes, scales, kind):
    return _orig_dequantize(codes, np.asarray(scales)[::-1], kind)


def check_pages_length_unbounded(block_table, seq_lens, page_size, num_pages, width=None):
    lens = [max(0, min(int(x), len(block_table[b]) * page_size)) for b, x in enumerate(seq_lens)]
    first_bad, att = _orig_check_pages(block_table, lens, page_size, num_pages, width)
    return first_bad, [a if int(x) == y else y for a, x, y in zip(att, seq_lens, lens)]


def attend_no_scale(q_row, keys, values, scale):
    return _orig_attend(q_row, keys, values, 1.0)


def attend_sign_flip(q_row, keys, values, scale):
    return _orig_attend(q_row, keys, values, -scale)


def attend_lse_without_max(q_row, keys, values, scale):
    o, lse = _orig_attend(q_row, keys, values, scale)
    if keys.shape[0] == 0:
        return o, lse
    s = scale * (keys @ q_row)
    return o, float(np.log(np.exp(s - s.max()).sum()))


def attend_reversed_values(q_row, keys, values, scale):
    return _orig_attend(q_row, keys, values[::-1], scale)


def key_limit_off_by_one(seq_len, seq_q, row, causal, prefix=None):
    if prefix is not None:
        return _orig_key_limit(seq_len, seq_q, row, causal, prefix)
    if not causal:
        return int(seq_len)
    return max(0, min(int(seq_len), int(seq_len) - int(seq_q) + int(row)))


def key_limit_top_left(seq_len, seq_q, row, causal, prefix=None):
    if prefix is not None:
        return _orig_key_limit(seq_len, seq_q, row, causal, prefix)
    if not causal:
        return int(seq_len)
    return max(0, min(int(seq_len), int(row) + 1))


def key_limit_prefix_off_by_one(seq_len, seq_q, row, causal, prefix=None):
    if prefix is None:
        return _orig_key_limit(seq_len, seq_q, row, causal)
    return max(0, min(int(seq_len), int(prefix) + int(row)))


def key_limit_prefix_ignores_row(seq_len, seq_q, row, causal, prefix=None):
    if prefix is None:
        return _orig_key_limit(seq_len, seq_q, row, causal)
    return max(0, min(int(seq_len), int(prefix) + 1))


def key_limit_prefix_only_when_causal(seq_len, seq_q, row, causal, prefix=None):
    return _orig_key_limit(seq_len, seq_q, row, causal, prefix if causal else None)


def check_pages_whole_row(block_table, seq_lens, page_size, num_pages, width=None):
    first_bad, lens = -1, []
    for b, length in enumerate(seq_lens):
        ok = all(0 <= int(x) < num_pages for x in block_table[b])
        if not ok and first_bad < 0:
            first_bad = b
        lens.append(int(length) if ok else 0)
    return first_bad, lens


def check_pages_inclusive_bound(block_table, seq_lens, page_size, num_pages, width=None):
    return _orig_check_pages(block_table, seq_lens, page_size, num_pages + 1, width)


def check_pages_last_bad(block_table, seq_lens, page_size, num_pages, width=None):
    first_bad, lens = _orig_check_pages(block_table, seq_lens, page_size, num_pages, width)
    bad = [b for b, (x, y) in enumerate(zip(lens, seq_lens)) if x != int(y)]
    return (bad[-1] if bad else -1), lens


def gather_reversed_pages(cache, table_row, seq_len):
    ps = cache.shape[1]
    n = O.pages_for(seq_len, ps)
    if n == 0:
        return _orig_gather(cache, table_row, seq_len)
    pages = [np.asarray(cache[int(table_row[s])], dtype=np.float64) for s in reversed(range(n))]
    return np.concatenate(pages, axis=0)[: int(seq_len)]


def split_floor_division(n_pages, num_splits):
    per = int(n_pages) // int(num_splits)
    return [(min(s * per, n_pages), min((s + 1) * per, n_pages)) for s in range(int(num_splits))]


def split_partials_token_granular(q, k_cache, v_cache, block_table, seq_lens, scale, causal,
                                  num_splits, prefix_offset=None):
    """Splits cut by ceil(L / S) tokens instead of whole pages: the same caches
    re-expressed as one-token pages, so the page-granular code splits tokens."""
    ps = k_cache.shape[1]
    k1 = np.asarray(k_cache).reshape((-1, 1) + k_cache.shape[2:])
    v1 = np.asarray(v_cache).reshape((-1, 1) + v_cache.shape[2:])
    bt = np.asarray(block_table, dtype=np.int64)
    table = np.zeros((bt.shape[0], bt.shape[1] * ps), dtype=np.int64)
    for b, length in enumerate(seq_lens):
        for t in range(int(length)):
            table[b, t] = bt[b, t // ps] * ps + t % ps
    return _orig_split_partials(q, k1, v1, table, seq_lens, scale, causal, num_splits,
                                prefix_offset)


def split_partials_width_sized(q, k_cache, v_cache, block_table, seq_lens, scale, causal,
                               num_splits, prefix_offset=None):
    """Pages per split sized by the table width W instead of the sequence's own
    page count n (ends still clamped to n)."""
    width = np.asarray(block_table).shape[1]

    def by_width(n_pages, splits):
        return [(min(a, n_pages), min(b, n_pages)) for a, b in _orig_split_ranges(width, splits)]

    saved = O.split_page_ranges
    O.split_page_ranges = by_width
    try:
        return _orig_split_partials(q, k_cache, v_cache, block_table, seq_lens, scale, causal,
                                    num_splits, prefix_offset)
    finally:
        O.split_page_ranges = saved


def combine_lse_double_max(part_out, part_lse):
    out, lse = _orig_combine(part_out, part_lse)
    m = np.max(np.asarray(part_lse), axis=-1)
    return out, np.where(np.isfinite(lse), lse + np.where(np.isfinite(m), m, 0.0), lse)


_orig_combine = O.combine
_orig_split_partials = O.split_partials
_orig_split_ranges = O.split_page_ranges

MUTATIONS = [
    ("kv_head_of", lambda q_head, group: q_head % group if group > 1 else q_head),
    ("attend", attend_no_scale),
    ("attend", attend_sign_flip),
    ("attend", attend_lse_without_max),
    ("attend", attend_reversed_values),
    ("key_limit", key_limit_off_by_one),
    ("key_limit", key_limit_top_left),
    ("key_limit", key_limit_prefix_off_by_one),
    ("key_limit", key_limit_prefix_ignores_row),
    ("key_limit", key_limit_prefix_only_when_causal),
    ("check_pages", check_pages_whole_row),
    ("check_pages", check_pages_inclusive_bound),
    ("check_pages", check_pages_last_bad),
    ("check_pages", check_pages_length_unbounded),
    ("code_value", code_value_fp8_bias8),
    ("code_value", code_value_fp8_subnormal),
    ("code_value", code_value_int8_unsigned),
    ("dequantize_cache", dequantize_no_scale),
    ("dequantize_cache", dequantize_heads_reversed),
    ("dequantize_cache", dequantize_pages_reversed),
    ("gather_logical", gather_reversed_pages),
    ("split_page_ranges", split_floor_division),
    ("split_partials", split_partials_token_granular),
    ("split_partials", split_partials_width_sized),
    ("combine", combine_lse_double_max),
]


@pytest.mark.parametrize("name,mutant", MUTATIONS,
                         ids=[f"{n}:{getattr(m, '__name__', 'lambda')}" for n, m in MUTATIONS])
def test_pins_catch_planted_mistake(monkeypatch, name, mutant):
    monkeypatch.setattr(O, name, mutant)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(exc).__name__))
    assert caught, f"no pin caught the planted mistake in {name}"
