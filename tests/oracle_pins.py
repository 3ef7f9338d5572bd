"""Checks that pin the CPU oracle to facts other than itself.

Each ``check_*`` function raises ``AssertionError`` when the oracle disagrees
with an independent source: a closed-form fixture under ``tests/golden``, a
pure-Python brute force, a closed form (``q = 0`` makes every valid score 0),
torch's float64 scaled-dot-product attention on the unpaged special case, or
an invariant (page shuffle, split equivalence, all-ones V).  The mutation
tests plant mistakes in the oracle and require at least one check to fail.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle.paged_attention as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
UNMAPPED = 0x7FFFFFFF


def _to_float(x):
    if isinstance(x, list):
        return [_to_float(v) for v in x]
    if x == "-inf":
        return -math.inf
    return float(x)


def load_golden(name):
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        raw = json.load(f)
    g = dict(raw)
    for key in ("q", "k_cache_pages", "v_cache_pages", "expected_out", "expected_lse",
                "expected_part_out", "expected_part_lse"):
        if key in raw:
            g[key] = np.array(_to_float(raw[key]), dtype=np.float64)
    g["block_table"] = np.array(raw["block_table"], dtype=np.int64)
    g["seq_lens"] = np.array(raw["seq_lens"], dtype=np.int64)
    return g


def _close(a, b, tol=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert not np.isnan(a).any(), "NaN in oracle output"
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        diff = np.where(same_inf, 0.0, np.abs(a - b))
    assert (diff <= tol).all(), f"max diff {np.nanmax(diff)}"


# ----------------------------------------------------------------------------- fixtures
def check_golden_hand():
    g = load_golden("hand_case")
    out, lse = O.attention(g["q"], g["k_cache_pages"], g["v_cache_pages"], g["block_table"],
                           g["seq_lens"], g["scale"], g["causal"])
    _close(out, g["expected_out"])
    _close(lse, g["expected_lse"])


def check_golden_split(name="split_closed_form"):
    g = load_golden(name)
    args = (g["q"], g["k_cache_pages"], g["v_cache_pages"], g["block_table"], g["seq_lens"],
            g["scale"], g["causal"])
    po, pl = O.split_partials(*args, g["num_splits"])
    _close(po, g["expected_part_out"])
    _close(pl, g["expected_part_lse"])
    out, lse = O.combine(po, pl)
    _close(out, g["expected_out"])
    _close(lse, g["expected_lse"])
    out2, lse2 = O.attention(*args)
    _close(out2, g["expected_out"])
    _close(lse2, g["expected_lse"])


def check_golden_causal():
    check_golden_split("causal_masked_split")


def check_golden_split_paged(names=("split_paged_closed_form", "split_paged_causal")):
    """Multi-token pages, a table wider than the sequences' page counts and
    ragged lengths: the partials of every listed split count, their combine
    and the unsplit result against the fixtures' closed forms."""
    for name in names:
        with open(os.path.join(GOLDEN, name + ".json")) as f:
            raw = json.load(f)
        g = load_golden(name)
        args = (g["q"], g["k_cache_pages"], g["v_cache_pages"], g["block_table"],
                g["seq_lens"], g["scale"], g["causal"])
        for s, exp in raw["splits"].items():
            po, pl = O.split_partials(*args, int(s))
            _close(po, np.array(_to_float(exp["expected_part_out"])))
            _close(pl, np.array(_to_float(exp["expected_part_lse"])))
            out, lse = O.combine(po, pl)
            _close(out, g["expected_out"])
            _close(lse, g["expected_lse"])
        out, lse = O.attention(*args)
        _close(out, g["expected_out"])
        _close(lse, g["expected_lse"])


# ----------------------------------------------------------------------------- problems
def random_problem(rng, batch=3, seq_q=1, hq=4, hkv=2, d=3, dv=None, ps=2, lens=None,
                   width=None, extra_pages=3, poison=True):
    """Small random paged problem in NumPy (pages shuffled, unused slots unmapped,
    unreferenced pages and in-page tails NaN)."""
    dv = d if dv is None else dv
    if lens is None:
        lens = [int(x) for x in rng.integers(0, 11, size=batch)]
    n_per = [-(-x // ps) for x in lens]
    width = max(max(n_per, default=0), 1) if width is None else width
    used = sum(n_per)
    phys = used + extra_pages
    perm = rng.permutation(phys)
    table = np.full((len(lens), width), UNMAPPED, dtype=np.int64)
    pos = 0
    for b, n in enumerate(n_per):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    k_cache = rng.standard_normal((phys, ps, hkv, d))
    v_cache = rng.standard_normal((phys, ps, hkv, dv))
    if poison:
        unused = perm[used:]
        k_cache[unused] = np.nan
        v_cache[unused] = np.nan
        for b, (x, n) in enumerate(zip(lens, n_per)):
            tail = n * ps - x
            if n and tail:
                k_cache[table[b, n - 1], ps - tail:] = np.nan
                v_cache[table[b, n - 1], ps - tail:] = np.nan
    q = rng.standard_normal((len(lens), seq_q, hq, d))
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, block_table=table,
                seq_lens=np.array(lens, dtype=np.int64), scale=1.0 / math.sqrt(d))


def brute_force(q, k_cache, v_cache, block_table, seq_lens, scale, causal, prefix=None):
    """Pure-Python attention: one key at a time, straight from the page table.
    With ``prefix`` (one offset per sequence) row i sits at key prefix[b] + i
    and the causal mask applies."""
    batch, seq_q, hq, d = q.shape
    ps, hkv, dv = k_cache.shape[1], k_cache.shape[2], v_cache.shape[3]
    group = hq // hkv
    out = [[[[0.0] * dv for _ in range(hq)] for _ in range(seq_q)] for _ in range(batch)]
    lse = [[[-math.inf] * hq for _ in range(seq_q)] for _ in range(batch)]
    for b in range(batch):
        length = int(seq_lens[b])
        for i in range(seq_q):
            masked = causal or prefix is not None
            position = length - seq_q + i if prefix is None else int(prefix[b]) + i
            for h in range(hq):
                kvh = h // group
                scores, rows = [], []
                for j in range(length):
                    if masked and j > position:
                        continue
                    page = int(block_table[b][j // ps])
                    slot = j % ps
                    dot = 0.0
                    for e in range(d):
                        dot += float(q[b, i, h, e]) * float(k_cache[page, slot, kvh, e])
                    scores.append(dot * scale)
                    rows.append([float(v_cache[page, slot, kvh, e]) for e in range(dv)])
                if not scores:
                    continue
                top = max(scores)
                weights = [math.exp(s - top) for s in scores]
                total = sum(weights)
                out[b][i][h] = [sum(w * r[e] for w, r in zip(weights, rows)) / total
                                for e in range(dv)]
                lse[b][i][h] = top + math.log(total)
    return np.array(out), np.array(lse)


# ----------------------------------------------------------------------------- checks
def check_brute_force(seed=0):
    rng = np.random.default_rng(seed)
    cases = [
        dict(batch=3, seq_q=1, hq=4, hkv=2, d=3, ps=2, causal=False),
        dict(batch=2, seq_q=3, hq=2, hkv=1, d=4, ps=3, causal=True),
        dict(batch=2, seq_q=2, hq=6, hkv=3, d=2, dv=3, ps=2, causal=True),
        dict(batch=2, seq_q=1, hq=8, hkv=2, d=5, ps=4, causal=False),
    ]
    for c in cases:
        causal = c.pop("causal")
        p = random_problem(rng, **c)
        args = (p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seq_lens"], p["scale"])
        out, lse = O.attention(*args, causal)
        bout, blse = brute_force(*args, causal)
        _close(out, bout, 1e-12)
        _close(lse, blse, 1e-12)
    # prefix-causal: offsets below 0, inside, at and past the sequence
    p = random_problem(rng, batch=4, seq_q=3, hq=4, hkv=2, d=3, ps=2, lens=[5, 7, 2, 6])
    args = (p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seq_lens"], p["scale"])
    for prefix in ([-2, 3, 2, 0], [1, 0, -1, 9], [4, 6, 0, 3]):
        for causal in (False, True):
            out, lse = O.attention(*args, causal, prefix_offset=prefix)
            bout, blse = brute_force(*args, causal, prefix=prefix)
            _close(out, bout, 1e-12)
            _close(lse, blse, 1e-12)


def check_q_zero_decode(seed=1):
    """q = 0: every valid score is 0, so lse = ln(L) and out = mean of the valid V rows."""
    rng = np.random.default_rng(seed)
    p = random_problem(rng, batch=5, hq=4, hkv=2, d=3, ps=3, lens=[1, 2, 7, 9, 12])
    p["q"][:] = 0.0
    out, lse = O.attention(p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seq_lens"],
                           p["scale"], False)
    ps = p["k_cache"].shape[1]
    for b, length in enumerate(p["seq_lens"]):
        for h in range(4):
            rows = [p["v_cache"][p["block_table"][b, j // ps], j % ps, h // 2] for j in range(length)]
            _close(out[b, 0, h], np.mean(rows, axis=0), 1e-12)
            _close(lse[b, 0, h], math.log(length), 1e-12)


def check_q_zero_causal(seed=2):
    """q = 0, causal bottom-right: row i sees min(L - Sq + i + 1, L) keys (none if <= 0)."""
    rng = np.random.default_rng(seed)
    for seq_q in (1, 3, 5):
        p = random_problem(rng, batch=3, seq_q=seq_q, hq=2, hkv=2, d=2, ps=2, lens=[3, 5, 8])
        p["q"][:] = 0.0
        out, lse = O.attention(p["q"], p["k_cache"], p["v_cache"], p["block_table"],
                               p["seq_lens"], p["scale"], True)
        for b, length in enumerate(p["seq_lens"]):
            for i in range(seq_q):
                visible = min(length - seq_q + i + 1, length)
                for h in range(2):
                    if visible <= 0:
                        assert lse[b, i, h] == -math.inf and (out[b, i, h] == 0).all()
                        continue
                    rows = [p["v_cache"][p["block_table"][b, j // 2], j % 2, h]
                            for j in range(visible)]
                    _close(out[b, i, h], np.mean(rows, axis=0), 1e-12)
                    _close(lse[b, i, h], math.log(visible), 1e-12)


def check_prefix_q_zero():
    """q = 0 with prefix offsets: lse = ln(keys visible); the counts below are
    worked out by hand for L = 10, Sq = 4 (row i sits at key prefix + i)."""
    rng = np.random.default_rng(11)
    p = random_problem(rng, batch=4, seq_q=4, hq=2, hkv=1, d=2, ps=3, lens=[10, 10, 10, 10])
    p["q"][:] = 0.0
    prefix = [4, -2, 12, 0]
    visible = [[5, 6, 7, 8],      # keys 0..4, 0..5, 0..6, 0..7
               [0, 0, 1, 2],      # rows at -2 and -1 see nothing
               [10, 10, 10, 10],  # past the end: every key
               [1, 2, 3, 4]]
    for causal in (False, True):
        out, lse = O.attention(p["q"], p["k_cache"], p["v_cache"], p["block_table"],
                               p["seq_lens"], p["scale"], causal, prefix_offset=prefix)
        for b in range(4):
            for i in range(4):
                for h in range(2):
                    n = visible[b][i]
                    if n == 0:
                        assert lse[b, i, h] == -math.inf and (out[b, i, h] == 0).all()
                        continue
                    rows = [p["v_cache"][p["block_table"][b, j // 3], j % 3, 0] for j in range(n)]
                    _close(out[b, i, h], np.mean(rows, axis=0), 1e-12)
                    _close(lse[b, i, h], math.log(n), 1e-12)


def check_prefix_bottom_right(seed=12):
    """A prefix offset of L - Sq is bottom-right causal, bit for bit, split or not."""
    rng = np.random.default_rng(seed)
    p = random_problem(rng, batch=4, seq_q=3, hq=4, hkv=2, d=3, ps=2, lens=[1, 4, 9, 16], width=8)
    args = (p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seq_lens"], p["scale"])
    prefix = [int(x) - 3 for x in p["seq_lens"]]
    for x, y in zip(O.attention(*args, True), O.attention(*args, False, prefix_offset=prefix)):
        assert np.array_equal(x, y)
    for x, y in zip(O.split_partials(*args, True, 3),
                    O.split_partials(*args, False, 3, prefix_offset=prefix)):
        assert np.array_equal(x, y)


def check_prefix_split_equivalence(seed=13):
    """With prefix offsets too, combining the split partials gives the unsplit result."""
    rng = np.random.default_rng(seed)
    p = random_problem(rng, batch=4, seq_q=3, hq=4, hkv=2, d=3, ps=2, lens=[3, 8, 11, 16], width=8)
    args = (p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seq_lens"], p["scale"])
    prefix = [-1, 2, 20, 7]
    out, lse = O.attention(*args, False, prefix_offset=prefix)
    assert np.isinf(lse[0, 0]).all() and np.isfinite(lse[1]).all()
    for splits in (1, 2, 3, 5, 8):
        po, pl = O.split_partials(*args, False, splits, prefix_offset=prefix)
        assert not np.isnan(po).any()
        co, cl = O.combine(po, pl)
        _close(co, out, 1e-12)
        _close(cl, lse, 1e-12)


def check_page_range():
    """Page-id range check on hand-made tables (page size 4, 6 pages)."""
    table = [[0, 5, UNMAPPED],     # L = 8: slots 0, 1 read, both in range
             [5, 6, 0],            # L = 5: slot 1 holds 6 = num_pages
             [3, -1, 2],           # L = 9: slot 1 negative
             [1, UNMAPPED, -7],    # L = 4: one slot read; the rest never looked at
             [UNMAPPED, 9, 9],     # L = 0: nothing read
             [2, 4, 5]]            # L = 12: all three slots, all in range
    lens = [8, 5, 9, 4, 0, 12]
    first_bad, attended = O.check_pages(table, lens, 4, 6)
    assert first_bad == 1
    assert attended == [8, 0, 0, 4, 0, 12]
    assert O.check_pages(table[2:], lens[2:], 4, 6) == (0, [0, 4, 0, 12])
    assert O.check_pages(table[3:], lens[3:], 4, 6) == (-1, [4, 0, 12])
    # the same tables against 7 pages: id 6 becomes valid
    assert O.check_pages(table, lens, 4, 7) == (2, [8, 5, 0, 4, 0, 12])
    # lengths past the table (3 slots of 4 tokens) or negative are rejected unread
    assert O.check_pages(table, [8, 13, -1, 0, 0, 0], 4, 6) == (1, [8, 0, 0, 0, 0, 0])
    # a table view narrower than its rows: the view's width bounds the length
    assert O.check_pages([[0, 1, 2], [3, 4, 5]], [8, 9], 4, 6) == (-1, [8, 9])
    assert O.check_pages([[0, 1, 2], [3, 4, 5]], [8, 9], 4, 6, width=2) == (1, [8, 0])


def check_code_values():
    """8-bit codes: special fp8 values worked out by hand from the format, and
    every code against torch's float8_e4m3fn and NumPy's int8 decoding."""
    import torch

    hand = {0x00: 0.0, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x48: 4.0, 0x50: 8.0, 0x7E: 448.0,
            0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0xB0: -0.5, 0xB8: -1.0,
            0xC4: -3.0, 0xFE: -448.0}
    for code, value in hand.items():
        assert O.code_value(code, "fp8_e4m3") == value, hex(code)
    assert math.isnan(O.code_value(0x7F, "fp8_e4m3")) and math.isnan(O.code_value(0xFF, "fp8_e4m3"))
    assert math.copysign(1.0, O.code_value(0x80, "fp8_e4m3")) == -1.0
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mine = np.array([O.code_value(c, "fp8_e4m3") for c in range(256)])
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(mine)) and np.array_equal(lib[~nan], mine[~nan])
    ints = np.arange(256, dtype=np.uint8).view(np.int8).astype(np.float64)
    assert [O.code_value(c, "int8") for c in range(256)] == ints.tolist()


def check_golden_quantized():
    """The hand case stored as int8 and as fp8 codes with per-(page, kv head) scales."""
    with open(os.path.join(GOLDEN, "quantized_hand_case.json")) as f:
        g = json.load(f)
    for kind, v in g["variants"].items():
        k = O.dequantize_cache(np.array(v["k_codes"]), np.array(v["k_scales"]), kind)
        vv = O.dequantize_cache(np.array(v["v_codes"]), np.array(v["v_scales"]), kind)
        out, lse = O.attention(np.array(g["q"]), k, vv, np.array(g["block_table"]),
                               np.array(g["seq_lens"]), g["scale"], g["causal"])
        _close(out, np.array(g["expected_out"]), 1e-15)
        _close(lse, np.array(g["expected_lse"]), 1e-15)


def check_quantized_scale_placement():
    """q = 0, so every output is the mean of the visible V rows; the means below
    are worked out by hand.  Hkv = 2 (G = 2), page size 2, L = 3, table [1, 0]:
    tokens 0 and 1 live in page 1, token 2 in page 0; V codes are 1 in kv head
    0 and 2 in kv head 1; V scales [page][kv head] = [[6, 1], [3, 7], [100, 100]].
    kv head 0: (3 + 3 + 6) / 3 = 4; kv head 1: (14 + 14 + 2) / 3 = 10."""
    for kind, one, two in (("int8", 1, 2), ("fp8_e4m3", 0x38, 0x40)):
        v_codes = np.zeros((3, 2, 2, 4), dtype=np.int64)
        v_codes[:, :, 0, :] = one
        v_codes[:, :, 1, :] = two
        v_scales = np.array([[6.0, 1.0], [3.0, 7.0], [100.0, 100.0]])
        k_codes = np.zeros((3, 2, 2, 4), dtype=np.int64)
        k_scales = np.ones((3, 2))
        q = np.zeros((1, 1, 4, 4))
        table = np.array([[1, 0, UNMAPPED]])
        out, lse = O.attention(q, O.dequantize_cache(k_codes, k_scales, kind),
                               O.dequantize_cache(v_codes, v_scales, kind), table,
                               np.array([3]), 0.5, False)
        _close(out[0, 0, :2], np.full((2, 4), 4.0), 1e-13)
        _close(out[0, 0, 2:], np.full((2, 4), 10.0), 1e-13)
        _close(lse, np.full((1, 1, 4), math.log(3.0)), 1e-13)


def quantized_problem(rng, kind, batch=3, seq_q=2, hq=4, hkv=2, d=4, ps=2, lens=(3, 7, 10)):
    """Random codes (fp8 NaN codes excluded) and scales of both signs."""
    p = random_problem(rng, batch=batch, seq_q=seq_q, hq=hq, hkv=hkv, d=d, ps=ps, lens=list(lens),
                       poison=False)
    phys = p["k_cache"].shape[0]
    allowed = np.array([c for c in range(256) if kind == "int8" or (c & 0x7F) != 0x7F])
    p["k_codes"] = rng.choice(allowed, size=(phys, ps, hkv, d))
    p["v_codes"] = rng.choice(allowed, size=(phys, ps, hkv, d))
    p["k_scales"] = rng.uniform(-1.0, 1.0, size=(phys, hkv)) / (40.0 if kind == "int8" else 1.0)
    p["v_scales"] = rng.uniform(-1.0, 1.0, size=(phys, hkv))
    return p


def check_quantized_scale_laws(seed=14):
    """Multiplying every V scale by c multiplies the output by c and leaves the
    LSE alone; multiplying every K scale by c equals multiplying the softmax
    scale by c."""
    rng = np.random.default_rng(seed)
    for kind in ("int8", "fp8_e4m3"):
        p = quantized_problem(rng, kind)
        k = O.dequantize_cache(p["k_codes"], p["k_scales"], kind)
        v = O.dequantize_cache(p["v_codes"], p["v_scales"], kind)
        rest = (p["block_table"], p["seq_lens"])
        out, lse = O.attention(p["q"], k, v, *rest, p["scale"], True)
        v4 = O.dequantize_cache(p["v_codes"], p["v_scales"] * 4.0, kind)
        out4, lse4 = O.attention(p["q"], k, v4, *rest, p["scale"], True)
        _close(out4, 4.0 * out, 1e-12)
        _close(lse4, lse, 1e-12)
        k3 = O.dequantize_cache(p["k_codes"], p["k_scales"] * 3.0, kind)
        out3, lse3 = O.attention(p["q"], k3, v, *rest, p["scale"], True)
        outs, lses = O.attention(p["q"], k, v, *rest, p["scale"] * 3.0, True)
        _close(out3, outs, 1e-12)
        _close(lse3, lses, 1e-12)


def check_sdpa(seed=3):
    """Unpaged special case against torch's float64 scaled_dot_product_attention."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(seed)
    for seq_q, causal, group in ((1, False, 4), (6, True, 2), (1, False, 1)):
        hkv = 2
        length = 6 if causal else 11
        p = random_problem(rng, batch=2, seq_q=seq_q, hq=hkv * group, hkv=hkv, d=8, ps=4,
                           lens=[length, length])
        out, _ = O.attention(p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seq_lens"],
                             p["scale"], causal)
        kc = torch.from_numpy(p["k_cache"])
        vc = torch.from_numpy(p["v_cache"])
        tok = torch.arange(length)
        for b in range(2):
            pages = torch.from_numpy(p["block_table"][b])[tok // 4]
            keys = kc[pages, tok % 4].repeat_interleave(group, dim=1)    # [L, Hq, D]
            vals = vc[pages, tok % 4].repeat_interleave(group, dim=1)
            qb = torch.from_numpy(p["q"][b]).transpose(0, 1)              # [Hq, Sq, D]
            ref = F.scaled_dot_product_attention(qb, keys.transpose(0, 1), vals.transpose(0, 1),
                                                 is_causal=causal, scale=p["scale"])
            _close(out[b], ref.transpose(0, 1).numpy(), 1e-12)


def check_shuffle_invariance(seed=4):
    """Relabelling physical pages together with the table changes nothing, bit for bit."""
    rng = np.random.default_rng(seed)
    p = random_problem(rng, batch=4, seq_q=2, hq=4, hkv=2, d=3, ps=2, lens=[3, 0, 6, 9])
    phys = p["k_cache"].shape[0]
    relabel = rng.permutation(phys)               # old page id -> new page id
    k2 = np.empty_like(p["k_cache"])
    v2 = np.empty_like(p["v_cache"])
    k2[relabel] = p["k_cache"]
    v2[relabel] = p["v_cache"]
    t2 = p["block_table"].copy()
    mapped = t2 != UNMAPPED
    t2[mapped] = relabel[t2[mapped]]
    for causal in (False, True):
        a = O.attention(p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seq_lens"],
                        p["scale"], causal)
        b = O.attention(p["q"], k2, v2, t2, p["seq_lens"], p["scale"], causal)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def check_split_equivalence(seed=5):
    """Combining the split partials reproduces the unsplit result for every S."""
    rng = np.random.default_rng(seed)
    for causal, seq_q in ((False, 1), (True, 4)):
        p = random_problem(rng, batch=4, seq_q=seq_q, hq=4, hkv=2, d=3, ps=2,
                           lens=[1, 4, 9, 16], width=8)
        args = (p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seq_lens"], p["scale"],
                causal)
        out, lse = O.attention(*args)
        for splits in range(1, 11):
            po, pl = O.split_partials(*args, splits)
            assert not np.isnan(po).any() and not np.isnan(pl).any()
            co, cl = O.combine(po, pl)
            _close(co, out, 1e-12)
            _close(cl, lse, 1e-12)


def check_v_ones(seed=6):
    """V = 1 everywhere valid: every row with a valid key outputs exactly 1 (softmax rows sum to 1)."""
    rng = np.random.default_rng(seed)
    p = random_problem(rng, batch=3, seq_q=3, hq=4, hkv=2, d=3, ps=2, lens=[2, 5, 8], poison=False)
    p["v_cache"][:] = 1.0
    out, lse = O.attention(p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seq_lens"],
                           p["scale"], True)
    valid = np.isfinite(lse)
    assert valid.any()
    _close(out[valid], np.ones_like(out[valid]), 1e-14)


def check_empty():
    """A sequence of length 0 yields output 0 and LSE -inf in every split."""
    rng = np.random.default_rng(7)
    p = random_problem(rng, batch=2, hq=2, hkv=1, d=2, ps=2, lens=[0, 3])
    out, lse = O.attention(p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seq_lens"],
                           p["scale"], False)
    assert (out[0] == 0).all() and (lse[0] == -math.inf).all()
    assert np.isfinite(lse[1]).all()
    po, pl = O.split_partials(p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seq_lens"],
                              p["scale"], False, 3)
    assert (po[0] == 0).all() and (pl[0] == -math.inf).all()


def check_split_ranges():
    """Ceiling division of pages per split with clamped ends."""
    assert O.split_page_ranges(3, 2) == [(0, 2), (2, 3)]
    assert O.split_page_ranges(5, 8) == [(0, 1), (1, 2), (2, 3), (3, 4), (4, 5), (5, 5), (5, 5),
                                         (5, 5)]
    assert O.split_page_ranges(0, 3) == [(0, 0), (0, 0), (0, 0)]
    assert O.split_page_ranges(32, 4) == [(0, 8), (8, 16), (16, 24), (24, 32)]
    # 17 tokens of 16-token pages, 8 splits: 2 pages, so splits 2..7 are empty
    assert O.split_page_ranges(2, 8)[2:] == [(2, 2)] * 6
    for n in range(0, 40):
        for s in range(1, 12):
            r = O.split_page_ranges(n, s)
            assert r[0][0] == 0 and r[-1][1] == n
            assert all(a <= b for a, b in r)
            assert all(r[k][1] == r[k + 1][0] for k in range(s - 1))


ALL_CHECKS = [
    check_golden_hand,
    check_golden_split,
    check_golden_causal,
    check_golden_split_paged,
    check_brute_force,
    check_q_zero_decode,
    check_q_zero_causal,
    check_sdpa,
    check_shuffle_invariance,
    check_split_equivalence,
    check_v_ones,
    check_empty,
    check_split_ranges,
    check_prefix_q_zero,
    check_prefix_bottom_right,
    check_prefix_split_equivalence,
    check_page_range,
    check_code_values,
    check_golden_quantized,
    check_quantized_scale_placement,
    check_quantized_scale_laws,
]
