"""Writes the closed-form fixtures in this folder.

The pages print no worked numeric example, so each fixture is a case built so
that its answer is a closed form (derivation stored beside the numbers).  The
values here come from ``math`` only; nothing is computed by the oracle or by
the HIP path.  Run ``python tests/golden/make_golden.py`` to rewrite them.
"""

import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
NEG_INF = "-inf"   # JSON has no infinity; readers map this string to -inf
UNMAPPED = 0x7FFFFFFF  # block-table id of a slot that holds no page

FIXTURES = {
    "hand_case": {
        "description": "Hand-worked paged attention case. One sequence of two tokens stored in two "
                       "one-token pages in swapped physical order.",
        "citation": "Definition of the result: softmax attention over the logical-order cache "
                    "(rocMLIR 'Paged Attention: rocmlir-gen changes', Technical Details, CPU "
                    "Validation); the paged input is a view of that cache (rocMLIR 'Paged "
                    "Attention: migraphx & highlevel pipeline changes', note on rock.deref). The "
                    "pages print no worked example; this case is constructed so the answer is a "
                    "closed form.",
        "derivation": "scores: q.k0 = 0, q.k1 = ln 3; weights e^0 = 1 and e^(ln 3) = 3 sum to 4; "
                      "out = (1*v0 + 3*v1)/4 = (0.25, 0.75); lse = ln(1 + 3) = ln 4.",
        "dtype": "f32", "page_size": 1, "num_q_heads": 1, "num_kv_heads": 1, "head_dim": 2,
        "scale": 1.0, "causal": False,
        "q": [[[[1.0, 0.0]]]],
        "k_cache_pages": [[[[math.log(3.0), 0.0]]], [[[0.0, 0.0]]]],
        "v_cache_pages": [[[[0.0, 1.0]]], [[[1.0, 0.0]]]],
        "block_table": [[1, 0]],
        "seq_lens": [2],
        "expected_out": [[[[0.25, 0.75]]]],
        "expected_lse": [[[math.log(4.0)]]],
    },
    "split_closed_form": {
        "description": "Split-KV closed form: L=3 one-token pages, S=2 splits, q=0 so every valid "
                       "score is 0 and each split's output is the mean of its V rows.",
        "citation": "Split ranges by ceiling division with the end clamped, per-split normalised "
                    "output and LSE, and the LSE combine: rocMLIR 'Fix split-kv attention masking "
                    "and sweep RMS', Technical Details (non-causal split-KV iteration math; "
                    "scaleFinalOutput; host reference f32 combine).",
        "derivation": "P = ceil(3/2) = 2: split 0 holds tokens 0,1 -> out (v0+v1)/2 = (0.5, 0.5), "
                      "lse ln 2; split 1 holds token 2 -> out v2 = (2, 2), lse ln 1 = 0. Combine: "
                      "weights 2 and 1 (exp of lse minus max, times 2) -> out (2*(0.5,0.5) + "
                      "1*(2,2))/3 = (1, 1), lse ln 2 + ln(1 + 1/2) = ln 3.",
        "dtype": "f32", "page_size": 1, "num_q_heads": 1, "num_kv_heads": 1, "head_dim": 2,
        "scale": 1.0, "causal": False, "num_splits": 2,
        "q": [[[[0.0, 0.0]]]],
        "k_cache_pages": [[[[0.3, -1.0]]], [[[2.0, 0.5]]], [[[-0.7, 0.1]]]],
        "v_cache_pages": [[[[1.0, 0.0]]], [[[0.0, 1.0]]], [[[2.0, 2.0]]]],
        "block_table": [[0, 1, 2]],
        "seq_lens": [3],
        "expected_part_out": [[[[[0.5, 0.5], [2.0, 2.0]]]]],
        "expected_part_lse": [[[[math.log(2.0), 0.0]]]],
        "expected_out": [[[[1.0, 1.0]]]],
        "expected_lse": [[[math.log(3.0)]]],
    },
    "causal_masked_split": {
        "description": "Causal prefill with fully masked splits: Sq = L = 4 one-token pages, S = 2, "
                       "q = 0. Rows 0 and 1 see no key of split 1, which must give (0, -inf) and "
                       "not NaN.",
        "citation": "Fully masked partitions contribute zero instead of NaN (-inf - (-inf) guard) "
                    "and a zero row sum stores 0 (scaleFinalOutput 0/0 guard); causal validity per "
                    "query row from its effective key length: rocMLIR 'Fix split-kv attention "
                    "masking and sweep RMS', Motivation and Technical Details.",
        "derivation": "Row i sees keys 0..i. P = ceil(4/2) = 2, split 0 = tokens 0,1, split 1 = "
                      "tokens 2,3. V rows v0=(1,0), v1=(0,1), v2=(2,2), v3=(4,0). Row 0: split0 "
                      "{0} -> (1,0), 0; split1 empty -> (0,0), -inf; combined (1,0), 0. Row 1: "
                      "split0 {0,1} -> (0.5,0.5), ln2; split1 empty; combined (0.5,0.5), ln2. "
                      "Row 2: split0 (0.5,0.5), ln2; split1 {2} -> (2,2), 0; combined (1,1), ln3. "
                      "Row 3: split0 (0.5,0.5), ln2; split1 {2,3} -> (3,1), ln2; combined "
                      "(7/4, 3/4), ln4.",
        "dtype": "f32", "page_size": 1, "num_q_heads": 1, "num_kv_heads": 1, "head_dim": 2,
        "scale": 1.0, "causal": True, "num_splits": 2,
        "q": [[[[0.0, 0.0]], [[0.0, 0.0]], [[0.0, 0.0]], [[0.0, 0.0]]]],
        "k_cache_pages": [[[[0.5, 0.5]]], [[[-1.0, 2.0]]], [[[0.25, 0.0]]], [[[3.0, -3.0]]]],
        "v_cache_pages": [[[[1.0, 0.0]]], [[[0.0, 1.0]]], [[[2.0, 2.0]]], [[[4.0, 0.0]]]],
        "block_table": [[0, 1, 2, 3]],
        "seq_lens": [4],
        "expected_part_out": [[[[[1.0, 0.0], [0.0, 0.0]]], [[[0.5, 0.5], [0.0, 0.0]]],
                               [[[0.5, 0.5], [2.0, 2.0]]], [[[0.5, 0.5], [3.0, 1.0]]]]],
        "expected_part_lse": [[[[0.0, NEG_INF]], [[math.log(2.0), NEG_INF]],
                               [[math.log(2.0), 0.0]], [[math.log(2.0), math.log(2.0)]]]],
        "expected_out": [[[[1.0, 0.0]], [[0.5, 0.5]], [[1.0, 1.0]], [[1.75, 0.75]]]],
        "expected_lse": [[[0.0], [math.log(2.0)], [math.log(3.0)], [math.log(4.0)]]],
    },
    "split_paged_closed_form": {
        "description": "Split-KV partition of multi-token pages: page size 4, two sequences of 10 "
                       "and 5 tokens (3 and 2 pages) in a 5-slot table whose unused slots hold an "
                       "unmapped id, S = 2 and S = 4, q = 0 so every valid score is 0 and each "
                       "split's output is the mean of its V rows. Tokens past a sequence's length "
                       "in its last page hold 1000 so that reading them changes the answer.",
        "citation": "Split ranges: the iterations (pages) of one sequence are ceil-divided among "
                    "the splits and each split's end is clamped to the sequence's own iteration "
                    "count, so trailing splits may be empty: rocMLIR 'Fix split-kv attention "
                    "masking and sweep RMS', Technical Details (non-causal split-KV iteration "
                    "math) and Test Coverage (split-KV lowering and per-row mask tests). Tokens "
                    "past the length are ignored and slots past a sequence's pages are never read: "
                    "rocm-libraries 'one K/V resource per page on the gfx942 2D i64 path', Coverage.",
        "derivation": "Sequence 0: L = 10, n = ceil(10/4) = 3 pages, V row of logical token t is "
                      "(t, t^2). Sequence 1: L = 5, n = 2, V row (20 + t, 1). "
                      "S = 2: sequence 0 has P = ceil(3/2) = 2 pages per split: split 0 = tokens "
                      "0..7, mean (3.5, 140/8 = 17.5), lse ln 8; split 1 = page 2 clamped to L = "
                      "tokens 8, 9, mean (8.5, (64+81)/2 = 72.5), lse ln 2. Sequence 1 has P = "
                      "ceil(2/2) = 1: split 0 = tokens 0..3, (21.5, 1), ln 4; split 1 = token 4, "
                      "(24, 1), ln 1 = 0. "
                      "S = 4: sequence 0, P = 1: tokens 0..3 (1.5, 14/4 = 3.5) ln 4; tokens 4..7 "
                      "(5.5, 126/4 = 31.5) ln 4; tokens 8, 9 (8.5, 72.5) ln 2; split 3 empty "
                      "(0, 0), -inf. Sequence 1, P = 1: (21.5, 1) ln 4; (24, 1) 0; splits 2 and 3 "
                      "empty. "
                      "Unsplit: sequence 0 mean of tokens 0..9 (4.5, 285/10 = 28.5), lse ln 10; "
                      "sequence 1 (22, 1), ln 5. "
                      "Splitting by ceil(L/S) tokens instead (S = 2: 5 tokens each) would give "
                      "ln 5 twice; sizing splits by the table width (P = ceil(5/2) = 3) would put "
                      "all of sequence 0 in split 0.",
        "dtype": "f32", "page_size": 4, "num_q_heads": 1, "num_kv_heads": 1, "head_dim": 2,
        "scale": 1.0, "causal": False,
        "q": [[[[0.0, 0.0]]], [[[0.0, 0.0]]]],
        # physical page p holds [4 tokens][1 kv head][2 dims]; sequence 0 uses pages 2, 0, 4
        # (tokens 0-3, 4-7, 8-11 with 10 and 11 past L), sequence 1 uses pages 1, 3
        # (tokens 0-3, 4-7 with 5-7 past L)
        "k_cache_pages": [
            [[[0.5, -1.0]], [[2.0, 0.25]], [[-3.0, 1.0]], [[0.0, 4.0]]],
            [[[1.0, 1.0]], [[-2.0, 0.5]], [[0.75, -0.5]], [[3.0, 3.0]]],
            [[[-1.0, 2.0]], [[0.125, 0.0]], [[5.0, -5.0]], [[-0.25, 1.5]]],
            [[[2.5, -2.5]], [[1000.0, 1000.0]], [[1000.0, 1000.0]], [[1000.0, 1000.0]]],
            [[[-0.5, 0.5]], [[1.5, -1.5]], [[1000.0, 1000.0]], [[1000.0, 1000.0]]],
        ],
        "v_cache_pages": [
            [[[4.0, 16.0]], [[5.0, 25.0]], [[6.0, 36.0]], [[7.0, 49.0]]],
            [[[20.0, 1.0]], [[21.0, 1.0]], [[22.0, 1.0]], [[23.0, 1.0]]],
            [[[0.0, 0.0]], [[1.0, 1.0]], [[2.0, 4.0]], [[3.0, 9.0]]],
            [[[24.0, 1.0]], [[1000.0, 1000.0]], [[1000.0, 1000.0]], [[1000.0, 1000.0]]],
            [[[8.0, 64.0]], [[9.0, 81.0]], [[1000.0, 1000.0]], [[1000.0, 1000.0]]],
        ],
        "block_table": [[2, 0, 4, UNMAPPED, UNMAPPED], [1, 3, UNMAPPED, UNMAPPED, UNMAPPED]],
        "seq_lens": [10, 5],
        "splits": {
            "2": {
                "expected_part_out": [[[[[3.5, 17.5], [8.5, 72.5]]]],
                                      [[[[21.5, 1.0], [24.0, 1.0]]]]],
                "expected_part_lse": [[[[math.log(8.0), math.log(2.0)]]],
                                      [[[math.log(4.0), 0.0]]]],
            },
            "4": {
                "expected_part_out": [[[[[1.5, 3.5], [5.5, 31.5], [8.5, 72.5], [0.0, 0.0]]]],
                                      [[[[21.5, 1.0], [24.0, 1.0], [0.0, 0.0], [0.0, 0.0]]]]],
                "expected_part_lse": [[[[math.log(4.0), math.log(4.0), math.log(2.0), NEG_INF]]],
                                      [[[math.log(4.0), 0.0, NEG_INF, NEG_INF]]]],
            },
        },
        "expected_out": [[[[4.5, 28.5]]], [[[22.0, 1.0]]]],
        "expected_lse": [[[math.log(10.0)]], [[math.log(5.0)]]],
    },
    "split_paged_causal": {
        "description": "Causal prefill over multi-token pages with split-KV: page size 2, Sq = L = 5 "
                       "(3 pages) in a 4-slot table with an unmapped tail, S = 2 and S = 3, q = 0. "
                       "Early rows see nothing of the later splits, which must give (0, -inf).",
        "citation": "Ceil-divided, clamped split ranges (rocMLIR 'Fix split-kv attention masking and "
                    "sweep RMS', Technical Details) and per-row causal validity from the row's "
                    "effective key length, with fully masked partitions contributing zero (same "
                    "page, Technical Details and the host reference's causal valid-split masking).",
        "derivation": "V row of logical token t is (t, 1); row i sees keys 0..i. S = 2: P = "
                      "ceil(3/2) = 2 pages, split 0 = tokens 0..3, split 1 = token 4 (token 5 of "
                      "the last page is past L). Row i < 4: split 0 = mean of 0..i = (i/2, 1), "
                      "lse ln(i+1); split 1 empty (0, 0), -inf. Row 4: split 0 (1.5, 1) ln 4; "
                      "split 1 (4, 1) ln 1 = 0. S = 3: P = 1, splits = tokens {0,1}, {2,3}, {4}. "
                      "Row 0: (0,1) 0; empty; empty. Row 1: (0.5,1) ln 2; empty; empty. Row 2: "
                      "(0.5,1) ln 2; (2,1) 0; empty. Row 3: (0.5,1) ln 2; (2.5,1) ln 2; empty. "
                      "Row 4: (0.5,1) ln 2; (2.5,1) ln 2; (4,1) 0. Combined row i: (i/2, 1), "
                      "lse ln(i+1). Splitting by ceil(L/S) tokens (S = 2: 3 tokens) would give "
                      "row 3 a split 1 of token 3.",
        "dtype": "f32", "page_size": 2, "num_q_heads": 1, "num_kv_heads": 1, "head_dim": 2,
        "scale": 1.0, "causal": True,
        "q": [[[[0.0, 0.0]], [[0.0, 0.0]], [[0.0, 0.0]], [[0.0, 0.0]], [[0.0, 0.0]]]],
        # the table is [1, 2, 0, unmapped]: page 1 holds tokens 0-1, page 2 tokens 2-3,
        # page 0 token 4 and (past L) token 5
        "k_cache_pages": [
            [[[0.5, 0.5]], [[1000.0, 1000.0]]],
            [[[-1.0, 2.0]], [[3.0, -3.0]]],
            [[[0.25, 0.0]], [[2.0, 1.0]]],
        ],
        "v_cache_pages": [
            [[[4.0, 1.0]], [[1000.0, 1000.0]]],
            [[[0.0, 1.0]], [[1.0, 1.0]]],
            [[[2.0, 1.0]], [[3.0, 1.0]]],
        ],
        "block_table": [[1, 2, 0, UNMAPPED]],
        "seq_lens": [5],
        "splits": {
            "2": {
                "expected_part_out": [[[[[0.0, 1.0], [0.0, 0.0]]], [[[0.5, 1.0], [0.0, 0.0]]],
                                       [[[1.0, 1.0], [0.0, 0.0]]], [[[1.5, 1.0], [0.0, 0.0]]],
                                       [[[1.5, 1.0], [4.0, 1.0]]]]],
                "expected_part_lse": [[[[0.0, NEG_INF]], [[math.log(2.0), NEG_INF]],
                                       [[math.log(3.0), NEG_INF]], [[math.log(4.0), NEG_INF]],
                                       [[math.log(4.0), 0.0]]]],
            },
            "3": {
                "expected_part_out": [[[[[0.0, 1.0], [0.0, 0.0], [0.0, 0.0]]],
                                       [[[0.5, 1.0], [0.0, 0.0], [0.0, 0.0]]],
                                       [[[0.5, 1.0], [2.0, 1.0], [0.0, 0.0]]],
                                       [[[0.5, 1.0], [2.5, 1.0], [0.0, 0.0]]],
                                       [[[0.5, 1.0], [2.5, 1.0], [4.0, 1.0]]]]],
                "expected_part_lse": [[[[0.0, NEG_INF, NEG_INF]],
                                       [[math.log(2.0), NEG_INF, NEG_INF]],
                                       [[math.log(2.0), 0.0, NEG_INF]],
                                       [[math.log(2.0), math.log(2.0), NEG_INF]],
                                       [[math.log(2.0), math.log(2.0), 0.0]]]],
            },
        },
        "expected_out": [[[[0.0, 1.0]], [[0.5, 1.0]], [[1.0, 1.0]], [[1.5, 1.0]], [[2.0, 1.0]]]],
        "expected_lse": [[[0.0], [math.log(2.0)], [math.log(3.0)], [math.log(4.0)],
                          [math.log(5.0)]]],
    },
    "quantized_hand_case": {
        "description": "The hand case above with K and V stored as 8-bit codes and one scale per "
                       "(page, kv head), once as int8 and once as fp8 E4M3. Scales differ between "
                       "K and V and between pages (one is 0, one negative) so that a scale taken "
                       "from the wrong cache, page or slot changes the answer.",
        "citation": "int8 paged attention (rocMLIR 'Paged Attention: rocmlir-gen changes', file "
                    "list: the int8 e2e test) and i8 split-KV attention (rocMLIR 'Fix split-kv "
                    "attention masking and sweep RMS', Motivation); fp8 K/V loaders (rocm-libraries "
                    "'one K/V resource per page on the gfx942 2D i64 path', review). Scale "
                    "granularity and the fp8 format are the reading taken here.",
        "derivation": "Physical page 0 holds token 1, page 1 holds token 0. int8: k1 = ln3 * (1, 0), "
                      "k0 = 0 * (5, -3) = (0, 0), v1 = 0.25 * (0, 4) = (0, 1), v0 = -0.5 * (-2, 0) = "
                      "(1, 0). fp8 (0x38 = 1, 0x50 = 8, 0xC4 = -3, 0x80 = -0, 0x48 = 4, 0xB0 = -0.5): "
                      "k1 = ln3 * (1, 0), k0 = 0 * (8, -3), v1 = 0.25 * (-0, 4) = (-0, 1), "
                      "v0 = -2 * (-0.5, 0) = (1, 0). Both give the hand case: out (0.25, 0.75), "
                      "lse ln 4.",
        "page_size": 1, "num_q_heads": 1, "num_kv_heads": 1, "head_dim": 2,
        "scale": 1.0, "causal": False,
        "q": [[[[1.0, 0.0]]]],
        "block_table": [[1, 0]],
        "seq_lens": [2],
        "variants": {
            "int8": {
                "k_codes": [[[[1, 0]]], [[[5, 0xFD]]]],
                "v_codes": [[[[0, 4]]], [[[0xFE, 0]]]],
                "k_scales": [[math.log(3.0)], [0.0]],
                "v_scales": [[0.25], [-0.5]],
            },
            "fp8_e4m3": {
                "k_codes": [[[[0x38, 0x00]]], [[[0x50, 0xC4]]]],
                "v_codes": [[[[0x80, 0x48]]], [[[0xB0, 0x00]]]],
                "k_scales": [[math.log(3.0)], [0.0]],
                "v_scales": [[0.25], [-2.0]],
            },
        },
        "expected_out": [[[[0.25, 0.75]]]],
        "expected_lse": [[[math.log(4.0)]]],
    },
}


def main():
    for name, obj in FIXTURES.items():
        with open(os.path.join(HERE, name + ".json"), "w") as f:
            json.dump(obj, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main()
