"""Writes tile_pruning_cases.json: hand-derived cases of the tile-pruning rule.

Source: TIGA-lang "基于 tile 剪枝的稀疏注意力" (tile-pruned sparse attention).
Its first section works one example: the highest score seen is 10, the next
tile's highest is 1, their weight ratio is exp(1 - 10), about 0.00012, and
with block_prune_threshold = 0.01 that tile is skipped.  Its rule section
admits a key tile iff its maximum score over the whole (query block, key tile)
reaches the query block's running maximum plus ln(rho).  Each case below
builds scores that are exact small numbers (dot products of one-hot or
integer vectors, scale 1), states the admitted tiles the rule gives, and the
softmax over the admitted keys in closed form.  Pure arithmetic; no oracle or
GPU code is called.
"""
import json
import math
import os

E = math.exp


def col(x):
    return [[float(a)] for a in x]


def case(name, q, k, v, rho, br, bc, admit, o, m, l, derivation):
    return {"name": name, "scale": 1.0, "rho": rho, "br": br, "bc": bc,
            "q": [q], "k": [k], "v": [v], "admit": [admit], "o": [o], "m": [m], "l": [l],
            "derivation": derivation}


CASES = []
# The page's example: tile 0 holds the best score 10, tile 1 tops out at 1.
q2 = col([1, 1])
k_ex = col([10, 8, 1, 0])
v_ex = col([1, 2, 3, 4])
o_skip = (1 + 2 * E(-2)) / (1 + E(-2))
CASES.append(case("page_example_rho_0.01_skips", q2, k_ex, v_ex, 0.01, 2, 2, [[1, 0]],
                  [[o_skip], [o_skip]], [10.0, 10.0], [1 + E(-2)] * 2,
                  "tile 1: 1 >= 10 + ln 0.01 = 5.39 fails -> skipped; rows see keys (10, 8): "
                  "o = (1 + 2 e^-2) / (1 + e^-2), m = 10, l = 1 + e^-2"))
l_all = 1 + E(-2) + E(-9) + E(-10)
o_all = (1 + 2 * E(-2) + 3 * E(-9) + 4 * E(-10)) / l_all
CASES.append(case("page_example_rho_1e-4_admits", q2, k_ex, v_ex, 1e-4, 2, 2, [[1, 1]],
                  [[o_all], [o_all]], [10.0, 10.0], [l_all] * 2,
                  "tile 1: 1 >= 10 + ln 1e-4 = 0.79 holds -> admitted; all four keys"))
# exp(1 - 10) = 1.234e-4 is the page's ratio: rho just above it skips, just below admits.
CASES.append(case("ratio_boundary_rho_1.3e-4_skips", q2, k_ex, v_ex, 1.3e-4, 2, 2, [[1, 0]],
                  [[o_skip], [o_skip]], [10.0, 10.0], [1 + E(-2)] * 2,
                  "exp(1 - 10) = 1.234e-4 < 1.3e-4 -> skipped"))
CASES.append(case("ratio_boundary_rho_1.1e-4_admits", q2, k_ex, v_ex, 1.1e-4, 2, 2, [[1, 1]],
                  [[o_all], [o_all]], [10.0, 10.0], [l_all] * 2,
                  "exp(1 - 10) = 1.234e-4 >= 1.1e-4 -> admitted"))
# The decision is per query block: row 1's own scores are low, but the block's
# running maximum (row 0's 10) decides for both rows.
qb = [[1.0, 0.0], [0.0, 1.0]]
vb = [[1.0, 10.0], [2.0, 20.0], [3.0, 30.0], [4.0, 40.0]]
w = [1.0, E(-1)]
ob = [sum(w[i] * vb[i][d] for i in range(2)) / sum(w) for d in range(2)]
CASES.append(case("block_rule_skips_for_every_row", qb, [[10, 0], [9, -1], [-5, 1], [-6, 0.5]], vb,
                  0.01, 2, 2, [[1, 0]], [ob, ob], [10.0, 0.0], [1 + E(-1)] * 2,
                  "block maximum after tile 0 is 10; tile 1 maximum 1 < 5.39 -> skipped for both "
                  "rows (row 1 alone would admit it); rows see keys 0, 1 with weights 1 : e^-1"))
w0 = [1.0, E(-1), E(-15), E(-16)]
w1 = [E(-7), E(-8), 1.0, E(-6.5)]
o0 = [sum(w0[i] * vb[i][d] for i in range(4)) / sum(w0) for d in range(2)]
o1 = [sum(w1[i] * vb[i][d] for i in range(4)) / sum(w1) for d in range(2)]
CASES.append(case("block_rule_admits_through_another_row", qb, [[10, 0], [9, -1], [-5, 7], [-6, 0.5]],
                  vb, 0.01, 2, 2, [[1, 1]], [o0, o1], [10.0, 7.0], [sum(w0), sum(w1)],
                  "tile 1 maximum is row 1's 7 >= 5.39 -> admitted for both rows (row 0's own "
                  "tile-1 scores are -5, -6)"))
# rho = 1: admitted iff the tile reaches the running maximum; a tie is admitted (>=).
CASES.append(case("rho_1_tie_admitted", col([1]), col([3, 3, 2.5]), col([1, 2, 4]), 1.0, 1, 1,
                  [[1, 1, 0]], [[1.5]], [3.0], [2.0],
                  "tiles of one key: 3 (admit), 3 >= 3 (admit), 2.5 < 3 (skip); o = (1 + 2)/2"))
# A ragged last tile: keys 0..4 with tiles {0,1}, {2,3}, {4}.
l_r = 1 + E(-10) + E(-1)
CASES.append(case("ragged_tiles", col([1]), col([10, 0, 0, 0, 9]), col([1, 2, 3, 4, 5]), 0.01, 1, 2,
                  [[1, 0, 1]], [[(1 + 2 * E(-10) + 5 * E(-1)) / l_r]], [10.0], [l_r],
                  "tile {0,1} max 10 admit; {2,3} max 0 < 5.39 skip; {4} max 9 >= 5.39 admit; "
                  "key 1 counts (its tile is admitted) although its score is 0"))

OUT = {
    "_citation": (
        "TIGA-lang '基于 tile 剪枝的稀疏注意力' (tile-pruned sparse attention): the worked "
        "example of its first section (best score 10, next tile best 1, exp(1 - 10) ~ 0.00012, "
        "skipped at block_prune_threshold = 0.01) and the admission inequality of its rule "
        "section (m_tile >= m_run,block + ln rho). Expected values are closed forms of the "
        "softmax over the admitted keys; generated by tests/golden/make_pruning_cases.py "
        "(pure arithmetic, no oracle call)."),
    "page_ratio": {"expression": "exp(1 - 10)", "printed": 0.00012, "value": E(1 - 10)},
    "cases": CASES,
}

if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tile_pruning_cases.json")
    with open(path, "w") as f:
        json.dump(OUT, f, indent=1)
    print("wrote", path)
