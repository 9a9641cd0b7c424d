"""Host accounting against the pages' worked numbers (CPU only)."""
import json
import os

import numpy as np

from jagged_candidate_isolated_amd import accounting as acc

G = os.path.join(os.path.dirname(__file__), "golden", "accounting.json")


def test_pair_work_example():
    g = json.load(open(G, encoding="utf-8"))["pair_work"]
    L = g["lengths"]
    assert acc.padded_positions(L) == g["padded_positions"]
    assert acc.ragged_positions(L) == g["ragged_positions"]
    assert round(acc.pair_work_ratio(L), 3) == g["pair_work_ratio_3dp"]


def test_four_d_flops_per_pair_convention():
    g = json.load(open(G, encoding="utf-8"))["transretrieval_flops"]
    f = acc.per_candidate_flops_transretrieval(g["D"], g["L_t"], g["L_u"], g["n_layer"])
    assert abs(f / 1e6 - g["reported_mflops"]) / g["reported_mflops"] <= g["relative_tolerance"]
    # its attention term is 4*D per (query, key) pair: L_t queries x L_u keys per layer
    attn = 4 * g["D"] * g["L_t"] * g["L_u"] * g["n_layer"]
    assert attn == acc.attention_flops(g["L_t"] * g["L_u"] * g["n_layer"], H=1, d=g["D"])


def test_isolation_pairs_match_mask_count():
    """Pairs counted by formula equal the admitted entries of the explicit oracle mask."""
    from oracle import attention as A
    from oracle import jagged as J
    rng = np.random.default_rng(3)
    for _ in range(20):
        B = int(rng.integers(1, 5))
        P = rng.integers(0, 3, B); h = rng.integers(0, 6, B); c = rng.integers(0, 5, B)
        lens = P + h + c
        offs = J.offsets_from_lengths(lens)
        cs = offs[:-1] + P + h
        seg = J.segment_ids(offs, cs)
        admitted = sum(int(A.isolation_mask(seg[offs[b]:offs[b + 1]]).sum()) for b in range(B))
        assert admitted == acc.isolation_pairs(P + h, c)


def test_tile_pairs_brute_force():
    """Tile-padded pair count against enumeration of every (tile row, tile column) pair."""
    rng = np.random.default_rng(4)
    for _ in range(30):
        B = int(rng.integers(1, 5))
        n_q = rng.integers(0, 300, B)
        n_kv = rng.integers(0, 200, B)
        bm, bn = int(rng.choice([32, 128, 256])), int(rng.choice([32, 64, 128]))
        want = 0
        for q, k in zip(n_q, n_kv):
            rows = sum(bm for t in range(0, int(q), bm))
            cols = sum(bn for t in range(0, int(k), bn))
            want += rows * cols
        assert acc.tile_pairs(n_q, n_kv, bm, bn) == want
    # exact tiles waste nothing; one row or key over a tile costs a whole tile
    assert acc.tile_pairs([256], [128], 128, 64) == 256 * 128
    assert acc.tile_pairs([257], [129], 128, 64) == 384 * 192
    assert acc.tile_pairs([0, 5], [7, 0], 128, 64) == 0
