"""Work and traffic accounting for jagged candidate-isolated attention (host logic).

Conventions:
  * Pair work.  HSTU scaling notes, section "不同长度不是边角问题": a batch of
    lengths n_i padded to the longest costs B * max(n)^2 dense pairs, while
    per-sequence (ragged) execution costs sum(n_i^2).
  * FLOPs per admitted (query, key) pair.  TransRetrieval review, section
    "改动二" (the per-request FLOP formula 4D * N_target * L_t * (4D + L_u) *
    N_layer): its attention term is 4 * D * L_t * L_u per layer, i.e. 4*D FLOPs
    per pair -- 2*D for the score and 2*D for the weighted value sum.  With H
    heads of width d, D = H * d.
  * Admitted pairs under candidate isolation (Candidate isolation attention
    mask page, section "段 ID：掩码的表达方式"): every valid query of user b reads the
    user's n_b segment-1 rows; a candidate also reads itself.  So a user costs
    n_b^2 + c_b * (n_b + 1) pairs, where n_b counts segment-1 rows and c_b valid
    candidates.  "Effective" counts real (non-pad) rows only; "executed" also
    counts padding rows admitted with attend_padded_history.
  * Algorithmic bytes: q, k, v read once and o written once.
"""
from __future__ import annotations

import numpy as np


def padded_positions(lengths) -> int:
    lengths = [int(n) for n in lengths]
    return len(lengths) * max(lengths) if lengths else 0


def ragged_positions(lengths) -> int:
    return int(sum(int(n) for n in lengths))


def pair_work_ratio(lengths) -> float:
    """Dense padded pair work over per-sequence pair work."""
    lengths = [int(n) for n in lengths]
    return len(lengths) * max(lengths) ** 2 / sum(n * n for n in lengths)


def per_candidate_flops_transretrieval(D: int, L_t: int, L_u: int, n_layer: int) -> int:
    """Per-candidate FLOPs of the TransRetrieval formula with N_target = 1."""
    return 4 * D * L_t * (4 * D + L_u) * n_layer


def isolation_pairs(n_hist, n_cand) -> int:
    """sum_b n_b^2 + c_b (n_b + 1) admitted pairs per head."""
    n = np.asarray(n_hist, dtype=np.int64)
    c = np.asarray(n_cand, dtype=np.int64)
    return int(np.sum(n * n + c * (n + 1)))


def attention_flops(pairs: int, H: int, d: int) -> int:
    return 4 * d * H * int(pairs)


def full_mode_counts(prefix, hist, cand, pad, attend_padded_history: bool):
    """(effective pairs, executed pairs) per head of a ``[prefix | pad | history | cand]`` batch."""
    n_real = np.asarray(prefix, np.int64) + np.asarray(hist, np.int64)
    n_exec = n_real + (np.asarray(pad, np.int64) if attend_padded_history else 0)
    return isolation_pairs(n_real, cand), isolation_pairs(n_exec, cand)


def full_mode_bytes(T: int, H: int, d: int, elem_bytes: int) -> int:
    return 4 * T * H * d * elem_bytes


def cand_only_pairs(hist, cand) -> int:
    """Candidate-only layer: each candidate reads its user's h_b frozen rows and itself."""
    h = np.asarray(hist, np.int64)
    c = np.asarray(cand, np.int64)
    return int(np.sum(c * (h + 1)))


def cand_only_bytes(Th: int, Tc: int, H: int, d: int, elem_bytes: int) -> int:
    return (2 * Th + 4 * Tc) * H * d * elem_bytes


def tile_pairs(n_q, n_kv, bm: int, bn: int) -> int:
    """(query, key) pairs the matrix cores execute per head when each user's n_q query rows
    go in tiles of bm rows and each tile loops over the user's n_kv keys in blocks of bn
    columns: the last query tile and the last key block run whole.  Users without queries
    or without keys run no key block."""
    q = np.asarray(n_q, np.int64)
    k = np.asarray(n_kv, np.int64)
    return int(np.sum(-(-q // bm) * bm * (-(-k // bn) * bn)))
