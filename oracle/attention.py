"""Oracle: explicit-mask dense softmax attention in float64 (test infrastructure only).

Candidate isolation attention mask page:
  * section "段 ID：掩码的表达方式" gives who may read whom, in terms of segment IDs:
    a query that is not padding reads every history key (segment 1) of its user, and a
    candidate query reads, besides those, its own row and no other candidate;
  * section "掩码长什么样" prints that rule as a table for P=1, H=3, C=3;
  * section "只更新候选的末尾层" describes candidate-only layers and their fallback
    (run the full layer, keep the candidate rows).
No position reads another user's rows (HSTU scaling notes, section
"手算 padding 的浪费与 offset"), so the mask is built per user and never across
users.

Readings: softmax attention, scale 1/sqrt(d) unless given; rows that admit no
key output 0.
"""
from __future__ import annotations

import math

import numpy as np

from .jagged import segment_ids

DEFAULT_SCALE = None   # None or <= 0 means 1/sqrt(d)


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if (scale is None or scale <= 0) else float(scale)


def isolation_mask_rows(seg, rows) -> np.ndarray:
    """Rows ``rows`` (local positions) of one user's [L, L] visibility mask from its segment IDs:
    every non-padding query row reads the user's history columns; a candidate row also reads
    its own column."""
    seg = np.asarray(seg)
    rows = np.asarray(rows, dtype=np.int64)
    role = seg[rows]
    visible = np.outer(role != 0, seg == 1)
    own = np.nonzero(role == -1)[0]
    visible[own, rows[own]] = True
    return visible


def isolation_mask(seg) -> np.ndarray:
    """One user's full [L, L] visibility mask (query rows x key columns)."""
    return isolation_mask_rows(seg, np.arange(len(seg)))


def masked_softmax_attention(q, k, v, mask, scale) -> np.ndarray:
    """softmax(scale * q k^T, masked to -inf where ``mask`` is False) v, in float64.

    q [Lq, d], k and v [Lk, d], mask [Lq, Lk].  A row with no admitted key gives 0."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    has_key = mask.any(axis=1)
    if not has_key.any():
        return out
    s = scale * (q[has_key] @ k.T)
    s = np.where(mask[has_key], s, -np.inf)
    s_max = s.max(axis=1, keepdims=True)
    e = np.exp(s - s_max)
    p = e / e.sum(axis=1, keepdims=True)
    out[has_key] = p @ v
    return out


def full_attention(q, k, v, offsets, cand_start, valid=None, attend_padded_history=False,
                   scale=DEFAULT_SCALE) -> np.ndarray:
    """Full-sequence mode over a jagged batch.  q, k, v [T, H, d]; returns float64 [T, H, d]."""
    q = np.asarray(q)
    T, H, d = q.shape
    sc = _scale(scale, d)
    offsets = np.asarray(offsets, dtype=np.int64)
    seg = segment_ids(offsets, cand_start, valid, attend_padded_history)
    out = np.zeros((T, H, d), dtype=np.float64)
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        if hi == lo:
            continue
        mask = isolation_mask(seg[lo:hi])
        for h in range(H):
            out[lo:hi, h] = masked_softmax_attention(q[lo:hi, h], k[lo:hi, h], v[lo:hi, h], mask, sc)
    return out


def full_attention_rows(q, k, v, offsets, cand_start, rows, heads, valid=None,
                        attend_padded_history=False, scale=DEFAULT_SCALE, seg=None) -> np.ndarray:
    """The same result as ``full_attention`` for the sampled (row, head) pairs only.

    Each sample's mask row is built from its own user's segment IDs; returns float64 [n, d]."""
    q = np.asarray(q)
    T, H, d = q.shape
    sc = _scale(scale, d)
    offsets = np.asarray(offsets, dtype=np.int64)
    if seg is None:
        seg = segment_ids(offsets, cand_start, valid, attend_padded_history)
    rows = np.asarray(rows, dtype=np.int64)
    heads = np.asarray(heads, dtype=np.int64)
    users = np.searchsorted(offsets, rows, side="right") - 1
    out = np.zeros((len(rows), d), dtype=np.float64)
    for b in np.unique(users):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        sel_b = np.nonzero(users == b)[0]
        for h in np.unique(heads[sel_b]):
            sel = sel_b[heads[sel_b] == h]
            mask = isolation_mask_rows(seg[lo:hi], rows[sel] - lo)
            out[sel] = masked_softmax_attention(q[rows[sel], h], k[lo:hi, h], v[lo:hi, h], mask, sc)
    return out


def _cand_only_user(q_c, k_h, v_h, k_c, v_c, rows_c, sc):
    """One user and head of a candidate-only layer, as the fallback: the full layer over
    [frozen history | candidates] with the candidate rows kept (history queries are never
    kept, so they are not formed)."""
    h_b, c_b = k_h.shape[0], k_c.shape[0]
    seg = np.array([1] * h_b + [-1] * c_b, dtype=np.int8)
    keys = np.concatenate([k_h, k_c], axis=0)
    vals = np.concatenate([v_h, v_c], axis=0)
    mask = isolation_mask_rows(seg, h_b + np.asarray(rows_c, dtype=np.int64))
    return masked_softmax_attention(q_c, keys, vals, mask, sc)


def cand_only_attention(q_cand, k_hist, v_hist, k_cand, v_cand, hist_offsets, cand_offsets,
                        scale=DEFAULT_SCALE) -> np.ndarray:
    """Candidate-only layer: candidate queries attend the user's frozen history K/V and their
    own K/V.  Returns float64 [Tc, H, d]."""
    q_cand = np.asarray(q_cand)
    Tc, H, d = q_cand.shape
    sc = _scale(scale, d)
    hoff = np.asarray(hist_offsets, dtype=np.int64)
    coff = np.asarray(cand_offsets, dtype=np.int64)
    out = np.zeros((Tc, H, d), dtype=np.float64)
    for b in range(len(coff) - 1):
        hl, hh, cl, ch = int(hoff[b]), int(hoff[b + 1]), int(coff[b]), int(coff[b + 1])
        if ch == cl:
            continue
        for h in range(H):
            out[cl:ch, h] = _cand_only_user(q_cand[cl:ch, h], k_hist[hl:hh, h], v_hist[hl:hh, h],
                                            k_cand[cl:ch, h], v_cand[cl:ch, h], np.arange(ch - cl), sc)
    return out


def cand_only_attention_rows(q_cand, k_hist, v_hist, k_cand, v_cand, hist_offsets, cand_offsets,
                             rows, heads, scale=DEFAULT_SCALE) -> np.ndarray:
    """``cand_only_attention`` for sampled (candidate row, head) pairs; float64 [n, d]."""
    q_cand = np.asarray(q_cand)
    Tc, H, d = q_cand.shape
    sc = _scale(scale, d)
    hoff = np.asarray(hist_offsets, dtype=np.int64)
    coff = np.asarray(cand_offsets, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    heads = np.asarray(heads, dtype=np.int64)
    users = np.searchsorted(coff, rows, side="right") - 1
    out = np.zeros((len(rows), d), dtype=np.float64)
    for b in np.unique(users):
        hl, hh, cl, ch = int(hoff[b]), int(hoff[b + 1]), int(coff[b]), int(coff[b + 1])
        sel_b = np.nonzero(users == b)[0]
        for h in np.unique(heads[sel_b]):
            sel = sel_b[heads[sel_b] == h]
            out[sel] = _cand_only_user(q_cand[rows[sel], h], k_hist[hl:hh, h], v_hist[hl:hh, h],
                                       k_cand[cl:ch, h], v_cand[cl:ch, h], rows[sel] - cl, sc)
    return out
