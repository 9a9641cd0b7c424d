"""Oracle: gradients of the candidate-isolated attention in float64 (test infrastructure only).

The pages train with this mask too (Candidate isolation attention mask page, section
"训练时的序列打包": sequence packing keeps the same attention contract), but they
print no backward formulas.  The gradients here are those of the forward oracle's
definition -- per user and head, P = softmax(scale * q k^T masked by the explicit
[L, L] isolation mask), O = P v -- taken with the textbook softmax derivative:

    dV = P^T dO
    dP = dO v^T
    dS = P * (dP - rowsum(dP * P))          (elementwise; masked entries have P = 0)
    dq = scale * dS k,   dk = scale * dS^T q

Rows that admit no key (segment 0) have P = 0: they get no gradient and give none.
A candidate-only layer's gradients are those of its fallback (the full layer over
[frozen history | candidates], keeping the candidate rows): the same formulas with a
zero output gradient on the history rows.
``attention_lse`` gives each row's log-sum-exp of its admitted scaled scores (natural
log), the statistic a backward pass reuses from the forward; -inf for such rows.

``gradient_error_scale`` is not a result of the method: it is the magnitude that
rounding-error analysis attaches to each gradient element when P and dS are rounded
to a narrow format before their products and o is stored in that format, so that a
test can bound a low-precision implementation's error (|err| <= c u (E + |grad|) for
unit roundoff u).
"""
from __future__ import annotations

import numpy as np

from .attention import _scale, isolation_mask
from .jagged import segment_ids


def _user_head_backward(q, k, v, do, mask, sc):
    """One user and head: returns dq, dk, dv (float64) for the [L, L] ``mask``."""
    s = sc * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    has = mask.any(axis=1)
    p = np.zeros_like(s)
    if has.any():
        m = s[has].max(axis=1, keepdims=True)
        e = np.where(mask[has], np.exp(s[has] - m), 0.0)
        p[has] = e / e.sum(axis=1, keepdims=True)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
    return sc * (ds @ k), sc * (ds.T @ q), dv


def full_attention_backward(q, k, v, do, offsets, cand_start, valid=None, attend_padded_history=False,
                            scale=None):
    """Gradients (dq, dk, dv) of full-sequence attention w.r.t. q, k, v for output gradient
    ``do``; all [T, H, d] float64."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); do = np.asarray(do, np.float64)
    T, H, d = q.shape
    sc = _scale(scale, d)
    offsets = np.asarray(offsets, dtype=np.int64)
    seg = segment_ids(offsets, cand_start, valid, attend_padded_history)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        if hi == lo:
            continue
        mask = isolation_mask(seg[lo:hi])
        for h in range(H):
            dq[lo:hi, h], dk[lo:hi, h], dv[lo:hi, h] = _user_head_backward(
                q[lo:hi, h], k[lo:hi, h], v[lo:hi, h], do[lo:hi, h], mask, sc)
    return dq, dk, dv


def attention_lse(q, k, offsets, cand_start, valid=None, attend_padded_history=False, scale=None):
    """Per (row, head) natural-log sum of exp(scale * q.k) over the row's admitted keys;
    float64 [T, H], -inf for rows that admit none."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    T, H, d = q.shape
    sc = _scale(scale, d)
    offsets = np.asarray(offsets, dtype=np.int64)
    seg = segment_ids(offsets, cand_start, valid, attend_padded_history)
    out = np.full((T, H), -np.inf)
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        if hi == lo:
            continue
        mask = isolation_mask(seg[lo:hi])
        has = mask.any(axis=1)
        for h in range(H):
            s = np.where(mask, sc * (q[lo:hi, h] @ k[lo:hi, h].T), -np.inf)[has]
            m = s.max(axis=1)
            out[lo:hi, h][has] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return out


def _user_head_error_scale(q, k, v, do, mask, sc):
    """One user and head: the error scales (Eq, Ek, Ev) of ``gradient_error_scale``."""
    s = np.where(mask, sc * (q @ k.T), -np.inf)
    has = mask.any(axis=1)
    p = np.zeros_like(s)
    if has.any():
        m = s[has].max(axis=1, keepdims=True)
        e = np.where(mask[has], np.exp(s[has] - m), 0.0)
        p[has] = e / e.sum(axis=1, keepdims=True)
    dp = do @ v.T
    ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
    # rowsum(dO * o) taken from a rounded o: o's own bound is u (|o| + P|v|) <= 2u P|v|
    dsum = 2.0 * (np.abs(do) * (p @ np.abs(v))).sum(axis=1, keepdims=True)
    aq, ak = np.abs(q), np.abs(k)
    eq = sc * (np.abs(ds) @ ak + dsum * (p @ ak))
    ek = sc * (np.abs(ds).T @ aq + p.T @ (dsum * aq))
    ev = p.T @ np.abs(do)
    return eq, ek, ev


def gradient_error_scale(q, k, v, do, offsets, cand_start, valid=None, attend_padded_history=False,
                         scale=None):
    """Per-element rounding-error scales (Eq, Ek, Ev), float64 [T, H, d] each:

        Eq = scale (|dS| |k| + D (P |k|)),   Ek = scale (|dS|^T |q| + P^T (D |q|)),   Ev = P^T |dO|

    with D_i = 2 sum_e |dO_ie| (P |v|)_ie.  The first terms are the sums of absolute
    products whose one rounded factor (dS, or P for dv) moves each product by at most u
    of itself; the D terms carry the error of rowsum(dO * o) when o was rounded.  Every
    entry is >= |gradient| (triangle inequality) and 0 on segment-0 rows."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); do = np.asarray(do, np.float64)
    T, H, d = q.shape
    sc = _scale(scale, d)
    offsets = np.asarray(offsets, dtype=np.int64)
    seg = segment_ids(offsets, cand_start, valid, attend_padded_history)
    eq, ek, ev = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        if hi == lo:
            continue
        mask = isolation_mask(seg[lo:hi])
        for h in range(H):
            eq[lo:hi, h], ek[lo:hi, h], ev[lo:hi, h] = _user_head_error_scale(
                q[lo:hi, h], k[lo:hi, h], v[lo:hi, h], do[lo:hi, h], mask, sc)
    return eq, ek, ev


def _cand_only_as_full(q_cand, k_hist, v_hist, k_cand, v_cand, do, hist_offsets, cand_offsets):
    """The page's fallback layout of a candidate-only layer: per user [frozen history |
    candidates] as one full-sequence user.  History rows are queries of the fallback too,
    but the layer keeps only the candidate rows, so their output gradient is 0 (and their q
    never matters).  Returns the full-layout arrays and the row maps."""
    hoff = np.asarray(hist_offsets, np.int64)
    coff = np.asarray(cand_offsets, np.int64)
    B = len(coff) - 1
    H, d = np.shape(q_cand)[1:]
    hist_rows, cand_rows, offsets, cand_start = [], [], [0], []
    for b in range(B):
        base = offsets[-1]
        nh, nc = int(hoff[b + 1] - hoff[b]), int(coff[b + 1] - coff[b])
        hist_rows.append(np.arange(base, base + nh))
        cand_rows.append(np.arange(base + nh, base + nh + nc))
        cand_start.append(base + nh)
        offsets.append(base + nh + nc)
    T = offsets[-1]
    hr = np.concatenate(hist_rows + [np.zeros(0, np.int64)]).astype(np.int64)
    cr = np.concatenate(cand_rows + [np.zeros(0, np.int64)]).astype(np.int64)
    q, k, v, g = (np.zeros((T, H, d)) for _ in range(4))
    q[cr] = q_cand; k[hr] = k_hist; k[cr] = k_cand
    v[hr] = v_hist; v[cr] = v_cand; g[cr] = do
    return q, k, v, g, np.asarray(offsets, np.int64), np.asarray(cand_start, np.int64), hr, cr


def cand_only_attention_backward(q_cand, k_hist, v_hist, k_cand, v_cand, do, hist_offsets, cand_offsets,
                                 scale=None):
    """Gradients of a candidate-only layer (Candidate isolation attention mask page, section
    "只更新候选的末尾层") w.r.t. its five inputs for the candidates' output gradient ``do``:
    (dq_cand, dk_hist, dv_hist, dk_cand, dv_cand), float64.  The layer is its fallback -- the
    full layer over [frozen history | candidates] keeping the candidate rows -- so these are
    that layer's gradients with a zero output gradient on the history rows."""
    q, k, v, g, off, cs, hr, cr = _cand_only_as_full(q_cand, k_hist, v_hist, k_cand, v_cand, do,
                                                     hist_offsets, cand_offsets)
    dq, dk, dv = full_attention_backward(q, k, v, g, off, cs, scale=scale)
    return dq[cr], dk[hr], dv[hr], dk[cr], dv[cr]


def cand_only_gradient_error_scale(q_cand, k_hist, v_hist, k_cand, v_cand, do, hist_offsets, cand_offsets,
                                   scale=None):
    """``gradient_error_scale`` of the candidate-only layer, per gradient in the order of
    ``cand_only_attention_backward``."""
    q, k, v, g, off, cs, hr, cr = _cand_only_as_full(q_cand, k_hist, v_hist, k_cand, v_cand, do,
                                                     hist_offsets, cand_offsets)
    eq, ek, ev = gradient_error_scale(q, k, v, g, off, cs, scale=scale)
    return eq[cr], ek[hr], ev[hr], ek[cr], ev[cr]
