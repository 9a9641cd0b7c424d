"""Oracle: right-anchored rotary position embedding in float64 (test infrastructure only).

Candidate isolation attention mask page, section "位置编码：候选共用一个位置": the
ranker's positions are right-anchored -- the newest history row always sits at
history_end - 1 however long the history is, and every candidate takes the single
position history_end -- so the rotary encoding cannot tell candidates apart and,
with the isolation mask, reordering candidates cannot change a score.

Readings where the page is silent (each listed in the design notes):
  * positions are row indices within the user's row [prefix | (pad) | history |
    candidates]; history_end is the candidate start, so position(row) =
    min(row - user_start, cand_start - user_start), plus an optional per-user base
    (a candidate-only layer gives its candidate rows base = frozen history length);
  * the rotary encoding itself is the standard one (Su et al., RoFormer): feature
    pairs (2i, 2i+1) rotate by the angle position * base^(-2i/d), base 10000 unless
    given;
  * it is applied to q and k of every row (values are not rotated), before the
    attention of the page's mask.
"""
from __future__ import annotations

import numpy as np

DEFAULT_BASE = 10000.0


def right_anchored_positions(offsets, cand_start, pos_base=None) -> np.ndarray:
    """Position of every row: pos_base[b] + min(row - offsets[b], cand_start[b] - offsets[b])."""
    offsets = np.asarray(offsets, dtype=np.int64)
    cand_start = np.asarray(cand_start, dtype=np.int64)
    B = len(offsets) - 1
    base = np.zeros(B, dtype=np.int64) if pos_base is None else np.asarray(pos_base, dtype=np.int64)
    pos = np.zeros(int(offsets[-1]) if B > 0 else 0, dtype=np.int64)
    for b in range(B):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        local = np.arange(hi - lo, dtype=np.int64)
        pos[lo:hi] = base[b] + np.minimum(local, int(cand_start[b]) - lo)
    return pos


def rotary_angles(pos, d, base=DEFAULT_BASE) -> np.ndarray:
    """Angle of feature pair i at each position: pos * base^(-2i/d); float64 [T, d/2]."""
    if d % 2:
        raise ValueError("the rotary encoding pairs features: d must be even")
    base = DEFAULT_BASE if (base is None or base <= 0) else float(base)
    inv_freq = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(x, pos, base=DEFAULT_BASE) -> np.ndarray:
    """Rotate features (2i, 2i+1) of every row of x [T, H, d] by its angle; float64."""
    x = np.asarray(x, dtype=np.float64)
    T, H, d = x.shape
    ang = rotary_angles(pos, d, base)[:, None, :]        # [T, 1, d/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def full_attention_rope(q, k, v, offsets, cand_start, valid=None, attend_padded_history=False,
                        scale=None, base=DEFAULT_BASE) -> np.ndarray:
    """Full-sequence attention of the page's mask on right-anchored rotary q and k."""
    from .attention import full_attention
    pos = right_anchored_positions(offsets, cand_start)
    return full_attention(rope(q, pos, base), rope(k, pos, base), v, offsets, cand_start, valid,
                          attend_padded_history, scale)


def cand_only_attention_rope(q_cand, k_hist, v_hist, k_cand, v_cand, hist_offsets, cand_offsets,
                             scale=None, base=DEFAULT_BASE) -> np.ndarray:
    """Candidate-only layer on rotary q and k: frozen history rows sit at their own
    positions 0 .. h_b-1, every candidate at h_b (the history end)."""
    from .attention import cand_only_attention
    hoff = np.asarray(hist_offsets, dtype=np.int64)
    coff = np.asarray(cand_offsets, dtype=np.int64)
    pos_h = right_anchored_positions(hoff, hoff[1:])
    pos_c = right_anchored_positions(coff, coff[:-1], pos_base=np.diff(hoff))
    return cand_only_attention(rope(q_cand, pos_c, base), rope(k_hist, pos_h, base), v_hist,
                               rope(k_cand, pos_c, base), v_cand, hoff, coff, scale)
