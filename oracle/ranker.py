"""Oracle: the ranker's layer stack over a jagged batch, in float64 (test infrastructure only).

Candidate isolation attention mask page, section "只更新候选的末尾层": the first
L - N layers run over the whole sequence [prefix | history | candidates] under the
isolation mask; then the hidden states are split into history and candidates, the
history states are frozen, and the last N layers update only the candidates, whose
queries read the frozen history (as keys and values) and their own key and value.
Section "位置编码：候选共用一个位置" places the rotary positions.  Because the history
never reads candidates (section "掩码长什么样"), the history's keys and values of
every layer are the same for any set of candidates: a later request for the same
users with new candidates can reuse them, and every layer then becomes a
candidate-only layer over that cache.

The pages do not print the layer's inside.  The reading taken here (each listed in
the design notes): a pre-norm attention block,

    h = rms_norm(x) * gain,   [q | k | v] = h W_qkv^T,   q, k <- rotary(q, k)
    x <- x + attention(q, k, v) W_o^T

with W_qkv [3D, D], W_o [D, D] (out x in), D = H d, heads laid out [H, d] inside a
row, rms_norm(x) = x / sqrt(mean(x^2) + eps), eps = 1e-6.  A frozen history row of a
candidate-only layer gives its key and value through that layer's own norm and
projections (and its rotary position).  No feed-forward block and no action head.

``candidate_only_layers_update_user_token`` (named on the page, section "只更新候选的末尾层",
with no further definition; off by default there).  Reading taken: with it on, a user's
prefix rows (the user tokens) keep being updated in the candidate-only layers, under the
same attention contract as in the full layers (they read the prefix and history rows,
never candidates); only the history rows stay frozen.  Such a layer is the page's
fallback with the prefix rows kept: the full layer over [prefix (current) | history
(frozen) | candidates (current)], after which the history rows are put back to their
frozen states.  The prefix never reads a candidate, so the keys and values a later
request reuses stay candidate-independent.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .attention import cand_only_attention, full_attention
from .rotary import DEFAULT_BASE, right_anchored_positions, rope

RMS_EPS = 1e-6


@dataclass
class Layer:
    gain: np.ndarray      # [D]
    w_qkv: np.ndarray     # [3D, D]
    w_o: np.ndarray       # [D, D]


def rms_norm(x, gain, eps=RMS_EPS) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain over the last axis; float64."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(gain, np.float64)


def _qkv(x, layer, H, d):
    h = rms_norm(x, layer.gain)
    qkv = h @ np.asarray(layer.w_qkv, np.float64).T
    D = H * d
    return (qkv[:, :D].reshape(-1, H, d), qkv[:, D:2 * D].reshape(-1, H, d),
            qkv[:, 2 * D:].reshape(-1, H, d))


def _out(x, o, layer):
    return np.asarray(x, np.float64) + o.reshape(o.shape[0], -1) @ np.asarray(layer.w_o, np.float64).T


def block_full(x, layer, offsets, cand_start, H, d, base=DEFAULT_BASE, scale=None) -> np.ndarray:
    """One full-sequence layer over x [T, D]; returns the new x."""
    q, k, v = _qkv(x, layer, H, d)
    pos = right_anchored_positions(offsets, cand_start)
    o = full_attention(rope(q, pos, base), rope(k, pos, base), v, offsets, cand_start, scale=scale)
    return _out(x, o, layer)


def history_kv(x_hist, layer, hist_offsets, H, d, base=DEFAULT_BASE):
    """Keys (rotated at positions 0 .. h_b-1) and values of frozen history rows [Th, D]."""
    _, k, v = _qkv(x_hist, layer, H, d)
    hoff = np.asarray(hist_offsets, np.int64)
    return rope(k, right_anchored_positions(hoff, hoff[1:]), base), v


def block_cand_only(x_cand, k_hist, v_hist, layer, hist_offsets, cand_offsets, H, d, base=DEFAULT_BASE,
                    scale=None) -> np.ndarray:
    """One candidate-only layer: candidates [Tc, D] read the user's history keys (already
    rotated) and values [Th, H, d] plus their own; returns the new candidate states."""
    q, k, v = _qkv(x_cand, layer, H, d)
    hoff = np.asarray(hist_offsets, np.int64)
    coff = np.asarray(cand_offsets, np.int64)
    pos = right_anchored_positions(coff, coff[:-1], pos_base=np.diff(hoff))
    o = cand_only_attention(rope(q, pos, base), k_hist, v_hist, rope(k, pos, base), v, hoff, coff, scale)
    return _out(x_cand, o, layer)


def split_history_and_candidates(x, offsets, cand_start):
    """(x_hist [Th, D], x_cand [Tc, D], hist_offsets, cand_offsets): each user's rows before
    its candidate start, then its candidate rows, both concatenated in user order."""
    offsets = np.asarray(offsets, np.int64)
    cand_start = np.asarray(cand_start, np.int64)
    hist_rows = [np.arange(offsets[b], cand_start[b]) for b in range(len(cand_start))]
    cand_rows = [np.arange(cand_start[b], offsets[b + 1]) for b in range(len(cand_start))]
    hoff = np.concatenate([[0], np.cumsum([len(r) for r in hist_rows])]).astype(np.int64)
    coff = np.concatenate([[0], np.cumsum([len(r) for r in cand_rows])]).astype(np.int64)
    hidx = np.concatenate(hist_rows + [np.zeros(0, np.int64)]).astype(np.int64)
    cidx = np.concatenate(cand_rows + [np.zeros(0, np.int64)]).astype(np.int64)
    x = np.asarray(x, np.float64)
    return x[hidx], x[cidx], hoff, coff


def block_user_token_layer(x_p, x_h, x_c, layer, p, hist_offsets, cand_offsets, H, d, base, scale):
    """One candidate-only layer that also updates the user tokens: the full layer over each
    user's [prefix x_p | frozen history x_h | candidates x_c], history rows put back.
    p[b] = user b's prefix rows, the first p[b] rows of its block in hist_offsets (those of
    x_h are the frozen copies, replaced here by x_p).  Returns (x_p, x_c, k_ph, v_ph): the
    new prefix and candidate states and the keys (rotated) and values of [prefix | history]
    rows this layer read."""
    hoff = np.asarray(hist_offsets, np.int64)
    coff = np.asarray(cand_offsets, np.int64)
    poff = np.concatenate([[0], np.cumsum(p)]).astype(np.int64)
    rows, offs, cs = [], [0], []
    for b in range(len(p)):
        blk = np.concatenate([x_p[poff[b]:poff[b + 1]], x_h[hoff[b] + p[b]:hoff[b + 1]], x_c[coff[b]:coff[b + 1]]])
        rows.append(blk)
        cs.append(offs[-1] + hoff[b + 1] - hoff[b])
        offs.append(offs[-1] + len(blk))
    X = np.concatenate(rows) if rows else np.zeros((0, x_c.shape[1]))
    offs, cs = np.asarray(offs, np.int64), np.asarray(cs, np.int64)
    _, k, v = _qkv(X, layer, H, d)
    kr = rope(k, right_anchored_positions(offs, cs), base)
    Y = block_full(X, layer, offs, cs, H, d, base, scale)
    new_p, new_c, k_ph, v_ph = [], [], [], []
    for b in range(len(p)):
        lo, c = offs[b], cs[b]
        new_p.append(Y[lo:lo + p[b]])
        new_c.append(Y[c:offs[b + 1]])
        k_ph.append(kr[lo:c]); v_ph.append(v[lo:c])
    cat = lambda parts, w: np.concatenate(parts) if parts else np.zeros((0,) + w)
    return (cat(new_p, (x_c.shape[1],)), cat(new_c, (x_c.shape[1],)), cat(k_ph, (H, d)), cat(v_ph, (H, d)))


def ranker_forward(x, layers, n_cand_only, offsets, cand_start, H, d, base=DEFAULT_BASE, scale=None,
                   user_tokens=None):
    """The layer stack over x [T, D]: len(layers) - n_cand_only full layers, the split, then
    n_cand_only candidate-only layers.  Returns (x_cand [Tc, D], x_hist [Th, D], cache):
    x_hist = the states of each user's rows before its candidate start after the last layer
    (frozen, or with ``user_tokens`` the prefix rows updated); cache[l] = (k_hist, v_hist)
    of layer l for those rows, the keys and values a later request reuses.

    ``user_tokens`` (int [B], prefix rows per user, or None): candidate_only_layers_update_user_token
    on, under the reading in this module's header."""
    n_full = len(layers) - n_cand_only
    cache = []
    for layer in layers[:n_full]:
        _, k, v = _qkv(x, layer, H, d)
        pos = right_anchored_positions(offsets, cand_start)
        kh = split_history_and_candidates(rope(k, pos, base).reshape(len(x), -1), offsets, cand_start)[0]
        vh = split_history_and_candidates(v.reshape(len(x), -1), offsets, cand_start)[0]
        cache.append((kh.reshape(-1, H, d), vh.reshape(-1, H, d)))
        x = block_full(x, layer, offsets, cand_start, H, d, base, scale)
    x_hist, x_cand, hoff, coff = split_history_and_candidates(x, offsets, cand_start)
    if user_tokens is None:
        for layer in layers[n_full:]:
            kh, vh = history_kv(x_hist, layer, hoff, H, d, base)
            cache.append((kh, vh))
            x_cand = block_cand_only(x_cand, kh, vh, layer, hoff, coff, H, d, base, scale)
        return x_cand, x_hist, cache
    p = np.asarray(user_tokens, np.int64)
    x_p = np.concatenate([x_hist[hoff[b]:hoff[b] + p[b]] for b in range(len(p))] + [np.zeros((0, x.shape[1]))])
    for layer in layers[n_full:]:
        x_p, x_cand, kh, vh = block_user_token_layer(x_p, x_hist, x_cand, layer, p, hoff, coff, H, d, base, scale)
        cache.append((kh, vh))
    poff = np.concatenate([[0], np.cumsum(p)])
    x_hist = x_hist.copy()
    for b in range(len(p)):
        x_hist[hoff[b]:hoff[b] + p[b]] = x_p[poff[b]:poff[b + 1]]
    return x_cand, x_hist, cache


def ranker_forward_cached(x_cand, cache, layers, hist_offsets, cand_offsets, H, d, base=DEFAULT_BASE,
                          scale=None) -> np.ndarray:
    """Candidates [Tc, D] of a request whose users' history keys and values per layer are in
    ``cache``: every layer is a candidate-only layer over the cache."""
    x = np.asarray(x_cand, np.float64)
    for layer, (kh, vh) in zip(layers, cache):
        x = block_cand_only(x, kh, vh, layer, hist_offsets, cand_offsets, H, d, base, scale)
    return x


# --------------------------------------------------------------------------- rounding-error scale
#
# Not a result of the method: the spread that the probabilistic model of rounding errors
# (each rounding multiplies its result by 1 + e, e independent and uniform in [-u, u])
# gives each element of one layer's update (new state - old state) when the layer is
# computed with h, q, k, v, the rotated q and k, the unnormalised attention weights before
# the P v product and the attention output o rounded to bfloat16 (u = 2^-8), everything
# else in float32.  The per-element standard deviation is estimated by running the layer
# with such perturbations drawn from a seeded generator; a test bounds an implementation of
# that arithmetic by a fixed multiple of it (plus float32-level terms, ``f32_slack``).

U_BF16 = 2.0 ** -8
U_F32 = 2.0 ** -24
ROUNDING_POINTS = ("norm", "proj", "rotary", "weights", "output")


def _perturbed_full_layer(x, layer, offsets, cand_start, H, d, base, scale, jitter):
    """``block_full``'s update of x [T, D] with ``jitter(point, array)`` applied at each
    rounding point; returns (update [T, D], attention output [T, H, d])."""
    from .attention import _scale
    x = np.asarray(x, np.float64)
    D = H * d
    h = jitter("norm", rms_norm(x, layer.gain))
    qkv = jitter("proj", h @ np.asarray(layer.w_qkv, np.float64).T)
    q, k, v = (qkv[:, i * D:(i + 1) * D].reshape(-1, H, d) for i in range(3))
    pos = right_anchored_positions(offsets, cand_start)
    qr, kr = jitter("rotary", rope(q, pos, base)), jitter("rotary", rope(k, pos, base))
    sc = _scale(scale, d)
    offsets = np.asarray(offsets, np.int64)
    o = np.zeros_like(qr)
    for b in range(len(offsets) - 1):
        lo, cs, hi = int(offsets[b]), int(cand_start[b]), int(offsets[b + 1])
        n = hi - lo
        if n == 0:
            continue
        # every row reads the rows before the candidate start; a candidate also itself
        mask = np.zeros((n, n), dtype=bool)
        mask[:, :cs - lo] = True
        mask[np.arange(n), np.arange(n)] = True
        for hh in range(H):
            s = np.where(mask, sc * (qr[lo:hi, hh] @ kr[lo:hi, hh].T), -np.inf)
            w = np.exp(s - s.max(axis=1, keepdims=True))
            o[lo:hi, hh] = jitter("output", (jitter("weights", w) @ v[lo:hi, hh]) / w.sum(axis=1, keepdims=True))
    return o.reshape(len(x), D) @ np.asarray(layer.w_o, np.float64).T, o


def full_layer_rounding_sigma(x, layer, offsets, cand_start, H, d, base=DEFAULT_BASE, scale=None,
                              points=ROUNDING_POINTS, samples=128, seed=0):
    """Per-element standard deviation [T, D] of ``block_full``'s update of x under the
    probabilistic rounding model at ``points`` (a subset of ROUNDING_POINTS), estimated from
    ``samples`` seeded draws."""
    rng = np.random.default_rng(seed)
    exact, _ = _perturbed_full_layer(x, layer, offsets, cand_start, H, d, base, scale, lambda p, a: a)

    def jitter(point, a):
        return a * (1.0 + rng.uniform(-U_BF16, U_BF16, a.shape)) if point in points else a
    acc = np.zeros_like(exact)
    for _ in range(samples):
        upd, _ = _perturbed_full_layer(x, layer, offsets, cand_start, H, d, base, scale, jitter)
        acc += (upd - exact) ** 2
    return np.sqrt(acc / samples)


def cand_only_layer_rounding_sigma(x_cand, x_hist, layer, hist_offsets, cand_offsets, H, d, base=DEFAULT_BASE,
                                   scale=None, points=ROUNDING_POINTS, samples=128, seed=0):
    """The same for a candidate-only layer's update of the candidates x_cand [Tc, D] over the
    frozen rows x_hist (their keys and values carry the same roundings), computed on the
    page's fallback layout: per user [frozen history | candidates], candidate rows kept."""
    x, off, cs, rows = _fallback_layout(x_hist, x_cand, hist_offsets, cand_offsets)
    return full_layer_rounding_sigma(x, layer, off, cs, H, d, base, scale, points, samples, seed)[rows]


def f32_slack(x, layer, offsets, cand_start, H, d, base=DEFAULT_BASE, scale=None):
    """Float32-level error terms of a layer's update [T, D]: the accumulation of o W_o^T over
    D products, the residual add, and a few float32 roundings of every earlier step relative
    to the update's magnitude."""
    upd, o = _perturbed_full_layer(x, layer, offsets, cand_start, H, d, base, scale, lambda p, a: a)
    wo = np.abs(np.asarray(layer.w_o, np.float64)).T
    D = H * d
    return (D + 2) * U_F32 * (np.abs(o.reshape(len(upd), D)) @ wo) + 4 * U_F32 * np.abs(np.asarray(x, np.float64)) \
        + 2.0 ** -18 * np.abs(upd)


def _fallback_layout(x_hist, x_cand, hist_offsets, cand_offsets):
    """Per user [frozen history rows | candidate rows] as one full-sequence batch: (x, offsets,
    cand_start, candidate rows)."""
    hoff = np.asarray(hist_offsets, np.int64)
    coff = np.asarray(cand_offsets, np.int64)
    parts, off, cs, rows = [], [0], [], []
    for b in range(len(coff) - 1):
        parts += [np.asarray(x_hist, np.float64)[hoff[b]:hoff[b + 1]], np.asarray(x_cand, np.float64)[coff[b]:coff[b + 1]]]
        cs.append(off[-1] + int(hoff[b + 1] - hoff[b]))
        rows += range(cs[-1], cs[-1] + int(coff[b + 1] - coff[b]))
        off.append(cs[-1] + int(coff[b + 1] - coff[b]))
    x = np.concatenate(parts) if parts else np.zeros((0, np.shape(x_cand)[1]))
    return x, np.asarray(off, np.int64), np.asarray(cs, np.int64), np.asarray(rows, np.int64)
