"""Pins for the layer-stack oracle (oracle/ranker.py).

Each ``pin_*`` raises AssertionError when the oracle disagrees with
 * torch's CPU ``rms_norm`` in float64 (a library routine) and the closed form of a
   constant row,
 * a separate float64 torch implementation of the whole stack: torch's ``linear``,
   ``rms_norm`` and ``scaled_dot_product_attention`` with the admitted keys written here
   from the plain-language rule, rotary positions from the page's rule and the rotation
   as complex multiplication, and the candidate-only layers done the page's fallback
   way (the full layer over the whole sequence, then the non-candidate rows put back to
   their frozen states),
 * closed forms (W_o = 0 leaves every state unchanged; W_q = W_k = 0 with W_v = W_o = I
   gives each row the mean of its admitted normalised rows), or
 * the page's invariants: candidate order, history independence, and the cached request
   (every layer candidate-only over the history keys and values) equal to the full one,
   also with the user tokens updated in the candidate-only layers (the same torch stack
   with only the history rows frozen).
They call the oracle through its module at call time, so tests can plant mistakes.
"""
from __future__ import annotations

import numpy as np

from oracle import ranker as RK

SHAPES = dict(prefix=[1, 0, 2, 1], hist=[3, 0, 4, 6], cand=[2, 3, 0, 4])


def _layout(prefix, hist, cand):
    lengths = np.asarray(prefix) + np.asarray(hist) + np.asarray(cand)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    cand_start = offsets[:-1] + np.asarray(prefix) + np.asarray(hist)
    return offsets, cand_start


def make_stack(seed, n_layers=3, H=2, d=4, shapes=SHAPES):
    rng = np.random.default_rng(seed)
    offsets, cand_start = _layout(**shapes)
    D = H * d
    x = rng.standard_normal((int(offsets[-1]), D))
    layers = [RK.Layer(gain=1.0 + 0.2 * rng.standard_normal(D),
                       w_qkv=rng.standard_normal((3 * D, D)) / np.sqrt(D),
                       w_o=rng.standard_normal((D, D)) / np.sqrt(D)) for _ in range(n_layers)]
    return x, layers, offsets, cand_start, H, d


def _torch_stack(x, layers, n_cand_only, offsets, cand_start, H, d, base, user_tokens=None):
    import torch
    import torch.nn.functional as F
    T, D = x.shape
    X = torch.from_numpy(np.asarray(x, np.float64))
    pos = torch.zeros(T, dtype=torch.float64)
    is_hist = torch.zeros(T, dtype=torch.bool)
    frozen_rows = torch.zeros(T, dtype=torch.bool)
    users = []
    for b in range(len(cand_start)):
        lo, cs, hi = int(offsets[b]), int(cand_start[b]), int(offsets[b + 1])
        p = 0 if user_tokens is None else int(user_tokens[b])
        for r in range(lo, hi):
            pos[r] = min(r, cs) - lo          # newest history row at cs-1-lo, candidates at cs-lo
            is_hist[r] = r < cs
            frozen_rows[r] = lo + p <= r < cs   # with user tokens updated, the prefix is not frozen
        # a row reads the rows before the candidate start, and a candidate also itself
        m = torch.tensor([[j < cs - lo or i == j for j in range(hi - lo)] for i in range(hi - lo)],
                         dtype=torch.bool).reshape(hi - lo, hi - lo)
        users.append((lo, hi, m))
    inv = base ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    rot = torch.polar(torch.ones(T, d // 2, dtype=torch.float64), pos[:, None] * inv[None, :])

    def rotate(t):
        c = torch.view_as_complex(t.reshape(T, H, d // 2, 2).contiguous())
        return torch.view_as_real(c * rot[:, None, :]).reshape(T, H, d)

    def layer(X, L):
        h = F.rms_norm(X, (D,), weight=torch.from_numpy(L.gain), eps=RK.RMS_EPS)
        q, k, v = F.linear(h, torch.from_numpy(L.w_qkv)).split(D, dim=1)
        q, k, v = rotate(q.reshape(T, H, d)), rotate(k.reshape(T, H, d)), v.reshape(T, H, d)
        out = torch.zeros(T, H, d, dtype=torch.float64)
        for lo, hi, m in users:
            if hi > lo:
                o = F.scaled_dot_product_attention(q[lo:hi].transpose(0, 1), k[lo:hi].transpose(0, 1),
                                                   v[lo:hi].transpose(0, 1), attn_mask=m)
                out[lo:hi] = o.transpose(0, 1)
        return X + F.linear(out.reshape(T, D), torch.from_numpy(L.w_o))

    n_full = len(layers) - n_cand_only
    for L in layers[:n_full]:
        X = layer(X, L)
    frozen = X.clone()
    for L in layers[n_full:]:
        X = torch.where(frozen_rows[:, None], frozen, layer(X, L))
    return X[~is_hist].numpy(), X[is_hist].numpy()


def pin_rms_norm():
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 12)) * rng.uniform(0.01, 10, (7, 1))
    g = rng.standard_normal(12)
    want = F.rms_norm(torch.from_numpy(x), (12,), weight=torch.from_numpy(g), eps=RK.RMS_EPS).numpy()
    assert np.max(np.abs(RK.rms_norm(x, g) - want)) <= 1e-12
    c = np.full((1, 5), -3.0)
    assert np.allclose(RK.rms_norm(c, np.arange(5.0)), -3.0 / np.sqrt(9.0 + RK.RMS_EPS) * np.arange(5.0),
                       rtol=0, atol=1e-15)


def pin_torch_stack():
    for seed, n_cand_only in ((11, 1), (12, 2), (13, 0)):
        x, layers, off, cs, H, d = make_stack(seed)
        got_c, got_h, _ = RK.ranker_forward(x, layers, n_cand_only, off, cs, H, d, base=50.0)
        want_c, want_h = _torch_stack(x, layers, n_cand_only, off, cs, H, d, base=50.0)
        assert np.max(np.abs(got_c - want_c)) <= 1e-10, seed
        assert np.max(np.abs(got_h - want_h)) <= 1e-10, seed


def pin_user_tokens():
    """candidate_only_layers_update_user_token: the torch stack with the prefix rows left
    out of the frozen set; no user tokens is the default stack; the cached request and the
    history's independence of candidates still hold."""
    x, layers, off, cs, H, d = make_stack(41)
    p = np.array(SHAPES["prefix"])
    for n_cand_only in (1, 2):
        got_c, got_h, _ = RK.ranker_forward(x, layers, n_cand_only, off, cs, H, d, base=50.0, user_tokens=p)
        want_c, want_h = _torch_stack(x, layers, n_cand_only, off, cs, H, d, base=50.0, user_tokens=p)
        assert np.max(np.abs(got_c - want_c)) <= 1e-10
        assert np.max(np.abs(got_h - want_h)) <= 1e-10
    base_c, base_h, base_cache = RK.ranker_forward(x, layers, 2, off, cs, H, d)
    z_c, z_h, z_cache = RK.ranker_forward(x, layers, 2, off, cs, H, d, user_tokens=np.zeros_like(p))
    assert np.max(np.abs(z_c - base_c)) <= 1e-12 and np.max(np.abs(z_h - base_h)) <= 1e-12
    xc, xh, cache = RK.ranker_forward(x, layers, 2, off, cs, H, d, user_tokens=p)
    assert np.max(np.abs(xh - base_h)) > 1e-3          # the prefix rows did move
    _, xc0, hoff, coff = RK.split_history_and_candidates(x, off, cs)
    again = RK.ranker_forward_cached(xc0, cache, layers, hoff, coff, H, d)
    assert np.max(np.abs(again - xc)) <= 1e-12
    x3 = x.copy()
    x3[int(cs[0])] += 5.0
    _, xh3, cache3 = RK.ranker_forward(x3, layers, 2, off, cs, H, d, user_tokens=p)
    assert np.array_equal(xh3, xh)
    for (k1, v1), (k2, v2) in zip(cache, cache3):
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def pin_closed_forms():
    x, layers, off, cs, H, d = make_stack(21)
    D = H * d
    # W_o = 0: every layer is the identity on the states
    flat = [RK.Layer(L.gain, L.w_qkv, np.zeros((D, D))) for L in layers]
    xc, xh, _ = RK.ranker_forward(x, flat, 1, off, cs, H, d)
    hist = np.concatenate([np.arange(off[b], cs[b]) for b in range(len(cs))]).astype(int)
    cand = np.concatenate([np.arange(cs[b], off[b + 1]) for b in range(len(cs))]).astype(int)
    assert np.array_equal(xc, x[cand]) and np.array_equal(xh, x[hist])
    # W_q = W_k = 0, W_v = W_o = I: one layer adds the mean of the admitted normalised rows
    w = np.zeros((3 * D, D))
    w[2 * D:] = np.eye(D)
    L = RK.Layer(layers[0].gain, w, np.eye(D))
    got = RK.block_full(x, L, off, cs, H, d)
    h = RK.rms_norm(x, L.gain)
    for b in range(len(cs)):
        lo, c, hi = int(off[b]), int(cs[b]), int(off[b + 1])
        for r in range(lo, hi):
            keys = list(range(lo, c)) + ([r] if r >= c else [])
            assert np.max(np.abs(got[r] - (x[r] + h[keys].mean(axis=0)))) <= 1e-12


def pin_invariants():
    x, layers, off, cs, H, d = make_stack(31)
    xc, xh, cache = RK.ranker_forward(x, layers, 1, off, cs, H, d)
    xh0, xc0, hoff, coff = RK.split_history_and_candidates(x, off, cs)
    # a later request with the same users: every layer candidate-only over the cache
    again = RK.ranker_forward_cached(xc0, cache, layers, hoff, coff, H, d)
    assert np.max(np.abs(again - xc)) <= 1e-12
    # candidates in another order: the same per-candidate outputs
    b = 3
    perm = np.arange(len(x))
    perm[int(cs[b]):int(off[b + 1])] = np.random.default_rng(5).permutation(
        np.arange(int(cs[b]), int(off[b + 1])))
    xc2, xh2, _ = RK.ranker_forward(x[perm], layers, 1, off, cs, H, d)
    inv = np.argsort(perm[int(cs[b]):int(off[b + 1])] - int(cs[b]))
    c0 = int(coff[b])
    assert np.max(np.abs(xc2[c0:c0 + len(inv)][inv] - xc[c0:c0 + len(inv)])) <= 1e-12
    assert np.array_equal(np.delete(xc2, np.s_[c0:c0 + len(inv)], 0), np.delete(xc, np.s_[c0:c0 + len(inv)], 0))
    # other candidates change nothing of the history (states or cache) nor of other candidates
    x3 = x.copy()
    x3[int(cs[0])] += 5.0
    xc3, xh3, cache3 = RK.ranker_forward(x3, layers, 1, off, cs, H, d)
    assert np.array_equal(xh3, xh)
    for (k1, v1), (k2, v2) in zip(cache, cache3):
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert np.array_equal(xc3[1:], xc[1:])


def _emulated_layer(x, L, offsets, cand_start, H, d, base, rounded):
    """One full-sequence layer in float64 torch, written here, with bfloat16 rounding (torch's)
    only at the points named in ``rounded``: "norm" (h), "proj" (q, k, v), "rotary" (the
    rotated q and k), "weights" (the unnormalised softmax weights before the P v product;
    their row sum stays exact) and "output" (the attention output).  Returns the new x."""
    import torch
    import torch.nn.functional as F
    T, D = x.shape

    def r(t, where):
        return t.to(torch.bfloat16).to(torch.float64) if where in rounded else t
    X = torch.from_numpy(np.asarray(x, np.float64))
    h = r(F.rms_norm(X, (D,), weight=torch.from_numpy(L.gain), eps=RK.RMS_EPS), "norm")
    q, k, v = r(F.linear(h, torch.from_numpy(L.w_qkv)), "proj").split(D, dim=1)
    pos = torch.zeros(T, dtype=torch.float64)
    for b in range(len(cand_start)):
        lo, cs, hi = int(offsets[b]), int(cand_start[b]), int(offsets[b + 1])
        for i in range(lo, hi):
            pos[i] = min(i, cs) - lo
    inv = base ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    rot = torch.polar(torch.ones(T, d // 2, dtype=torch.float64), pos[:, None] * inv[None, :])

    def rotate(t):
        c = torch.view_as_complex(t.reshape(T, H, d // 2, 2).contiguous())
        return r(torch.view_as_real(c * rot[:, None, :]).reshape(T, H, d), "rotary")
    q, k, v = rotate(q), rotate(k), v.reshape(T, H, d)
    out = torch.zeros(T, H, d, dtype=torch.float64)
    sc = 1.0 / np.sqrt(d)
    for b in range(len(cand_start)):
        lo, cs, hi = int(offsets[b]), int(cand_start[b]), int(offsets[b + 1])
        n = hi - lo
        if n == 0:
            continue
        m = torch.tensor([[j < cs - lo or i == j for j in range(n)] for i in range(n)], dtype=torch.bool).reshape(n, n)
        for hh in range(H):
            s = (sc * q[lo:hi, hh] @ k[lo:hi, hh].T).masked_fill(~m, float("-inf"))
            w = torch.exp(s - s.max(dim=1, keepdim=True).values)
            out[lo:hi, hh] = r((r(w, "weights") @ v[lo:hi, hh]) / w.sum(dim=1, keepdim=True), "output")
    return (X + F.linear(out.reshape(T, D), torch.from_numpy(L.w_o))).numpy()


EMULATED = ("norm", "proj", "rotary", "weights", "output")


def _fallback(x_hist, x_cand, hoff, coff):
    """Per user [frozen history | candidates] as one full-sequence layout, and its candidate rows."""
    rows, off, cs, cand_rows = [], [0], [], []
    for b in range(len(coff) - 1):
        rows += [x_hist[hoff[b]:hoff[b + 1]], x_cand[coff[b]:coff[b + 1]]]
        cs.append(off[-1] + hoff[b + 1] - hoff[b])
        cand_rows += list(range(cs[-1], cs[-1] + coff[b + 1] - coff[b]))
        off.append(cs[-1] + coff[b + 1] - coff[b])
    return np.concatenate(rows), np.asarray(off), np.asarray(cs), np.asarray(cand_rows, np.int64)


def pin_layer_rounding_sigma():
    """The rounding spread of one layer's update (``full_layer_rounding_sigma``,
    ``cand_only_layer_rounding_sigma``) against deterministic round-to-nearest-even
    emulations written here (torch's bfloat16 rounding): for each rounding point alone and
    for all of them, the emulated update's error stays within 8 sigma of that point's
    spread, element by element, and its root mean square over sigma lies in [0.1, 2] alone
    and in [0.3, 1.2] for all points together (the
    spread is neither too small nor vacuous; a dominant softmax weight of exactly 1 rounds
    without error, which the model does not know, hence the low end).  Both layer kinds, a flat and a sharp
    softmax.  W_o = 0 gives zero spread."""
    base = 50.0
    for sharp in (1.0, 4.0):
        x, layers, off, cs, H, d = make_stack(61 + int(sharp), n_layers=1, H=2, d=8)
        L = RK.Layer(layers[0].gain, layers[0].w_qkv * sharp, layers[0].w_o)
        xh, xc, hoff, coff = RK.split_history_and_candidates(x, off, cs)
        kh, vh = RK.history_kv(xh, L, hoff, H, d, base)
        fx, foff, fcs, frows = _fallback(xh, xc, hoff, coff)
        cases = (
            ("full", RK.block_full(x, L, off, cs, H, d, base),
             lambda pts: RK.full_layer_rounding_sigma(x, L, off, cs, H, d, base, points=pts, samples=256),
             lambda rnd: _emulated_layer(x, L, off, cs, H, d, base, rnd)),
            ("cand-only", RK.block_cand_only(xc, kh, vh, L, hoff, coff, H, d, base),
             lambda pts: RK.cand_only_layer_rounding_sigma(xc, xh, L, hoff, coff, H, d, base, points=pts,
                                                           samples=256),
             lambda rnd: _emulated_layer(fx, L, foff, fcs, H, d, base, rnd)[frows]),
        )
        # the model runs the layer itself: unperturbed, it is the oracle's layer
        upd, _ = RK._perturbed_full_layer(x, L, off, cs, H, d, base, None, lambda p, a: a)
        assert np.max(np.abs(x + upd - cases[0][1])) <= 1e-12
        for kind, ref, sigma, emulate in cases:
            for pts in [(p,) for p in EMULATED] + [EMULATED]:
                sg = sigma(pts)
                assert sg.shape == ref.shape and np.all(sg >= 0), (kind, pts)
                err = np.abs(emulate(set(pts)) - ref)
                live = sg > 0          # e.g. a lone candidate's output does not depend on its rotation
                assert np.all(err[~live] <= 1e-14), (kind, pts)
                z = err[live] / sg[live]
                assert np.all(z <= 8.0), (kind, pts, sharp, float(z.max()))
                rms = float(np.sqrt(np.mean(z * z)))
                lo_rms, hi_rms = (0.3, 1.2) if len(pts) > 1 else (0.1, 2.0)
                assert lo_rms <= rms <= hi_rms, (kind, pts, sharp, rms)
    x, layers, off, cs, H, d = make_stack(65, n_layers=1, H=2, d=8)
    L = RK.Layer(layers[0].gain, layers[0].w_qkv, np.zeros((H * d, H * d)))
    assert np.all(RK.full_layer_rounding_sigma(x, L, off, cs, H, d, base, samples=4) == 0)

def _float32_layer(x, L, offsets, cand_start, H, d, base):
    """One full-sequence layer computed entirely in float32 torch, written here (angles in
    float64, then cast): the float32-level arithmetic that ``f32_slack`` bounds.  Returns the
    new x in float64."""
    import torch
    import torch.nn.functional as F
    T, D = x.shape
    f = torch.float32
    X = torch.from_numpy(np.asarray(x, np.float32))
    h = F.rms_norm(X, (D,), weight=torch.from_numpy(np.asarray(L.gain, np.float32)), eps=RK.RMS_EPS)
    q, k, v = F.linear(h, torch.from_numpy(np.asarray(L.w_qkv, np.float32))).split(D, dim=1)
    pos = torch.zeros(T, dtype=torch.float64)
    for b in range(len(cand_start)):
        lo, cs, hi = int(offsets[b]), int(cand_start[b]), int(offsets[b + 1])
        for i in range(lo, hi):
            pos[i] = min(i, cs) - lo
    inv = base ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = pos[:, None] * inv[None, :]
    c, s_ = torch.cos(ang).to(f)[:, None, :], torch.sin(ang).to(f)[:, None, :]

    def rot(t):
        t = t.reshape(T, H, d // 2, 2)
        a, b2 = t[..., 0], t[..., 1]
        return torch.stack([a * c - b2 * s_, a * s_ + b2 * c], -1).reshape(T, H, d)
    q, k, v = rot(q), rot(k), v.reshape(T, H, d)
    out = torch.zeros(T, H, d, dtype=f)
    sc = 1.0 / np.sqrt(d)
    for b in range(len(cand_start)):
        lo, cs, hi = int(offsets[b]), int(cand_start[b]), int(offsets[b + 1])
        n = hi - lo
        if n == 0:
            continue
        m = torch.tensor([[j < cs - lo or i == j for j in range(n)] for i in range(n)], dtype=torch.bool)
        for hh in range(H):
            s = (sc * q[lo:hi, hh] @ k[lo:hi, hh].T).masked_fill(~m, float("-inf"))
            w = torch.exp(s - s.max(dim=1, keepdim=True).values)
            out[lo:hi, hh] = (w @ v[lo:hi, hh]) / w.sum(dim=1, keepdim=True)
    return (X + F.linear(out.reshape(T, D), torch.from_numpy(np.asarray(L.w_o, np.float32)))).numpy().astype(np.float64)


def pin_f32_slack():
    """``f32_slack`` against a layer computed entirely in float32 here: element by element
    the float32 layer stays within the slack of the float64 oracle layer, and the slack is
    not vacuous (on a sharp softmax the float32 error reaches more than a third of it).
    Three shapes, a flat and a sharp softmax, and a residual stream scaled by 1000 (the
    normalised layer's update does not change, the residual add's rounding grows)."""
    base = 50.0
    worst = 0.0
    for seed, H, d, sharp, xs in ((71, 2, 8, 1.0, 1.0), (72, 2, 8, 4.0, 1.0), (73, 4, 16, 1.0, 1.0),
                                  (74, 2, 8, 1.0, 1e3)):
        x, layers, off, cs, H, d = make_stack(seed, n_layers=1, H=H, d=d)
        x = x * xs
        L = RK.Layer(layers[0].gain, layers[0].w_qkv * sharp, layers[0].w_o)
        ref = RK.block_full(x, L, off, cs, H, d, base)
        err = np.abs(_float32_layer(x, L, off, cs, H, d, base) - ref)
        sl = RK.f32_slack(x, L, off, cs, H, d, base)
        assert sl.shape == ref.shape and np.all(sl > 0)
        ratio = float(np.max(err / sl))
        assert ratio <= 1.0, (seed, sharp, xs, ratio)
        worst = max(worst, ratio)
    assert worst >= 0.35, worst


RANKER_PINS = [pin_rms_norm, pin_torch_stack, pin_user_tokens, pin_closed_forms, pin_invariants,
               pin_layer_rounding_sigma, pin_f32_slack]
