"""Pins for the backward oracle (oracle/backward.py).

Each ``pin_*`` raises AssertionError when the oracle's gradients disagree with
 * central finite differences of the (separately pinned) forward oracle,
 * torch autograd through torch's CPU scaled_dot_product_attention in float64, with the
   admitted key sets written here from the plain-language rule (a library routine),
 * exactly rounded log-sum-exp sums (math.fsum) for ``attention_lse``,
 * closed forms (a one-row user; a candidate's own key and value),
 * the page's isolation invariants carried over to gradients, or
 * for ``gradient_error_scale``: the triangle inequality, its equality case, and the
   error of gradients computed with P, dS and o rounded to bfloat16 by torch.
They call the oracle through its modules at call time, so tests can plant mistakes.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import attention as A
from oracle import backward as G
from _pins import rng_for, tiny_batches
from workloads import make_full_batch


def _grads(fb, do, scale=None):
    return G.full_attention_backward(fb.q, fb.k, fb.v, do, fb.offsets, fb.cand_start, fb.valid,
                                     fb.attend_padded_history, scale)


def pin_finite_differences():
    """d(sum(O * dO))/dx by central differences of the forward oracle, every entry of
    every tiny batch (holes, empty users, padding with both flags)."""
    eps = 1e-6
    for fb in tiny_batches():
        q, k, v = (np.asarray(x, np.float64) for x in (fb.q, fb.k, fb.v))
        rng = rng_for(91)
        do = rng.standard_normal(q.shape)

        def loss(qq, kk, vv):
            o = A.full_attention(qq, kk, vv, fb.offsets, fb.cand_start, fb.valid, fb.attend_padded_history)
            return float(np.sum(o * do))
        got = G.full_attention_backward(q, k, v, do, fb.offsets, fb.cand_start, fb.valid,
                                        fb.attend_padded_history)
        for which, x in enumerate((q, k, v)):
            num = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                i = it.multi_index
                xp, xm = x.copy(), x.copy()
                xp[i] += eps; xm[i] -= eps
                args_p = [q, k, v]; args_p[which] = xp
                args_m = [q, k, v]; args_m[which] = xm
                num[i] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            err = np.max(np.abs(num - got[which]))
            assert err <= 1e-6 * (1 + np.max(np.abs(num))), (fb.name, "qkv"[which], err)


def pin_torch_autograd():
    """Gradients through torch's fp64 SDPA with a boolean mask written from the rule:
    history rows see the user's history, candidates see the history and themselves."""
    import torch
    F = torch.nn.functional
    rng = rng_for(92)
    fb = make_full_batch(rng, "bwd-sdpa", prefix=[1, 3, 0], hist=[4, 2, 3], cand=[3, 2, 0], H=2, d=8,
                         dtype="f32", scaled=False)
    do = rng.standard_normal(fb.q.shape)
    dq, dk, dv = _grads(fb, do)
    for b in range(fb.B):
        lo, cs, hi = int(fb.offsets[b]), int(fb.cand_start[b]), int(fb.offsets[b + 1])
        L = hi - lo
        allowed = np.zeros((L, L), dtype=bool)
        for i in range(L):
            for j in range(cs - lo):
                allowed[i, j] = True          # everyone sees the history
            if i >= cs - lo:
                allowed[i, i] = True          # a candidate also sees itself
        t = [torch.from_numpy(np.ascontiguousarray(x[lo:hi].transpose(1, 0, 2))).double().requires_grad_()
             for x in (fb.q, fb.k, fb.v)]
        o = F.scaled_dot_product_attention(*t, attn_mask=torch.from_numpy(allowed))
        o.backward(torch.from_numpy(np.ascontiguousarray(do[lo:hi].transpose(1, 0, 2))))
        for g_t, mine in zip(t, (dq, dk, dv)):
            ref = g_t.grad.numpy().transpose(1, 0, 2)
            assert np.max(np.abs(ref - mine[lo:hi])) <= 1e-11, b


def pin_lse():
    for fb in tiny_batches():
        lse = G.attention_lse(fb.q, fb.k, fb.offsets, fb.cand_start, fb.valid, fb.attend_padded_history)
        sc = 1.0 / math.sqrt(fb.d)
        from oracle.jagged import segment_ids
        seg = segment_ids(fb.offsets, fb.cand_start, fb.valid, fb.attend_padded_history)
        for b in range(fb.B):
            lo, hi = int(fb.offsets[b]), int(fb.offsets[b + 1])
            for i in range(lo, hi):
                if seg[i] == 0:
                    keys = []
                else:
                    keys = [j for j in range(lo, hi) if seg[j] == 1] + ([i] if seg[i] == -1 else [])
                for h in range(fb.H):
                    if not keys:
                        assert lse[i, h] == -np.inf
                        continue
                    s = [sc * math.fsum(float(fb.q[i, h, t]) * float(fb.k[j, h, t]) for t in range(fb.d))
                         for j in keys]
                    m = max(s)
                    want = m + math.log(math.fsum(math.exp(x - m) for x in s))
                    assert abs(lse[i, h] - want) <= 1e-12, (fb.name, i, h)


def pin_closed_forms():
    rng = rng_for(93)
    # a one-row user (its own single key): P = 1, so dv = do and dq = dk = 0
    fb = make_full_batch(rng, "one-row", prefix=[1, 0], hist=[0, 0], cand=[0, 1], H=2, d=4,
                         dtype="f32", scaled=False)
    do = rng.standard_normal(fb.q.shape)
    dq, dk, dv = _grads(fb, do)
    assert np.max(np.abs(dv - do)) <= 1e-15 and np.max(np.abs(dq)) == 0 and np.max(np.abs(dk)) == 0
    # a candidate's own key and value are read only by that candidate:
    # dv_c = p_cc do_c and dk_c = scale * p_cc (do_c . (v_c - o_c)) q_c
    fb = make_full_batch(rng, "cand-own", prefix=[2], hist=[3], cand=[4], H=1, d=6, dtype="f32",
                         scaled=False)
    do = rng.standard_normal(fb.q.shape)
    dq, dk, dv = _grads(fb, do)
    o = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start)
    lse = G.attention_lse(fb.q, fb.k, fb.offsets, fb.cand_start)
    sc = 1.0 / math.sqrt(fb.d)
    for c in range(int(fb.cand_start[0]), fb.T):
        qc, kc, vc = (np.asarray(x[c, 0], np.float64) for x in (fb.q, fb.k, fb.v))
        p = math.exp(sc * float(np.dot(qc, kc)) - lse[c, 0])
        assert np.max(np.abs(dv[c, 0] - p * do[c, 0])) <= 1e-12
        want = sc * p * float(np.dot(do[c, 0], vc - o[c, 0])) * qc
        assert np.max(np.abs(dk[c, 0] - want)) <= 1e-12


def pin_isolation_of_gradients():
    """Gradients of one user never depend on another user's values; padding rows (flag
    False) get none; a candidate's output gradient never reaches other candidates' k, v."""
    rng = rng_for(94)
    fb = make_full_batch(rng, "iso", prefix=[1, 2], hist=[3, 2], cand=[3, 2], pad=[2, 0], H=2, d=4,
                         dtype="f32", scaled=False)
    do = rng.standard_normal(fb.q.shape)
    g0 = _grads(fb, do)
    q2 = fb.q.copy(); q2[int(fb.offsets[1]):] *= 3.0
    g1 = G.full_attention_backward(q2, fb.k, fb.v, do, fb.offsets, fb.cand_start, fb.valid)
    lo1 = int(fb.offsets[1])
    for a, b in zip(g0, g1):
        assert np.array_equal(a[:lo1], b[:lo1])
    pad = np.nonzero(fb.valid == 0)[0]
    for g in g0:
        assert np.all(g[pad] == 0)
    # output gradient on one candidate only: other candidates' k and v get nothing
    c0 = int(fb.cand_start[0])
    do1 = np.zeros_like(do); do1[c0] = do[c0]
    dq, dk, dv = _grads(fb, do1)
    others = [c for c in range(c0 + 1, lo1)]
    assert np.all(dk[others] == 0) and np.all(dv[others] == 0)


def _rounded_grads(fb, do, sc):
    """Gradients with P, o and dS rounded to bfloat16 (torch's rounding) and every other
    step in float64: the arithmetic ``gradient_error_scale`` bounds."""
    import torch

    def r(x):
        return x.to(torch.bfloat16).to(torch.float64)
    seg = G.segment_ids(fb.offsets, fb.cand_start, fb.valid, fb.attend_padded_history)
    out = [np.zeros(fb.q.shape) for _ in range(3)]
    for b in range(fb.B):
        lo, hi = int(fb.offsets[b]), int(fb.offsets[b + 1])
        rows = range(lo, hi)
        adm = np.array([[bool(seg[i]) and (seg[j] == 1 or (i == j and seg[i] == -1)) for j in rows]
                        for i in rows], bool).reshape(hi - lo, hi - lo)
        m = torch.from_numpy(adm)
        for h in range(fb.H):
            q, k, v, g = (torch.from_numpy(np.asarray(x[lo:hi, h], np.float64)) for x in (fb.q, fb.k, fb.v, do))
            s = (sc * q @ k.T).masked_fill(~m, float("-inf"))
            p = torch.softmax(s, dim=1).nan_to_num(0.0)
            o = r(p @ v)
            ds = r(p * (g @ v.T - (g * o).sum(dim=1, keepdim=True)))
            out[0][lo:hi, h] = r(sc * ds @ k).numpy()
            out[1][lo:hi, h] = r(sc * ds.T @ q).numpy()
            out[2][lo:hi, h] = r(r(p).T @ g).numpy()
    return out


def pin_error_scale():
    rng = rng_for(95)
    u = 2.0 ** -8                     # unit roundoff of bfloat16 (8 significant bits)
    for flag in (False, True):
        fb = make_full_batch(rng, "err-scale", prefix=[1, 2, 0], hist=[5, 0, 9], cand=[3, 2, 1],
                             pad=[2, 0, 1], attend_padded_history=flag, H=2, d=8, dtype="f32",
                             scaled=False)
        do = rng.standard_normal(fb.q.shape)
        sc = 1.0 / math.sqrt(fb.d)
        grads = _grads(fb, do)
        es = G.gradient_error_scale(fb.q, fb.k, fb.v, do, fb.offsets, fb.cand_start, fb.valid, flag)
        seg = G.segment_ids(fb.offsets, fb.cand_start, fb.valid, flag)
        for g, e in zip(grads, es):
            assert np.all(e >= np.abs(g) * (1 - 1e-12) - 1e-15)      # triangle inequality
            assert np.all(e[seg == 0] == 0)
        # equality case: every product of dv = P^T dO has one sign when dO >= 0
        ev = G.gradient_error_scale(fb.q, fb.k, fb.v, np.abs(do), fb.offsets, fb.cand_start, fb.valid,
                                    flag)[2]
        dv = _grads(fb, np.abs(do))[2]
        assert np.max(np.abs(ev - dv)) <= 1e-12 * max(1.0, float(np.max(ev)))
        # the scale bounds the error of the rounded computation
        for g, e, gr in zip(grads, es, _rounded_grads(fb, do, sc)):
            assert np.all(np.abs(gr - g) <= 1.02 * u * (e + np.abs(g)) + 1e-300)


def pin_cand_only_finite_differences():
    """The candidate-only layer's gradients against central differences of the candidate-only
    forward oracle (its own code path, not the fallback layout), every input element."""
    from workloads import make_cand_only_batch
    rng = rng_for(96)
    cb = make_cand_only_batch(rng, "co-fd", hist=[3, 0, 2], cand=[2, 2, 1], H=1, d=3, dtype="f32", scaled=False)
    do = rng.standard_normal(cb.q_cand.shape)
    ins = [np.asarray(x, np.float64).copy() for x in (cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand)]
    got = G.cand_only_attention_backward(*ins, do, cb.hist_offsets, cb.cand_offsets)

    def loss(args):
        return float(np.sum(A.cand_only_attention(*args, cb.hist_offsets, cb.cand_offsets) * do))
    eps = 1e-6
    for i, x in enumerate(ins):
        num = np.zeros_like(x)
        for j in np.ndindex(x.shape):
            xp = [a.copy() for a in ins]; xm = [a.copy() for a in ins]
            xp[i][j] += eps; xm[i][j] -= eps
            num[j] = (loss(xp) - loss(xm)) / (2 * eps)
        assert np.max(np.abs(num - got[i])) <= 1e-6, i


def pin_cand_only_dq_independent_of_history_gradient():
    """A candidate's dq and its own key's and value's gradients are those of the full layer's
    candidate rows whatever output gradient the history rows carry there."""
    from workloads import split_to_cand_only
    rng = rng_for(97)
    fb = make_full_batch(rng, "co-full", prefix=[1, 0], hist=[3, 2], cand=[2, 3], H=2, d=4, dtype="f32",
                         scaled=False)
    do = rng.standard_normal(fb.q.shape)
    full = _grads(fb, do)
    cb = split_to_cand_only(fb)
    cr, hr = cb.meta["cand_rows"], cb.meta["hist_rows"]
    got = G.cand_only_attention_backward(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand, do[cr],
                                         cb.hist_offsets, cb.cand_offsets)
    assert np.max(np.abs(got[0] - full[0][cr])) <= 1e-12
    assert np.max(np.abs(got[3] - full[1][cr])) <= 1e-12 and np.max(np.abs(got[4] - full[2][cr])) <= 1e-12
    # the history keys differ by exactly the history queries' part: zero it in the full layer
    do0 = do.copy(); do0[hr] = 0.0
    full0 = _grads(fb, do0)
    assert np.max(np.abs(got[1] - full0[1][hr])) <= 1e-12 and np.max(np.abs(got[2] - full0[2][hr])) <= 1e-12


def _fallback_layout_here(cb, q_hist_rows):
    """The page's fallback layout of a candidate-only layer, built here row by row (not with
    the oracle's helper): per user [frozen history | candidates] as one full-sequence user.
    History rows get the queries ``q_hist_rows`` (their output gradient is zero, so these
    must not matter).  Returns an object with the full-sequence fields and the row maps."""
    from types import SimpleNamespace
    hoff, coff = np.asarray(cb.hist_offsets), np.asarray(cb.cand_offsets)
    q, k, v, rows_h, rows_c, offsets, cand_start = [], [], [], [], [], [0], []
    for b in range(len(coff) - 1):
        for j in range(int(hoff[b]), int(hoff[b + 1])):
            rows_h.append(len(q))
            q.append(q_hist_rows[j]); k.append(cb.k_hist[j]); v.append(cb.v_hist[j])
        cand_start.append(len(q))
        for j in range(int(coff[b]), int(coff[b + 1])):
            rows_c.append(len(q))
            q.append(cb.q_cand[j]); k.append(cb.k_cand[j]); v.append(cb.v_cand[j])
        offsets.append(len(q))
    shape = (0,) + tuple(np.shape(cb.q_cand)[1:])
    arr = [np.asarray(x, np.float64).reshape((-1,) + shape[1:]) for x in (q, k, v)]
    return SimpleNamespace(q=arr[0], k=arr[1], v=arr[2], offsets=np.asarray(offsets, np.int64),
                           cand_start=np.asarray(cand_start, np.int64), valid=None,
                           attend_padded_history=False, B=len(coff) - 1, H=shape[1], d=shape[2],
                           hr=np.asarray(rows_h, np.int64), cr=np.asarray(rows_c, np.int64))


def pin_cand_only_error_scale():
    """``cand_only_gradient_error_scale`` (the tolerance scale of the five candidate-only
    gradients) against:
     * ``gradient_error_scale`` (pinned above) of the fallback layout built here, with a zero
       output gradient on the history rows and random queries there, taken at the rows each
       gradient belongs to;
     * the triangle inequality against the candidate-only gradients (pinned by finite
       differences);
     * its equality case: with dO >= 0 every product of the history values' gradient has one
       sign, so that scale equals the gradient;
     * the error of candidate-only gradients computed with P, o and dS rounded to bfloat16."""
    from workloads import make_cand_only_batch
    rng = rng_for(98)
    u = 2.0 ** -8
    cb = make_cand_only_batch(rng, "co-err", hist=[4, 0, 3, 2], cand=[2, 3, 1, 0], H=2, d=6, dtype="f32",
                              scaled=False)
    ins = [np.asarray(x, np.float64) for x in (cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand)]
    do = rng.standard_normal(cb.q_cand.shape)
    es = G.cand_only_gradient_error_scale(*ins, do, cb.hist_offsets, cb.cand_offsets)
    grads = G.cand_only_attention_backward(*ins, do, cb.hist_offsets, cb.cand_offsets)
    fl = _fallback_layout_here(cb, rng.standard_normal((cb.Th,) + tuple(cb.q_cand.shape[1:])))
    g_full = np.zeros(fl.q.shape)
    g_full[fl.cr] = do
    eq, ek, ev = G.gradient_error_scale(fl.q, fl.k, fl.v, g_full, fl.offsets, fl.cand_start)
    want = (eq[fl.cr], ek[fl.hr], ev[fl.hr], ek[fl.cr], ev[fl.cr])
    names = ("dq_cand", "dk_hist", "dv_hist", "dk_cand", "dv_cand")
    for name, e, w, g in zip(names, es, want, grads):
        assert e.shape == w.shape, name
        assert np.max(np.abs(e - w), initial=0.0) <= 1e-12 * max(1.0, float(np.max(w, initial=0.0))), name
        assert np.all(e >= np.abs(g) * (1 - 1e-12) - 1e-15), name          # triangle inequality
    # history keys of the user without candidates (the last one) get a zero scale
    last = slice(int(cb.hist_offsets[3]), int(cb.hist_offsets[4]))
    assert np.all(es[1][last] == 0) and np.all(es[2][last] == 0)
    # equality case for the history values' gradient
    e_abs = G.cand_only_gradient_error_scale(*ins, np.abs(do), cb.hist_offsets, cb.cand_offsets)[2]
    dv_abs = G.cand_only_attention_backward(*ins, np.abs(do), cb.hist_offsets, cb.cand_offsets)[2]
    assert np.max(np.abs(e_abs - dv_abs)) <= 1e-12 * max(1.0, float(np.max(e_abs)))
    # the scale bounds the error of the rounded computation, gradient by gradient
    sc = 1.0 / math.sqrt(cb.d)
    gr = _rounded_grads(fl, g_full, sc)
    rounded = (gr[0][fl.cr], gr[1][fl.hr], gr[2][fl.hr], gr[1][fl.cr], gr[2][fl.cr])
    for name, g, e, r in zip(names, grads, es, rounded):
        assert np.all(np.abs(r - g) <= 1.02 * u * (e + np.abs(g)) + 1e-300), name


BWD_PINS = [pin_finite_differences, pin_torch_autograd, pin_lse, pin_closed_forms,
            pin_isolation_of_gradients, pin_error_scale, pin_cand_only_finite_differences,
            pin_cand_only_dq_independent_of_history_gradient,
            pin_cand_only_error_scale]
