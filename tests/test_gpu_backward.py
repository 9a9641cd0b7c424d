"""GPU parity of the backward pass (rr_attn_plan / rr_attn_run_lse / rr_attn_bwd_run and
rr_attn_bwd) against the float64 oracle's gradients of the same masked attention."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from _gpu import assert_close, assert_close_grad, full_dev, gpu, needs_gpu, rr, to_dev, torch_dtype
from oracle import attention as A
from oracle import backward as BW
from oracle.jagged import segment_ids

pytestmark = [gpu, needs_gpu]


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _train_step(fb, do_seed, scale=None, host=True):
    """Forward with lse, then backward, through the C ABI.  Returns the device tensors (and,
    with ``host``, float64 host copies of o, lse, dq, dk, dv)."""
    dv = full_dev(fb)
    T, H, d = fb.q.shape
    dout = W.draw_output_grad(do_seed, T, H, d, fb.dtype)
    dv["dout"] = to_dev(dout, torch_dtype(fb.dtype))
    ws = rr().rr_attn_plan(dv["offsets"], dv["cand_start"], T, H, d, dv["q"].dtype, dv["valid"],
                           fb.attend_padded_history, backward=True)
    o, lse = rr().rr_attn_run_lse(dv["q"], dv["k"], dv["v"], fb.B, ws, scale=scale)
    dq, dk, dvv = rr().rr_attn_bwd_run(dv["q"], dv["k"], dv["v"], o, dv["dout"], lse, fb.B, ws,
                                       scale=scale)
    torch.cuda.synchronize()
    out = dict(dout=dout, dev=dv, raw=(o, lse, dq, dk, dvv))
    if host:
        out.update(o=_np(o), lse=lse.cpu().numpy().astype(np.float64), dq=_np(dq), dk=_np(dk), dv=_np(dvv))
    return out


def _check_grads(fb, got, what, scale=None):
    args = (fb.q, fb.k, fb.v, got["dout"], fb.offsets, fb.cand_start, fb.valid, fb.attend_padded_history,
            scale)
    ref = BW.full_attention_backward(*args)
    es = BW.gradient_error_scale(*args)
    for name, r, e in zip(("dq", "dk", "dv"), ref, es):
        assert_close_grad(got[name], r, e, f"{what} {name}")
    seg = segment_ids(fb.offsets, fb.cand_start, fb.valid, fb.attend_padded_history)
    for name in ("dq", "dk", "dv"):
        assert not got[name][seg == 0].any(), f"{what} {name}: padding rows not zero"


def _batch(name, d, seed, **kw):
    rng = np.random.default_rng(seed)
    base = dict(prefix=[4, 2, 0, 3, 1], hist=[300, 0, 45, 700, 129], cand=[37, 5, 0, 128, 1], H=3)
    base.update(kw)
    return W.make_full_batch(rng, name, d=d, scaled=False, seed=seed, **base)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_ragged(d):
    """Users with an empty history, no candidates, one candidate, and tails of every size."""
    fb = _batch("bwd-ragged", d, 7000 + d)
    got = _train_step(fb, 7100 + d)
    _check_grads(fb, got, f"ragged d={d}")


@pytest.mark.parametrize("attend", [False, True])
def test_backward_padding_and_holes(attend):
    rng = np.random.default_rng(71)
    fb0 = _batch("bwd-pad", 128, 7200, pad=[0, 3, 20, 0, 64])
    valid = np.ones(fb0.T, np.uint8) if fb0.valid is None else fb0.valid.copy()
    valid[rng.choice(fb0.T, 40, replace=False)] = 0      # holes anywhere, candidates included
    fb = W.FullBatch(**{**fb0.__dict__, "valid": valid, "attend_padded_history": attend})
    got = _train_step(fb, 7300 + int(attend))
    _check_grads(fb, got, f"padding attend={attend}")


def test_lse_matches_oracle():
    for fb in (_batch("lse-bf16", 64, 7400, pad=[0, 0, 5, 0, 9]), W.config1()):
        dv = full_dev(fb)
        T, H, d = fb.q.shape
        ws = rr().rr_attn_plan(dv["offsets"], dv["cand_start"], T, H, d, dv["q"].dtype, dv["valid"],
                               fb.attend_padded_history)
        o, lse = rr().rr_attn_run_lse(dv["q"], dv["k"], dv["v"], fb.B, ws)
        o_plain = rr().rr_attn_run(dv["q"], dv["k"], dv["v"], fb.B, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o_plain), "the lse output changed o"
        ref = BW.attention_lse(fb.q, fb.k, fb.offsets, fb.cand_start, fb.valid, fb.attend_padded_history)
        got = lse.cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref)
        assert np.array_equal(np.isfinite(got), fin) and np.all(got[~fin] == -np.inf)
        err = np.abs(got[fin] - ref[fin]) - (1e-5 + 2e-6 * np.abs(ref[fin]))
        assert float(err.max()) <= 0, f"{fb.name}: lse off by {float(np.abs(got[fin] - ref[fin]).max()):.3e}"


def test_backward_forward_outputs_and_custom_scale():
    fb = _batch("bwd-scale", 64, 7500)
    got = _train_step(fb, 7501, scale=0.05)
    ref_o = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, scale=0.05)
    assert_close(got["o"], ref_o, "bf16", "forward of the backward plan")
    _check_grads(fb, got, "scale 0.05", scale=0.05)


def test_backward_deterministic_and_one_call():
    fb = _batch("bwd-det", 128, 7600)
    a = _train_step(fb, 7601)
    o, lse, dq, dk, dv = a["raw"]
    d = a["dev"]
    for _ in range(2):
        g = rr().rr_attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, d["offsets"], d["cand_start"],
                             d["valid"], fb.attend_padded_history)
        torch.cuda.synchronize()
        for x, y, n in zip(g, (dq, dk, dv), ("dq", "dk", "dv")):
            assert torch.equal(x, y), f"{n} differs between calls"


def test_backward_candidate_order():
    """Permuting one user's candidates permutes every candidate's gradients and every dq
    bit for bit (each depends on its own row and the user's history only)."""
    fb = _batch("bwd-perm", 128, 7700)
    base = _train_step(fb, 7701)
    b = 3
    cs, hi = int(fb.cand_start[b]), int(fb.offsets[b + 1])
    perm = np.arange(fb.T)
    perm[cs:hi] = cs + np.random.default_rng(5).permutation(hi - cs)
    fb2 = W.FullBatch(**{**fb.__dict__, "q": fb.q[perm], "k": fb.k[perm], "v": fb.v[perm]})
    dout = base["dout"][perm]
    dv = full_dev(fb2)
    dv["dout"] = to_dev(dout, torch.bfloat16)
    T, H, d = fb2.q.shape
    ws = rr().rr_attn_plan(dv["offsets"], dv["cand_start"], T, H, d, torch.bfloat16, backward=True)
    o, lse = rr().rr_attn_run_lse(dv["q"], dv["k"], dv["v"], fb2.B, ws)
    g = rr().rr_attn_bwd_run(dv["q"], dv["k"], dv["v"], o, dv["dout"], lse, fb2.B, ws)
    torch.cuda.synchronize()
    dq2, dk2, dv2 = (_np(x) for x in g)
    assert np.array_equal(dq2, base["dq"][perm]), "dq changed with candidate order"
    cand = np.zeros(fb.T, bool)
    for u in range(fb.B):
        cand[int(fb.cand_start[u]):int(fb.offsets[u + 1])] = True
    assert np.array_equal(dk2[cand], base["dk"][perm][cand])
    assert np.array_equal(dv2[cand], base["dv"][perm][cand])


def _one_user(fb, b, h, dout):
    """User b, head h of a batch as a one-user, one-head batch for the oracle: its
    gradients and their error scales."""
    lo, hi = int(fb.offsets[b]), int(fb.offsets[b + 1])
    sl = slice(lo, hi)
    valid = None if fb.valid is None else fb.valid[sl]
    args = (fb.q[sl, h:h + 1], fb.k[sl, h:h + 1], fb.v[sl, h:h + 1], dout[sl, h:h + 1],
            np.array([0, hi - lo], np.int32), np.array([int(fb.cand_start[b]) - lo], np.int32), valid,
            fb.attend_padded_history)
    return BW.full_attention_backward(*args), BW.gradient_error_scale(*args)


@pytest.mark.parametrize("cfg", [3, 5, 6])
def test_backward_full_size_sampled_users(cfg):
    """The lognormal-history batch (d=64), the skew batch and the padded skew batch (d=128,
    wide query tiles) at full size; the oracle checks whole users (every row, one head each):
    the shortest, median and longest history."""
    fb = W.make_config(cfg)
    got = _train_step(fb, 7800 + cfg, host=False)
    _, _, dq, dk, dv = got["raw"]
    order = np.argsort(fb.hist, kind="stable")
    picks = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})
    rng = np.random.default_rng(cfg)
    for b in picks:
        lo, hi = int(fb.offsets[b]), int(fb.offsets[b + 1])
        h = int(rng.integers(0, fb.H))
        ref, es = _one_user(fb, b, h, got["dout"])
        for name, t, r, e in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, es):
            assert_close_grad(_np(t[lo:hi, h:h + 1]), r, e, f"config {cfg} user {b} head {h} {name}")


def test_backward_random_batches():
    """Twelve random small batches (users, lengths, heads, head width 64 or 128, padding
    holes and flag drawn per batch): every gradient against the oracle under the rounding
    bound; for unpadded batches also the candidate-only layer's gradients."""
    rng = np.random.default_rng(2025)
    for i in range(12):
        B = int(rng.integers(1, 8))
        d = int(rng.choice([64, 128]))
        H = int(rng.integers(1, 4))
        P = rng.integers(0, 4, B)
        h = rng.integers(0, 180, B) * (rng.random(B) > 0.2)
        c = rng.integers(0, 140, B) * (rng.random(B) > 0.2)
        holes = bool(rng.random() < 0.3)
        flag = bool(holes and rng.random() < 0.5)
        lens = P + h + c
        valid = (rng.random(int(lens.sum())) > 0.3).astype(np.uint8) if holes else None
        fb = W.make_full_batch(rng, f"bwd-rand{i}", prefix=P, hist=h, cand=c, H=H, d=d, scaled=False,
                               valid=valid, attend_padded_history=flag, seed=9400 + i)
        print(f"[backward random {i}] B={B} T={fb.T} H={H} d={d} holes={holes} flag={flag}", flush=True)
        got = _train_step(fb, 9500 + i)
        _check_grads(fb, got, f"random batch {i}")
        if not holes:
            cb = W.split_to_cand_only(fb)
            dout, grads, _ = _cand_only_train(cb, 9600 + i)
            _check_cand_only(cb, dout, grads, f"random batch {i}, candidate-only")


def _many_users_batch(seed, d=64):
    """More users (2300) than the work-list builder sorts in LDS: the plans keep the user
    order and read the per-user counts back from global memory."""
    rng = np.random.default_rng(seed)
    B = 2300
    P = rng.integers(0, 3, B)
    h = rng.integers(0, 40, B) * (rng.random(B) > 0.1)
    c = rng.integers(0, 6, B) * (rng.random(B) > 0.1)
    h[::97] = 130
    c[::89] = 131
    return W.make_full_batch(rng, f"bwd-many{seed}", prefix=P, hist=h, cand=c, H=2, d=d, scaled=False,
                             seed=seed + 1)


def test_backward_more_users_than_the_lds_sort():
    fb = _many_users_batch(7100)
    print(f"[backward, many users] B={fb.B} T={fb.T}", flush=True)
    got = _train_step(fb, 7102)
    _check_grads(fb, got, f"{fb.B} users")


# ---------------------------------------------------------------- candidate-only layers

def _cand_only_train(cb, do_seed):
    from _gpu import cand_only_dev
    dv = cand_only_dev(cb)
    Tc, H, d = cb.q_cand.shape
    dout = W.draw_output_grad(do_seed, Tc, H, d, cb.dtype)
    dout_d = to_dev(dout, torch_dtype(cb.dtype))
    ws = rr().rr_cand_only_train_plan(dv["hist_offsets"], dv["cand_offsets"], cb.Th, Tc, H, d, dv["q_cand"].dtype)
    o, lse = rr().rr_cand_only_run_lse(dv["q_cand"], dv["k_hist"], dv["v_hist"], dv["k_cand"], dv["v_cand"], cb.B, ws)
    grads = rr().rr_cand_only_bwd_run(dv["q_cand"], dv["k_hist"], dv["v_hist"], dv["k_cand"], dv["v_cand"], o,
                                      dout_d, lse, dv["hist_offsets"], dv["cand_offsets"], ws)
    torch.cuda.synchronize()
    return dout, grads, o


def _check_cand_only(cb, dout, grads, what):
    args = (cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand, dout, cb.hist_offsets, cb.cand_offsets)
    ref = BW.cand_only_attention_backward(*args)
    es = BW.cand_only_gradient_error_scale(*args)
    for name, g, r, e in zip(("dq_cand", "dk_hist", "dv_hist", "dk_cand", "dv_cand"), grads, ref, es):
        assert_close_grad(_np(g), r, e, f"{what} {name}")


@pytest.mark.parametrize("d", [64, 128])
def test_cand_only_backward(d):
    """Every gradient of a candidate-only layer: users with a long history, none, no
    candidates, one candidate; against the oracle under the rounding bound; history keys of
    users without candidates get exactly 0."""
    rng = np.random.default_rng(8000 + d)
    cb = W.make_cand_only_batch(rng, "co-bwd", hist=[300, 0, 45, 700, 129], cand=[37, 6, 0, 128, 1], H=3, d=d,
                                scaled=False, seed=8100 + d)
    dout, grads, _ = _cand_only_train(cb, 8200 + d)
    _check_cand_only(cb, dout, grads, f"cand-only d={d}")
    lo, hi = int(cb.hist_offsets[2]), int(cb.hist_offsets[3])
    assert not _np(grads[1])[lo:hi].any() and not _np(grads[2])[lo:hi].any()
    again = _cand_only_train(cb, 8200 + d)[1]
    for a, b in zip(grads, again):
        assert torch.equal(a, b), "repeated calls differ"


def test_cand_only_backward_matches_full_candidate_rows():
    """A candidate's dq and its own key's and value's gradients are bit for bit those the
    full-sequence backward gives its row (the layer's fallback)."""
    rng = np.random.default_rng(8300)
    fb = W.make_full_batch(rng, "co-vs-full", prefix=[4, 2, 0, 3], hist=[300, 0, 45, 700], cand=[37, 6, 0, 128],
                           H=2, d=128, scaled=False, seed=8301)
    full = _train_step(fb, 8302)
    cb = W.split_to_cand_only(fb)
    cr = cb.meta["cand_rows"]
    from _gpu import cand_only_dev
    dv = cand_only_dev(cb)
    Tc, H, d = cb.q_cand.shape
    dout_d = to_dev(full["dout"][cr], torch.bfloat16)
    ws = rr().rr_cand_only_train_plan(dv["hist_offsets"], dv["cand_offsets"], cb.Th, Tc, H, d, torch.bfloat16)
    o, lse = rr().rr_cand_only_run_lse(dv["q_cand"], dv["k_hist"], dv["v_hist"], dv["k_cand"], dv["v_cand"], cb.B, ws)
    g = rr().rr_cand_only_bwd_run(dv["q_cand"], dv["k_hist"], dv["v_hist"], dv["k_cand"], dv["v_cand"], o, dout_d,
                                  lse, dv["hist_offsets"], dv["cand_offsets"], ws)
    torch.cuda.synchronize()
    assert np.array_equal(_np(o), full["o"][cr])
    assert np.array_equal(_np(g[0]), full["dq"][cr])
    assert np.array_equal(_np(g[3]), full["dk"][cr]) and np.array_equal(_np(g[4]), full["dv"][cr])


def test_cand_only_backward_more_users_than_the_lds_sort():
    cb = W.split_to_cand_only(_many_users_batch(7200, d=128))
    print(f"[candidate-only backward, many users] B={cb.B} Th={cb.Th} Tc={cb.Tc}", flush=True)
    dout, grads, _ = _cand_only_train(cb, 7202)
    _check_cand_only(cb, dout, grads, f"candidate-only, {cb.B} users")


def test_cand_only_backward_config4_sampled_users():
    """The candidate-only workload (B=512, frozen histories up to 4000 rows, 512 candidates
    each, H=8, d=128) at full size; whole users (one head each) against the oracle."""
    cb = W.config4()
    dout, grads, _ = _cand_only_train(cb, 8400)
    hl = np.diff(cb.hist_offsets)
    order = np.argsort(hl, kind="stable")
    rng = np.random.default_rng(4)
    for b in sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])}):
        hs = slice(int(cb.hist_offsets[b]), int(cb.hist_offsets[b + 1]))
        cs = slice(int(cb.cand_offsets[b]), int(cb.cand_offsets[b + 1]))
        h = int(rng.integers(0, cb.H))
        sub = [x[s, h:h + 1] for x, s in ((cb.q_cand, cs), (cb.k_hist, hs), (cb.v_hist, hs), (cb.k_cand, cs),
                                           (cb.v_cand, cs))]
        args = (*sub, dout[cs, h:h + 1], [0, hs.stop - hs.start], [0, cs.stop - cs.start])
        ref = BW.cand_only_attention_backward(*args)
        es = BW.cand_only_gradient_error_scale(*args)
        for name, gt, s, r, e in zip(("dq_cand", "dk_hist", "dv_hist", "dk_cand", "dv_cand"), grads,
                                     (cs, hs, hs, cs, cs), ref, es):
            assert_close_grad(_np(gt[s, h:h + 1]), r, e, f"config 4 user {b} head {h} {name}")
