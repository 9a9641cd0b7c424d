"""Seeded random sweep over the shapes the fixed GPU cases do not reach: up to 80 users, up to 8
heads, head widths 16-128, history lengths log-uniform up to 2500 with empty users, up to 400
candidates, padding holes with both flag values, and batches long enough for the wide query
tile.  Per batch: every element of the full-sequence output against the oracle; the separately
planned launch bit-identical to the one-call path; for unpadded batches the candidate-only layer
against the oracle and bit for bit against the full rows, and the in-kernel query rotation bit
for bit against the rotary pass plus sampled rows against the rotary oracle; for the cheaper
bf16 batches at d 64 and 128 the backward gradients (both layer kinds) under the rounding bound.
A second sweep takes only batches of a few long users (the wide query tile, where planned runs
bound the scores by the key norms), with unscaled q and k in about half of them."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W
from _gpu import assert_close, full_dev, gpu, needs_gpu, rr, run_cand_only, run_full, sample_full_rows
from oracle import attention as A
from oracle import rotary as R
from test_gpu_backward import _cand_only_train, _check_cand_only, _check_grads, _train_step

pytestmark = [gpu, needs_gpu]

N_CASES = 120
SEED = 77000
MAX_COST = 2.5e9       # sum over users of L^2 * H * d, so the oracle finishes each batch in about a second
MAX_BWD_COST = 8e8


def _case(i):
    rng = np.random.default_rng(SEED + i)
    if rng.random() < 0.12:   # few long users: the wide tile
        B = int(rng.integers(1, 4))
        P, h, c = rng.integers(0, 6, B), rng.integers(1500, 3200, B), rng.integers(600, 1400, B)
        H = int(rng.integers(1, 3))
    else:
        B = int(rng.integers(1, 81))
        P = rng.integers(0, 9, B)
        h = np.exp(rng.uniform(0, np.log(2500), B)).astype(np.int64) * (rng.random(B) > 0.1)
        c = rng.integers(0, 400, B) * (rng.random(B) > 0.1)
        H = int(rng.integers(1, 9))
    d = int(rng.choice([32, 64, 128, 16])) if rng.random() < 0.9 else 128
    dtype = "f32" if (d == 16 or rng.random() < 0.15) else "bf16"
    L = P + h + c
    cost = float((L.astype(np.float64) ** 2).sum()) * H * d
    while cost > MAX_COST:
        h, c = h // 2, c // 2
        L = P + h + c
        cost = float((L.astype(np.float64) ** 2).sum()) * H * d
    holes = bool(rng.random() < 0.25)
    flag = bool(holes and rng.random() < 0.5)
    valid = (rng.random(int(L.sum())) > 0.3).astype(np.uint8) if holes else None
    fb = W.make_full_batch(rng, f"sweep{i}", prefix=P, hist=h, cand=c, H=H, d=d, dtype=dtype,
                           scaled=(dtype == "bf16"), valid=valid, attend_padded_history=flag,
                           seed=SEED + 10_000 + i)
    base = float(rng.choice([500.0, 10000.0]))
    return fb, holes, cost, base


N_WIDE = 24
WIDE_SEED = 95000
MAX_WIDE_COST = 1e10


def _wide_case(i):
    """A few long users (the wide query tile), bf16, with q and k unscaled in about half the
    batches: larger scores move rows' references over more key tiles, so the waves leave the
    tile-maximum loop for the key-norm-bounded loop at varied points."""
    rng = np.random.default_rng(WIDE_SEED + i)
    B = int(rng.integers(1, 4))
    P, h, c = rng.integers(0, 6, B), rng.integers(1500, 3200, B), rng.integers(200, 1400, B)
    H = int(rng.integers(1, 3))
    d = int(rng.choice([32, 64, 128]))
    L = P + h + c
    cost = float((L.astype(np.float64) ** 2).sum()) * H * d
    while cost > MAX_WIDE_COST:
        h, c = (h * 3) // 4, (c * 3) // 4
        L = P + h + c
        cost = float((L.astype(np.float64) ** 2).sum()) * H * d
    holes = bool(rng.random() < 0.3)
    flag = bool(holes and rng.random() < 0.5)
    valid = (rng.random(int(L.sum())) > 0.3).astype(np.uint8) if holes else None
    fb = W.make_full_batch(rng, f"sweep-wide{i}", prefix=P, hist=h, cand=c, H=H, d=d, dtype="bf16",
                           scaled=bool(rng.random() < 0.5), valid=valid, attend_padded_history=flag,
                           seed=WIDE_SEED + 1_000 + i)
    return fb, holes, cost, float(rng.choice([500.0, 10000.0]))


def test_random_sweep():
    for i in range(N_CASES):
        _check_case(i, i, *_case(i))


def test_random_wide_sweep():
    for i in range(N_WIDE):
        _check_case(f"wide {i}", i, *_wide_case(i))


def _check_case(label, k, fb, holes, cost, base):
    """Every check of one batch; ``k`` offsets the seeds of the sampled rows and gradients."""
    dtype, d, flag = fb.dtype, fb.d, fb.attend_padded_history
    print(f"[sweep {label}] B={fb.B} T={fb.T} H={fb.H} d={d} {dtype} holes={holes} flag={flag} "
          f"wide={fb.T >= 2048 * fb.B}", flush=True)
    dv = full_dev(fb)
    full = run_full(fb, dv)
    ref = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, fb.valid, flag)
    assert_close(full, ref, dtype, f"sweep {label}")
    mfma = dtype == "bf16" and d >= 32
    if mfma:
        ws = rr().rr_attn_plan(dv["offsets"], dv["cand_start"], fb.T, fb.H, d, dv["q"].dtype, dv["valid"], flag)
        planned = rr().rr_attn_run(dv["q"], dv["k"], dv["v"], fb.B, ws)
        torch.cuda.synchronize()
        assert np.array_equal(planned.float().cpu().numpy().astype(np.float64), full), f"sweep {label}: planned"
    if not holes:
        cb = W.split_to_cand_only(fb)
        co = run_cand_only(cb)
        cref = A.cand_only_attention(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand, cb.hist_offsets,
                                     cb.cand_offsets)
        assert_close(co, cref, dtype, f"sweep {label}, candidate-only")
        if mfma:
            assert np.array_equal(co, full[cb.meta["cand_rows"]]), f"sweep {label}: candidate-only rows"
            _, k_rot = rr().rr_rope_qk(None, dv["k"], dv["offsets"], dv["cand_start"], theta_base=base)
            q_rot, _ = rr().rr_rope_qk(dv["q"], None, dv["offsets"], dv["cand_start"], theta_base=base)
            fused = rr().rr_attn_fwd_rope(dv["q"], k_rot, dv["v"], dv["offsets"], dv["cand_start"],
                                          theta_base=base)
            two = rr().rr_attn_fwd(q_rot, k_rot, dv["v"], dv["offsets"], dv["cand_start"])
            torch.cuda.synchronize()
            assert torch.equal(fused, two), f"sweep {label}: in-kernel rotation"
            if fb.T:
                rows, heads = sample_full_rows(fb, 6, seed=k)
                pos = R.right_anchored_positions(fb.offsets, fb.cand_start)
                rref = A.full_attention_rows(R.rope(fb.q, pos, base), R.rope(fb.k, pos, base), fb.v,
                                             fb.offsets, fb.cand_start, rows, heads)
                got = fused.float().cpu().numpy().astype(np.float64)[rows, heads]
                assert_close(got, rref, "bf16", f"sweep {label}, rotary")
    if d in (64, 128) and dtype == "bf16" and cost < MAX_BWD_COST:
        got = _train_step(fb, SEED + 20_000 + k)
        _check_grads(fb, got, f"sweep {label} backward")
        if not holes:
            cb = W.split_to_cand_only(fb)
            dout, grads, _ = _cand_only_train(cb, SEED + 30_000 + k)
            _check_cand_only(cb, dout, grads, f"sweep {label} candidate-only backward")
