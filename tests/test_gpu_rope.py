"""GPU parity of the right-anchored rotary encoding (rr_rope_positions, rr_rope_qk) and of
rotary attention (rr_rope_qk then rr_attn_fwd / rr_cand_only_attn_fwd) against the oracle."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import workloads as W
from _gpu import (assert_close, cand_only_dev, full_dev, gpu, needs_gpu, rr, run_cand_only, run_full,
                  sample_full_rows, to_dev)
from oracle import attention as A
from oracle import rotary as R

pytestmark = [gpu, needs_gpu]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rope_dev(q, k, offsets, cand_start, pos_base=None, base=None):
    qo, ko = rr().rr_rope_qk(q, k, offsets, cand_start, pos_base=pos_base, theta_base=base)
    torch.cuda.synchronize()
    return qo, ko


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_positions_bit_exact():
    with open(os.path.join(GOLDEN, "rope_positions.json"), encoding="utf-8") as f:
        cases = json.load(f)["cases"]
    for c in cases:
        base = None if c["pos_base"] is None else to_dev(np.array(c["pos_base"], np.int32))
        got = rr().rr_rope_positions(to_dev(np.array(c["offsets"], np.int32)),
                                     to_dev(np.array(c["cand_start"], np.int32)), len(c["positions"]),
                                     pos_base=base)
        assert got.cpu().numpy().tolist() == c["positions"], c["name"]
    for fb in (W.config3(), W.config5_padded(attend_padded_history=False)):
        got = rr().rr_rope_positions(to_dev(fb.offsets), to_dev(fb.cand_start), fb.T).cpu().numpy()
        assert np.array_equal(got, R.right_anchored_positions(fb.offsets, fb.cand_start)), fb.name


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 64, 128])
def test_rotation_values(dtype, d):
    rng = np.random.default_rng(11 + d)
    fb = W.make_full_batch(rng, "rope-vals", prefix=4, hist=[0, 9000, 37, 600], cand=[5, 70, 1, 300],
                           H=3, d=d, dtype=dtype, scaled=False, seed=500 + d)
    dv = full_dev(fb)
    qo, ko = _rope_dev(dv["q"], dv["k"], dv["offsets"], dv["cand_start"])
    pos = R.right_anchored_positions(fb.offsets, fb.cand_start)
    for name, got, x in (("q", qo, fb.q), ("k", ko, fb.k)):
        ref = R.rope(x, pos)
        g = _np(got)
        if dtype == "f32":
            err = float(np.max(np.abs(g - ref)))
            assert err <= 2e-6, f"{name}: fp32 rotation max|err| {err:.3e}"
        else:   # one rounding to bf16 of a float rotation: within one ulp (2^-7 relative)
            ex = np.abs(g - ref) - (2.0 ** -7) * np.abs(ref) - 1e-5
            assert float(ex.max()) <= 0, f"{name}: bf16 rotation off by more than one rounding"
    # in place gives the same bits; q alone and k alone give the same bits
    q2, k2 = dv["q"].clone(), dv["k"].clone()
    rr().rr_rope_qk(q2, k2, dv["offsets"], dv["cand_start"], in_place=True)
    qa, _ = rr().rr_rope_qk(dv["q"], None, dv["offsets"], dv["cand_start"])
    _, kb = rr().rr_rope_qk(None, dv["k"], dv["offsets"], dv["cand_start"])
    torch.cuda.synchronize()
    assert torch.equal(q2, qo) and torch.equal(k2, ko) and torch.equal(qa, qo) and torch.equal(kb, ko)


def _rope_attention(fb, base=None):
    dv = full_dev(fb)
    dv["q"], dv["k"] = _rope_dev(dv["q"], dv["k"], dv["offsets"], dv["cand_start"], base=base)
    return run_full(fb, dv)


def test_config1_rope_attention_fp32():
    fb = W.config1()
    got = _rope_attention(fb)
    ref = R.full_attention_rope(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start)
    assert_close(got, ref, "f32", "config 1 with rotary q/k")


@pytest.mark.parametrize("d", [64, 128])
def test_rope_attention_bf16(d):
    rng = np.random.default_rng(21 + d)
    fb = W.make_full_batch(rng, "rope-attn", prefix=[4, 2, 0, 3], hist=[700, 90, 0, 2100],
                           cand=[300, 40, 5, 129], H=4, d=d, seed=600 + d)
    got = _rope_attention(fb, base=500.0)
    ref = R.full_attention_rope(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, base=500.0)
    assert_close(got, ref, "bf16", f"rotary attention d={d}")


def test_rope_attention_config3_sampled():
    fb = W.config3()
    got = _rope_attention(fb)
    rows, heads = sample_full_rows(fb, per_user=2, seed=7)
    pos = R.right_anchored_positions(fb.offsets, fb.cand_start)
    ref = A.full_attention_rows(R.rope(fb.q, pos), R.rope(fb.k, pos), fb.v, fb.offsets, fb.cand_start,
                                rows, heads)
    assert_close(got[rows, heads], ref, "bf16", "config 3 with rotary q/k, sampled")


@pytest.mark.parametrize("cfg", [2, 5])
def test_rope_step_full_size_sampled(cfg):
    """The rotary step in the form the benchmark times it -- keys rotated by rr_rope_qk, queries
    inside rr_attn_fwd_rope -- on the short-history and skew batches at full size: every
    output bit-identical to rotating q and k first and running rr_attn_fwd, and sampled rows
    against the rotary oracle."""
    fb = W.make_config(cfg)
    dv = full_dev(fb)
    _, k_rot = _rope_dev(None, dv["k"], dv["offsets"], dv["cand_start"])
    q_rot, _ = _rope_dev(dv["q"], None, dv["offsets"], dv["cand_start"])
    fused = rr().rr_attn_fwd_rope(dv["q"], k_rot, dv["v"], dv["offsets"], dv["cand_start"])
    two_pass = rr().rr_attn_fwd(q_rot, k_rot, dv["v"], dv["offsets"], dv["cand_start"])
    torch.cuda.synchronize()
    assert torch.equal(fused, two_pass), f"config {cfg}: in-kernel rotation differs from the rotary pass"
    rows, heads = sample_full_rows(fb, 2, seed=cfg)
    pos = R.right_anchored_positions(fb.offsets, fb.cand_start)
    ref = A.full_attention_rows(R.rope(fb.q, pos), R.rope(fb.k, pos), fb.v, fb.offsets, fb.cand_start, rows, heads)
    assert_close(_np(fused)[rows, heads], ref, "bf16", f"config {cfg} rotary step, sampled")


def test_rope_candidates_interchangeable_bit_identical():
    rng = np.random.default_rng(31)
    fb = W.make_full_batch(rng, "rope-perm", prefix=[4, 2, 0, 3], hist=[700, 90, 0, 260],
                           cand=[300, 40, 5, 129], H=4, d=128, seed=3131)
    base = _rope_attention(fb)
    b = 0
    cs, hi = int(fb.cand_start[b]), int(fb.offsets[b + 1])
    perm = np.arange(fb.T)
    perm[cs:hi] = cs + np.random.default_rng(5).permutation(hi - cs)
    fb2 = W.FullBatch(**{**fb.__dict__, "q": fb.q[perm], "k": fb.k[perm], "v": fb.v[perm]})
    assert np.array_equal(_rope_attention(fb2), base[perm]), "candidate order changed outputs"


def test_rope_cand_only_equals_full_rows():
    rng = np.random.default_rng(41)
    fb = W.make_full_batch(rng, "rope-co", prefix=[4, 2, 0, 3], hist=[700, 90, 0, 260],
                           cand=[300, 40, 5, 129], H=4, d=128, seed=4141)
    full = _rope_attention(fb)
    cb = W.split_to_cand_only(fb)
    dv = cand_only_dev(cb)
    hoff, coff = dv["hist_offsets"], dv["cand_offsets"]
    hist_len = (hoff[1:] - hoff[:-1]).contiguous()
    _, dv["k_hist"] = _rope_dev(None, dv["k_hist"], hoff, hoff[1:].contiguous())
    dv["q_cand"], dv["k_cand"] = _rope_dev(dv["q_cand"], dv["k_cand"], coff, coff[:-1].contiguous(),
                                           pos_base=hist_len)
    co = run_cand_only(cb, dv)
    assert np.array_equal(co, full[cb.meta["cand_rows"]])
    ref = R.cand_only_attention_rope(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand,
                                     cb.hist_offsets, cb.cand_offsets)
    assert_close(co, ref, "bf16", "candidate-only layer with rotary q/k")


# ---------------------------------------------------------------- queries rotated inside the attention


@pytest.mark.parametrize("d,wide,H", [(32, False, 3), (64, False, 3), (128, False, 3), (64, True, 2), (128, True, 2),
                                      (128, True, 32)])
def test_fused_query_rotation_equals_the_rotary_pass(d, wide, H):
    """rr_attn_fwd_rope (q rotated in the kernel's registers) gives the same bits as
    rr_rope_qk followed by rr_attn_fwd, on the in-kernel-plan path and the separate plan,
    narrow and wide tiles; and it matches the rotary oracle.  With 32 heads the wide batch
    is planned separately in every call, so the rotating kernel also runs with the key-norm
    bound (its bound taken from the rotated queries)."""
    rng = np.random.default_rng(600 + d + wide + H)
    if wide:
        fb = W.make_full_batch(rng, "rope-fused-wide", prefix=[3, 1], hist=[3000, 2200], cand=[1500, 2100], H=H, d=d,
                               seed=610 + d + H)
    else:
        fb = W.make_full_batch(rng, "rope-fused", prefix=[4, 0, 2, 1], hist=[700, 0, 57, 260], cand=[33, 9, 0, 129],
                               H=H, d=d, seed=620 + d)
    assert (fb.T >= 2048 * fb.B) == wide
    dv = full_dev(fb)
    base = 500.0
    _, k_rot = _rope_dev(None, dv["k"], dv["offsets"], dv["cand_start"], base=base)
    q_rot, _ = _rope_dev(dv["q"], None, dv["offsets"], dv["cand_start"], base=base)
    fused = rr().rr_attn_fwd_rope(dv["q"], k_rot, dv["v"], dv["offsets"], dv["cand_start"], theta_base=base)
    two_pass = rr().rr_attn_fwd(q_rot, k_rot, dv["v"], dv["offsets"], dv["cand_start"])
    ws = rr().rr_attn_plan(dv["offsets"], dv["cand_start"], fb.T, fb.H, fb.d, dv["q"].dtype)
    planned = rr().rr_attn_run(q_rot, k_rot, dv["v"], fb.B, ws)
    torch.cuda.synchronize()
    assert torch.equal(fused, two_pass), "fused rotation differs from the rotary pass"
    assert torch.equal(fused, planned)
    rows, heads = sample_full_rows(fb, 8, seed=d)
    pos = R.right_anchored_positions(fb.offsets, fb.cand_start)
    qr, kr = R.rope(fb.q, pos, base), R.rope(fb.k, pos, base)
    ref = A.full_attention_rows(qr, kr, fb.v, fb.offsets, fb.cand_start, rows, heads)
    assert_close(_np(fused)[rows, heads], ref, "bf16", "fused rotary attention")


@pytest.mark.parametrize("d", [64, 128])
def test_fused_query_rotation_candidate_only(d):
    """rr_cand_only_attn_fwd_rope: candidates rotated in the kernel at their user's history
    length; equal bit for bit to rr_rope_qk + rr_cand_only_attn_fwd and to the fused
    full-sequence layer's candidate rows."""
    rng = np.random.default_rng(650 + d)
    fb = W.make_full_batch(rng, "rope-fused-co", prefix=[2, 0, 1], hist=[400, 0, 90], cand=[64, 7, 130], H=2, d=d,
                           seed=660 + d)
    cb = W.split_to_cand_only(fb)
    dc = cand_only_dev(cb)
    hlen = (dc["hist_offsets"][1:] - dc["hist_offsets"][:-1]).contiguous()
    _, kh = _rope_dev(None, dc["k_hist"], dc["hist_offsets"], dc["hist_offsets"][1:].contiguous())
    qc, kc = _rope_dev(dc["q_cand"], dc["k_cand"], dc["cand_offsets"], dc["cand_offsets"][:-1].contiguous(),
                       pos_base=hlen)
    fused = rr().rr_cand_only_attn_fwd_rope(dc["q_cand"], kh, dc["v_hist"], kc, dc["v_cand"], dc["hist_offsets"],
                                            dc["cand_offsets"])
    two_pass = rr().rr_cand_only_attn_fwd(qc, kh, dc["v_hist"], kc, dc["v_cand"], dc["hist_offsets"],
                                          dc["cand_offsets"])
    dv = full_dev(fb)
    _, k_rot = _rope_dev(None, dv["k"], dv["offsets"], dv["cand_start"])
    full = rr().rr_attn_fwd_rope(dv["q"], k_rot, dv["v"], dv["offsets"], dv["cand_start"])
    torch.cuda.synchronize()
    assert torch.equal(fused, two_pass)
    assert torch.equal(fused, full[torch.from_numpy(cb.meta["cand_rows"]).to(full.device)])
    ref = R.cand_only_attention_rope(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand, cb.hist_offsets,
                                     cb.cand_offsets)
    assert_close(_np(fused), ref, "bf16", "fused rotary candidate-only attention")
