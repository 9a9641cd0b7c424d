"""Pins for the rotary-position oracle (oracle/rotary.py).

Each ``pin_*`` raises AssertionError when the oracle disagrees with
 * the positions derived by hand from the page (tests/golden/rope_positions.json),
 * rotations written as complex multiplications with angles fixed by hand (base 16 and
   d = 8 give frequencies 1, 1/2, 1/4, 1/8 exactly; d = 4, base 10000 gives 1 and 1/100),
 * properties every rotary encoding has (isometry, identity at position 0, scores that
   depend only on position differences),
 * a brute-force attention over hand-rotated q and k on a tiny batch (math.fsum), or
 * the page's claims: candidates are interchangeable, and a candidate-only layer equals
   the full layer's candidate rows.
They call the oracle through its module at call time, so tests can plant mistakes.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import attention as A
from oracle import rotary as R
from workloads import make_full_batch, split_to_cand_only

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _hand_rotate(x, angles):
    """x [T, H, d] rotated pairwise as complex numbers z_i = x_2i + j x_2i+1 times e^{j angle}."""
    x = np.asarray(x, dtype=np.float64)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * np.exp(1j * np.asarray(angles, dtype=np.float64))[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def pin_positions_golden():
    with open(os.path.join(GOLDEN, "rope_positions.json"), encoding="utf-8") as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = R.right_anchored_positions(c["offsets"], c["cand_start"], c["pos_base"])
        assert got.tolist() == c["positions"], c["name"]


def pin_rotation_by_hand():
    rng = _rng(71)
    pos = np.array([0, 1, 3, 7, 250])
    x = rng.standard_normal((len(pos), 3, 8))
    hand = pos[:, None] * np.array([1.0, 0.5, 0.25, 0.125])[None, :]    # 16^(-2i/8) = 2^-i
    assert np.max(np.abs(R.rope(x, pos, base=16.0) - _hand_rotate(x, hand))) <= 1e-12
    x4 = rng.standard_normal((len(pos), 2, 4))
    hand4 = pos[:, None] * np.array([1.0, 0.01])[None, :]                # 10000^(-2/4) = 1/100
    assert np.max(np.abs(R.rope(x4, pos) - _hand_rotate(x4, hand4))) <= 1e-12
    # d = 2: the unit vector (1, 0) at position p goes to (cos p, sin p) for any base
    e = np.zeros((3, 1, 2)); e[:, 0, 0] = 1.0
    p = np.array([0, 2, 5])
    got = R.rope(e, p, base=123.0)
    assert np.max(np.abs(got[:, 0, 0] - np.cos(p))) <= 1e-15
    assert np.max(np.abs(got[:, 0, 1] - np.sin(p))) <= 1e-15


def pin_rotation_properties():
    rng = _rng(72)
    x = rng.standard_normal((6, 2, 16))
    pos = np.array([0, 0, 9, 40, 1000, 12345])
    y = R.rope(x, pos)
    assert np.array_equal(y[:2], x[:2]), "position 0 must leave a row unchanged"
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.max(np.abs(n0 - n1) / (1 + n0)) <= 1e-12, "each pair keeps its length"
    # scores depend on position differences only
    q = rng.standard_normal((1, 1, 16)); k = rng.standard_normal((1, 1, 16))
    s = [float(np.sum(R.rope(q, [a + t]) * R.rope(k, [b + t]))) for (a, b, t) in
         [(5, 2, 0), (5, 2, 100), (5, 2, 3000)]]
    assert max(s) - min(s) <= 1e-9
    s2 = float(np.sum(R.rope(q, [6]) * R.rope(k, [2])))
    assert abs(s2 - s[0]) > 1e-6, "a different offset must change the score"


def _tiny_batch(seed, d=8, H=2):
    rng = _rng(seed)
    return make_full_batch(rng, "rope-tiny", prefix=[1, 0, 2], hist=[3, 2, 0], cand=[3, 1, 2], H=H, d=d,
                           dtype="f32", scaled=False, seed=seed)


def pin_brute_force():
    """Attention over hand-rotated q and k (v unrotated), each output an exactly rounded
    sum, against the oracle's composition, with base 16 and d = 8."""
    fb = _tiny_batch(73)
    pos = np.asarray(R.right_anchored_positions(fb.offsets, fb.cand_start))
    ang = pos[:, None] * np.array([1.0, 0.5, 0.25, 0.125])[None, :]
    q, k = _hand_rotate(fb.q, ang), _hand_rotate(fb.k, ang)
    v = np.asarray(fb.v, np.float64)
    sc = 1.0 / math.sqrt(fb.d)
    want = np.zeros_like(v)
    for b in range(fb.B):
        lo, cs, hi = int(fb.offsets[b]), int(fb.cand_start[b]), int(fb.offsets[b + 1])
        for r in range(lo, hi):
            keys = list(range(lo, cs)) + ([r] if r >= cs else [])
            for h in range(fb.H):
                s = [sc * math.fsum(q[r, h] * k[j, h]) for j in keys]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for c in range(fb.d):
                    want[r, h, c] = math.fsum(e[i] * v[j, h, c] for i, j in enumerate(keys)) / tot
    got = R.full_attention_rope(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, base=16.0)
    assert np.max(np.abs(got - want)) <= 1e-12


def pin_candidates_interchangeable():
    """[Isolation] §位置编码: with right-anchored positions and the isolation mask,
    reordering, adding or removing candidates leaves every other output unchanged."""
    rng = _rng(74)
    fb = make_full_batch(rng, "rope-perm", prefix=[2, 1], hist=[5, 3], cand=[6, 4], H=2, d=8,
                         dtype="f32", scaled=False, seed=74)
    base = R.full_attention_rope(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start)
    cs, hi = int(fb.cand_start[0]), int(fb.offsets[1])
    perm = np.arange(fb.T)
    perm[cs:hi] = cs + _rng(5).permutation(hi - cs)
    got = R.full_attention_rope(fb.q[perm], fb.k[perm], fb.v[perm], fb.offsets, fb.cand_start)
    assert np.max(np.abs(got - base[perm])) <= 1e-12, "candidate order changed outputs"
    keep = np.r_[0:cs + 2, hi:fb.T]
    drop = hi - cs - 2
    off = fb.offsets.copy(); off[1:] -= drop
    cst = fb.cand_start.copy(); cst[1:] -= drop
    got = R.full_attention_rope(fb.q[keep], fb.k[keep], fb.v[keep], off, cst)
    assert np.max(np.abs(got - base[keep])) <= 1e-12, "removing candidates changed outputs"


def pin_cand_only_equals_full():
    rng = _rng(75)
    fb = make_full_batch(rng, "rope-co", prefix=[2, 0, 1], hist=[4, 3, 0], cand=[3, 2, 2], H=2, d=8,
                         dtype="f32", scaled=False, seed=75)
    full = R.full_attention_rope(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start)
    cb = split_to_cand_only(fb)
    co = R.cand_only_attention_rope(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand,
                                    cb.hist_offsets, cb.cand_offsets)
    assert np.max(np.abs(co - full[cb.meta["cand_rows"]])) <= 1e-12


ROPE_PINS = [pin_positions_golden, pin_rotation_by_hand, pin_rotation_properties, pin_brute_force,
             pin_candidates_interchangeable, pin_cand_only_equals_full]
