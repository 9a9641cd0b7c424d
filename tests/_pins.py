"""Pins for the oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
 * a worked example printed on a page (golden fixtures under tests/golden/),
 * brute force with exactly rounded sums on tiny inputs (written here, from the
   plain-language rule, without segment IDs),
 * a library routine (torch's CPU scaled_dot_product_attention in float64),
 * a closed form, or
 * an invariant stated on the Candidate isolation attention mask page.
They read the oracle's functions through its modules at call time, so
tests/test_oracle_mutations.py can plant a mistake in the oracle and check that
some pin fails.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import attention as A
from oracle import jagged as J
from workloads import make_full_batch, make_cand_only_batch, split_to_cand_only

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_json(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def load_mask_table():
    seg, rows, names, readings = None, [], [], []
    with open(os.path.join(GOLDEN, "mask_table.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "seg":
                seg = np.array([int(x) for x in parts[1:]], dtype=np.int8)
                continue
            names.append(parts[0])
            rows.append([int(x) for x in parts[1:8]])
            readings.append(len(parts) > 8 and parts[8] == "reading")
    return seg, np.array(rows, dtype=bool), names, readings


def rng_for(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------- brute force

def brute_force_full(q, k, v, offsets, cand_start, valid, attend_padded_history, scale):
    """Admitted sets straight from the page's prose: a prefix/history row sees every
    prefix/history row of its own user; a candidate sees those rows and itself; padding
    sees nothing (and, with attend_padded_history, padding before the candidates counts
    as history).  Scores, weights and sums use math.fsum (exactly rounded)."""
    T, H, d = q.shape
    out = np.zeros((T, H, d))
    B = len(offsets) - 1
    for b in range(B):
        lo, hi, cs = int(offsets[b]), int(offsets[b + 1]), int(cand_start[b])

        def real(r):
            return True if valid is None else bool(valid[r])

        def history_row(r):
            return r < cs and (real(r) or attend_padded_history)

        def candidate_row(r):
            return r >= cs and real(r)

        history = [j for j in range(lo, hi) if history_row(j)]
        for i in range(lo, hi):
            if history_row(i):
                keys = history
            elif candidate_row(i):
                keys = history + [i]
            else:
                continue
            for h in range(H):
                s = [scale * math.fsum(float(q[i, h, t]) * float(k[j, h, t]) for t in range(d))
                     for j in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                z = math.fsum(w)
                for t in range(d):
                    out[i, h, t] = math.fsum(wj * float(v[j, h, t]) for wj, j in zip(w, keys)) / z
    return out


def brute_force_cand_only(cb, scale):
    H, d = cb.H, cb.d
    out = np.zeros((cb.Tc, H, d))
    for b in range(cb.B):
        hl, hh = int(cb.hist_offsets[b]), int(cb.hist_offsets[b + 1])
        for i in range(int(cb.cand_offsets[b]), int(cb.cand_offsets[b + 1])):
            keys = [cb.k_hist[j] for j in range(hl, hh)] + [cb.k_cand[i]]
            vals = [cb.v_hist[j] for j in range(hl, hh)] + [cb.v_cand[i]]
            for h in range(H):
                s = [scale * math.fsum(float(cb.q_cand[i, h, t]) * float(kk[h, t]) for t in range(d))
                     for kk in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                z = math.fsum(w)
                for t in range(d):
                    out[i, h, t] = math.fsum(wj * float(vv[h, t]) for wj, vv in zip(w, vals)) / z
    return out


def tiny_batches():
    """Tiny full batches covering: prefix/no prefix, empty users, users without candidates
    or without history, holes from padding, both flag values."""
    rng = rng_for(7)
    out = []
    out.append(make_full_batch(rng, "t-plain", prefix=[1, 0, 2], hist=[2, 3, 0], cand=[2, 1, 3],
                               H=2, d=4, dtype="f32", scaled=False))
    out.append(make_full_batch(rng, "t-empty", prefix=[0, 1, 0, 0], hist=[0, 2, 0, 3], cand=[0, 0, 2, 2],
                               H=1, d=3, dtype="f32", scaled=False))
    for flag in (False, True):
        out.append(make_full_batch(rng, f"t-pad-{flag}", prefix=[1, 1], hist=[1, 3], cand=[2, 2],
                                   pad=[2, 0], H=2, d=4, dtype="bf16", scaled=True,
                                   attend_padded_history=flag))
    holes = np.ones(12, dtype=np.uint8)
    holes[[1, 4, 9]] = 0      # a history hole, a candidate hole, another history hole
    for flag in (False, True):
        out.append(make_full_batch(rng, f"t-holes-{flag}", prefix=[1, 0], hist=[3, 3], cand=[2, 3],
                                   H=1, d=5, dtype="f32", scaled=False, valid=holes,
                                   attend_padded_history=flag))
    return out


# --------------------------------------------------------------------------- pins

def pin_offsets_worked_example():
    g = _load_json("offsets_worked_example.json")
    offs = J.offsets_from_lengths([len(s) for s in g["sequences"]])
    assert list(offs) == g["offsets"], offs
    values = [x for s in g["sequences"] for x in s]
    assert values == g["values"]
    for i, s in enumerate(g["sequences"]):
        assert values[offs[i]:offs[i + 1]] == s
    lo, hi = g["third_sequence_slice"]
    assert (int(offs[2]), int(offs[3])) == (lo, hi)
    assert len(g["sequences"]) * max(len(s) for s in g["sequences"]) == g["dense_positions"]
    assert int(offs[-1]) == g["valid_positions"]


def pin_mask_table():
    seg, table, names, _ = load_mask_table()
    got = A.isolation_mask(seg)
    assert got.shape == table.shape
    bad = np.argwhere(got != table)
    assert bad.size == 0, [(names[i], names[j]) for i, j in bad]
    # the same user, laid out through offsets and the segment rule, gives the same seg
    seg2 = J.segment_ids([0, 7], [4], None, False)
    assert np.array_equal(seg2, seg), seg2


def pin_config1_layout():
    g = _load_json("config1_layout.json")
    B = len(g["hist"])
    lens = [g["prefix"] + g["hist"][b] + g["cand"][b] for b in range(B)]
    offs = J.offsets_from_lengths(lens)
    assert list(offs) == g["offsets"]
    seg = J.segment_ids(g["offsets"], g["cand_start"], None, False)
    assert list(seg) == g["seg"], list(seg)
    bnd = J.bounds(g["offsets"], seg)
    assert [[int(bnd[0, b]), int(bnd[1, b])] for b in range(B)] == g["hist_bounds"]
    assert [[int(bnd[2, b]), int(bnd[3, b])] for b in range(B)] == g["cand_bounds"]
    # with every row valid the flag changes nothing
    assert list(J.segment_ids(g["offsets"], g["cand_start"], None, True)) == g["seg"]


def pin_padded_segments():
    g = _load_json("padded_segments.json")
    T = g["offsets"][-1]
    valid = np.ones(T, dtype=np.uint8)
    valid[g["invalid_rows"]] = 0
    B = len(g["cand_start"])
    for flag, key in ((False, "false"), (True, "true")):
        seg = J.segment_ids(g["offsets"], g["cand_start"], valid, flag)
        assert list(seg) == g["seg_" + key], (flag, list(seg))
        bnd = J.bounds(g["offsets"], seg)
        assert [[int(bnd[0, b]), int(bnd[1, b])] for b in range(B)] == g["hist_bounds_" + key]
        assert [[int(bnd[2, b]), int(bnd[3, b])] for b in range(B)] == g["cand_bounds_" + key]
    # empty users: empty hulls sit at the user's start (history) and end (candidates)
    seg = J.segment_ids([0, 0, 2, 2], [0, 2, 2], None, False)
    bnd = J.bounds([0, 0, 2, 2], seg)
    assert bnd.tolist() == [[0, 0, 2], [0, 2, 2], [0, 2, 2], [0, 2, 2]], bnd.tolist()


def pin_brute_force():
    for fb in tiny_batches():
        sc = 1.0 / math.sqrt(fb.d)
        got = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, fb.valid,
                               fb.attend_padded_history)
        ref = brute_force_full(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, fb.valid,
                               fb.attend_padded_history, sc)
        err = np.max(np.abs(got - ref)) if got.size else 0.0
        assert err <= 1e-12, (fb.name, err)
        # the sampled-row variant agrees with the full one exactly on every row
        rows = np.repeat(np.arange(fb.T), fb.H)
        heads = np.tile(np.arange(fb.H), fb.T)
        part = A.full_attention_rows(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, rows, heads,
                                     fb.valid, fb.attend_padded_history)
        assert np.max(np.abs(part - got[rows, heads])) <= 1e-12, fb.name
    rng = rng_for(11)
    cb = make_cand_only_batch(rng, "t-co", hist=[0, 3, 1], cand=[2, 2, 1], H=2, d=4, dtype="f32",
                              scaled=False)
    got = A.cand_only_attention(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand,
                                cb.hist_offsets, cb.cand_offsets)
    ref = brute_force_cand_only(cb, 0.5)
    assert np.max(np.abs(got - ref)) <= 1e-12


def pin_library_sdpa():
    import torch
    F = torch.nn.functional
    rng = rng_for(13)
    # two-tower user tower: prefix + history only, every row segment 1, plain bidirectional
    fb = make_full_batch(rng, "two-tower", prefix=[2, 0, 1], hist=[5, 7, 1], cand=0, H=3, d=8,
                         dtype="f32", scaled=False)
    got = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start)
    for b in range(fb.B):
        lo, hi = int(fb.offsets[b]), int(fb.offsets[b + 1])
        t = [torch.from_numpy(np.ascontiguousarray(x[lo:hi].transpose(1, 0, 2))).double()
             for x in (fb.q, fb.k, fb.v)]
        ref = F.scaled_dot_product_attention(*t).numpy().transpose(1, 0, 2)
        assert np.max(np.abs(got[lo:hi] - ref)) <= 1e-12, b
    # candidate rows: SDPA over the user's history keys plus the candidate's own key
    fb = make_full_batch(rng, "with-cands", prefix=[1, 3], hist=[4, 2], cand=[3, 2], H=2, d=8,
                         dtype="f32", scaled=False)
    got = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start)
    for b in range(fb.B):
        lo, cs, hi = int(fb.offsets[b]), int(fb.cand_start[b]), int(fb.offsets[b + 1])
        for i in range(cs, hi):
            idx = list(range(lo, cs)) + [i]
            qq = torch.from_numpy(fb.q[i:i + 1].transpose(1, 0, 2).copy()).double()
            kk = torch.from_numpy(fb.k[idx].transpose(1, 0, 2).copy()).double()
            vv = torch.from_numpy(fb.v[idx].transpose(1, 0, 2).copy()).double()
            ref = F.scaled_dot_product_attention(qq, kk, vv).numpy().transpose(1, 0, 2)[0]
            assert np.max(np.abs(got[i] - ref)) <= 1e-12, (b, i)
        # history rows: SDPA over history keys only
        t = [torch.from_numpy(np.ascontiguousarray(x[lo:cs].transpose(1, 0, 2))).double()
             for x in (fb.q, fb.k, fb.v)]
        ref = F.scaled_dot_product_attention(*t).numpy().transpose(1, 0, 2)
        assert np.max(np.abs(got[lo:cs] - ref)) <= 1e-12, b


def pin_closed_forms():
    rng = rng_for(17)
    # (i) a candidate of a user with no prefix and no history reads only itself: o = v_c
    fb = make_full_batch(rng, "no-hist", prefix=[0, 1], hist=[0, 2], cand=[3, 1], H=2, d=4,
                         dtype="f32", scaled=False)
    got = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start)
    assert np.array_equal(got[0:3], fb.v[0:3].astype(np.float64))
    cb = make_cand_only_batch(rng, "co-no-hist", hist=[0, 2], cand=[2, 1], H=1, d=4, dtype="f32",
                              scaled=False)
    got = A.cand_only_attention(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand,
                                cb.hist_offsets, cb.cand_offsets)
    assert np.array_equal(got[0:2], cb.v_cand[0:2].astype(np.float64))
    # (ii) k = 0: history rows average the history values; candidates average history + own
    fb = make_full_batch(rng, "k-zero", prefix=[1, 2], hist=[3, 4], cand=[2, 3], H=2, d=3,
                         dtype="f32", scaled=False)
    fb.k[:] = 0
    got = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start)
    for b in range(fb.B):
        lo, cs, hi = int(fb.offsets[b]), int(fb.cand_start[b]), int(fb.offsets[b + 1])
        n = cs - lo
        for h in range(fb.H):
            for t in range(fb.d):
                col = [float(x) for x in fb.v[lo:cs, h, t]]
                mean_h = math.fsum(col) / n
                assert np.all(np.abs(got[lo:cs, h, t] - mean_h) <= 1e-14)
                for i in range(cs, hi):
                    mean_c = math.fsum(col + [float(fb.v[i, h, t])]) / (n + 1)
                    assert abs(got[i, h, t] - mean_c) <= 1e-14
    # (iii) a user of a single row reads only itself
    fb = make_full_batch(rng, "single", prefix=[1, 0], hist=[0, 1], cand=[0, 0], H=2, d=4,
                         dtype="f32", scaled=False)
    got = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start)
    assert np.array_equal(got, fb.v.astype(np.float64))
    # padding rows output zero
    fb = make_full_batch(rng, "pad-zero", prefix=[1], hist=[2], cand=[2], pad=[3], H=1, d=4,
                         dtype="f32", scaled=False)
    got = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, fb.valid, False)
    assert np.all(got[1:4] == 0.0) and np.all(np.abs(got[[0, 4, 5, 6, 7]]) > 0)


def pin_invariants():
    rng = rng_for(19)
    base = make_full_batch(rng, "inv", prefix=[2, 1, 3], hist=[5, 4, 6], cand=[4, 3, 5], H=2, d=8,
                           dtype="f32", scaled=False)
    o = A.full_attention(base.q, base.k, base.v, base.offsets, base.cand_start)
    # candidate permutation: each candidate's output follows it
    b = 1
    lo, cs, hi = int(base.offsets[b]), int(base.cand_start[b]), int(base.offsets[b + 1])
    perm = np.arange(base.T)
    perm[cs:hi] = cs + rng.permutation(hi - cs)
    o_p = A.full_attention(base.q[perm], base.k[perm], base.v[perm], base.offsets, base.cand_start)
    assert np.max(np.abs(o_p - o[perm])) <= 1e-12
    # removing other candidates of user 1 (keep its first) leaves the kept rows unchanged
    keep = np.r_[0:cs + 1, hi:base.T]
    offs2 = base.offsets.copy()
    offs2[b + 1:] -= (hi - cs - 1)
    cst2 = base.cand_start.copy()
    cst2[b + 1:] -= (hi - cs - 1)
    o_r = A.full_attention(base.q[keep], base.k[keep], base.v[keep], offs2, cst2)
    assert np.max(np.abs(o_r - o[keep])) <= 1e-12
    # adding candidates to user 1 leaves its history rows and old candidates unchanged
    extra = 3
    ins = np.r_[0:hi, [hi - 1] * extra, hi:base.T]
    offs3 = base.offsets.copy()
    offs3[b + 1:] += extra
    cst3 = base.cand_start.copy()
    cst3[b + 1:] += extra
    q3, k3, v3 = base.q[ins].copy(), base.k[ins].copy(), base.v[ins].copy()
    newrows = slice(hi, hi + extra)
    q3[newrows] = rng.standard_normal((extra, base.H, base.d))
    k3[newrows] = rng.standard_normal((extra, base.H, base.d)) * 4
    v3[newrows] = rng.standard_normal((extra, base.H, base.d)) * 100
    o_a = A.full_attention(q3, k3, v3, offs3, cst3)
    old = np.r_[0:hi, hi + extra:base.T + extra]
    assert np.max(np.abs(o_a[old] - o)) <= 1e-12
    # history rows do not depend on candidates (changing every candidate's q, k, v)
    q4, k4, v4 = base.q.copy(), base.k.copy(), base.v.copy()
    for bb in range(base.B):
        s = slice(int(base.cand_start[bb]), int(base.offsets[bb + 1]))
        q4[s] += 3.0
        k4[s] *= -2.0
        v4[s] += 50.0
    o4 = A.full_attention(q4, k4, v4, base.offsets, base.cand_start)
    for bb in range(base.B):
        s = slice(int(base.offsets[bb]), int(base.cand_start[bb]))
        assert np.array_equal(o4[s], o[s])
    # other users: perturbing user 2 leaves users 0 and 1 bit-identical
    q5, k5, v5 = base.q.copy(), base.k.copy(), base.v.copy()
    s2 = slice(int(base.offsets[2]), int(base.offsets[3]))
    q5[s2] *= 7.0
    k5[s2] += 1.0
    v5[s2] = -v5[s2] + 1e3
    o5 = A.full_attention(q5, k5, v5, base.offsets, base.cand_start)
    s01 = slice(0, int(base.offsets[2]))
    assert np.array_equal(o5[s01], o[s01])


def pin_cand_only_equals_full():
    rng = rng_for(23)
    fb = make_full_batch(rng, "co-eq", prefix=[2, 0, 1, 0], hist=[5, 0, 7, 3], cand=[3, 2, 4, 0],
                         H=2, d=8, dtype="f32", scaled=False)
    o_full = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start)
    cb = split_to_cand_only(fb)
    o_co = A.cand_only_attention(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand,
                                 cb.hist_offsets, cb.cand_offsets)
    assert np.max(np.abs(o_co - o_full[cb.meta["cand_rows"]])) <= 1e-12
    rows = np.arange(cb.Tc)
    heads = rows % cb.H
    part = A.cand_only_attention_rows(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand,
                                      cb.hist_offsets, cb.cand_offsets, rows, heads)
    assert np.max(np.abs(part - o_co[rows, heads])) <= 1e-12


ALL_PINS = [pin_offsets_worked_example, pin_mask_table, pin_config1_layout, pin_padded_segments,
            pin_brute_force, pin_library_sdpa, pin_closed_forms, pin_invariants,
            pin_cand_only_equals_full]
