"""Tile-shape independence and sentinel tests on the GPU.

The library picks the query-tile height of an attention launch from the batch's average
rows per user (128-row tiles for short users, 256-row tiles from 2048 rows per user on
average), so one user's tile shape depends on its batch-mates.  The candidate isolation
attention mask page (section "核心结论") makes a candidate's score a function of its own
user's rows alone, which is what lets scores be cached across requests; here that is
required bit for bit: a long user run alone (wide tiles) gives the same outputs as the
same user inside a batch of many short users (narrow tiles), in full-sequence mode, in
candidate-only mode and through the layer stack's cached request.

The sentinel tests put +1e3 in the values of every key a query must not read (other
candidates, padding under attend_padded_history=False, other users' rows, other users'
frozen history in candidate-only mode) on the wide-tile path, padded and not, and in
candidate-only mode on both tile shapes, and compare every output with the oracle: a leak
of one such key moves an output by about 1e3 / (keys read), far outside the tolerance.
"""
import numpy as np
import pytest
import torch

import workloads as W
from _gpu import (assert_close, cand_only_dev, full_dev, gpu, needs_gpu, rr, run_cand_only, run_full, to_dev)
from oracle import attention as A

pytestmark = [gpu, needs_gpu]

WIDE_ROWS = 2048     # average rows per user from which the library takes the 256-row tiles


def _log(msg):
    print(msg, flush=True)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _planned(fb, dev, scale=None):
    """plan + run (the separate planning launch) of a full-sequence batch."""
    ws = rr().rr_attn_plan(dev["offsets"], dev["cand_start"], fb.T, fb.H, fb.d, dev["q"].dtype,
                           valid=dev["valid"], attend_padded_history=fb.attend_padded_history)
    out = rr().rr_attn_run(dev["q"], dev["k"], dev["v"], fb.B, ws, scale=scale)
    torch.cuda.synchronize()
    return _np(out)


def _long_and_short(d, H, seed, long_user, short_users=40):
    """The long user alone, and the same user (same values) first in a batch of short users."""
    rng = np.random.default_rng(seed)
    P, h, c = long_user
    alone = W.make_full_batch(rng, "long-alone", prefix=[P], hist=[h], cand=[c], H=H, d=d, seed=seed)
    sp = rng.integers(0, 4, short_users)
    sh = rng.integers(0, 60, short_users)
    scnd = rng.integers(0, 12, short_users)
    short = W.make_full_batch(rng, "short", prefix=sp, hist=sh, cand=scnd, H=H, d=d, seed=seed + 1)
    L = alone.T
    batch = W.make_full_batch(rng, "mixed", prefix=np.r_[P, sp], hist=np.r_[h, sh], cand=np.r_[c, scnd], H=H, d=d,
                              seed=seed + 2)
    batch = W.FullBatch(**{**batch.__dict__, "q": np.concatenate([alone.q, short.q]),
                           "k": np.concatenate([alone.k, short.k]), "v": np.concatenate([alone.v, short.v])})
    assert alone.T >= WIDE_ROWS * alone.B, "the lone user must take the wide tiles"
    assert batch.T < WIDE_ROWS * batch.B, "the batch must take the narrow tiles"
    return alone, batch, L


@pytest.mark.parametrize("d", [32, 64, 128])
def test_wide_equals_narrow_full_mode(d):
    alone, batch, L = _long_and_short(d, 3, 700 + d, (4, 2500, 700))
    _log(f"[tiles full] d={d} alone T={alone.T} batch B={batch.B} T={batch.T}")
    da, db = full_dev(alone), full_dev(batch)
    outs = [run_full(alone, da), _planned(alone, da), run_full(batch, db)[:L], _planned(batch, db)[:L]]
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(o, outs[0]), f"variant {i} differs from the lone user's wide-tile output"
    rows = np.r_[0:8, 2000:2010, alone.T - 8:alone.T]
    heads = np.arange(len(rows)) % alone.H
    ref = A.full_attention_rows(alone.q, alone.k, alone.v, alone.offsets, alone.cand_start, rows, heads)
    assert_close(outs[0][rows, heads], ref, "bf16", "long user, sampled")


@pytest.mark.parametrize("d", [32, 64, 128])
def test_wide_tile_short_key_lists(d):
    """The wide tile takes key tiles in pairs (one barrier per two tiles): users whose key
    lists end at and around tile boundaries (0 to 5 tiles of 64 keys, 0 to 3 of 128 at
    d = 32) but with 2048 candidates each, so that the batch runs on 256-row tiles; the
    same users followed by 300 tiny users run on 128-row tiles.  Bit-identical rows, and
    sampled rows against the oracle."""
    rng = np.random.default_rng(900 + d)
    H = 2
    nkv = np.array([0, 1, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257, 320, 321])
    prefix = np.minimum(nkv, 3)
    wide = W.make_full_batch(rng, "wide-short-keys", prefix=prefix, hist=nkv - prefix, cand=2048, H=H, d=d,
                             seed=910 + d)
    tiny = W.make_full_batch(rng, "tiny", prefix=rng.integers(0, 3, 300), hist=rng.integers(0, 5, 300),
                             cand=rng.integers(1, 4, 300), H=H, d=d, seed=920 + d)
    L = wide.T
    mixed = W.make_full_batch(rng, "mixed", prefix=np.r_[wide.prefix, tiny.prefix], hist=np.r_[wide.hist, tiny.hist],
                              cand=np.r_[wide.cand, tiny.cand], H=H, d=d, seed=930 + d)
    mixed = W.FullBatch(**{**mixed.__dict__, "q": np.concatenate([wide.q, tiny.q]),
                           "k": np.concatenate([wide.k, tiny.k]), "v": np.concatenate([wide.v, tiny.v])})
    assert wide.T >= WIDE_ROWS * wide.B and mixed.T < WIDE_ROWS * mixed.B
    _log(f"[tiles short keys] d={d} wide B={wide.B} T={wide.T} mixed B={mixed.B} T={mixed.T}")
    dw, dm = full_dev(wide), full_dev(mixed)
    outs = [run_full(wide, dw), _planned(wide, dw), run_full(mixed, dm)[:L], _planned(mixed, dm)[:L]]
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(o, outs[0]), f"variant {i} differs from the wide-tile output"
    # per user: its first and last key rows, its first two and last candidates
    rows = []
    for b in range(wide.B):
        lo, cs, hi = int(wide.offsets[b]), int(wide.cand_start[b]), int(wide.offsets[b + 1])
        rows += ([lo, cs - 1] if cs > lo else []) + [cs, cs + 1, hi - 1]
    rows = np.array(rows)
    heads = np.arange(len(rows)) % H
    ref = A.full_attention_rows(wide.q, wide.k, wide.v, wide.offsets, wide.cand_start, rows, heads)
    assert_close(outs[0][rows, heads], ref, "bf16", "short key lists on the wide tile, sampled")


@pytest.mark.parametrize("d", [64, 128])
def test_wide_equals_narrow_candidate_only(d):
    """A user with 2500 candidates over 1800 frozen rows: alone (wide tiles), inside a batch
    of short users (narrow tiles), and the full-sequence layer's candidate rows."""
    rng = np.random.default_rng(800 + d)
    H = 2
    alone = W.make_cand_only_batch(rng, "co-alone", hist=[1800], cand=[2500], H=H, d=d, seed=810 + d)
    nh = rng.integers(0, 90, 40)
    nc = rng.integers(1, 20, 40)
    short = W.make_cand_only_batch(rng, "co-short", hist=nh, cand=nc, H=H, d=d, seed=820 + d)
    cat = lambda a, b: np.concatenate([a, b])
    batch = W.CandOnlyBatch(**{**short.__dict__,
                               "q_cand": cat(alone.q_cand, short.q_cand), "k_cand": cat(alone.k_cand, short.k_cand),
                               "v_cand": cat(alone.v_cand, short.v_cand), "k_hist": cat(alone.k_hist, short.k_hist),
                               "v_hist": cat(alone.v_hist, short.v_hist),
                               "hist_offsets": cat([0], 1800 + short.hist_offsets).astype(short.hist_offsets.dtype),
                               "cand_offsets": cat([0], 2500 + short.cand_offsets).astype(short.cand_offsets.dtype),
                               "name": "co-mixed"})
    assert alone.Tc >= WIDE_ROWS * alone.B and batch.Tc < WIDE_ROWS * batch.B
    _log(f"[tiles cand-only] d={d} alone Tc={alone.Tc} batch B={batch.B} Tc={batch.Tc}")
    a = run_cand_only(alone)
    b = run_cand_only(batch)[:alone.Tc]
    assert np.array_equal(a, b), "candidate-only: narrow and wide tiles differ"
    # the page's fallback: the full layer over [frozen history | candidates], candidate rows
    fb = W.FullBatch(name="co-full", q=np.concatenate([alone.k_hist * 0, alone.q_cand]),
                     k=np.concatenate([alone.k_hist, alone.k_cand]), v=np.concatenate([alone.v_hist, alone.v_cand]),
                     offsets=np.array([0, 4300], np.int32), cand_start=np.array([1800], np.int32), prefix=np.array([0]),
                     hist=np.array([1800]), cand=np.array([2500]), pad=np.array([0]), valid=None,
                     attend_padded_history=False, H=H, d=d, dtype="bf16", seed=0)
    full = run_full(fb)
    assert np.array_equal(full[1800:], a), "candidate-only differs from the full layer's candidate rows"
    rows = np.r_[0:6, 1200:1206, alone.Tc - 6:alone.Tc]
    heads = np.arange(len(rows)) % H
    ref = A.cand_only_attention_rows(alone.q_cand, alone.k_hist, alone.v_hist, alone.k_cand, alone.v_cand,
                                     alone.hist_offsets, alone.cand_offsets, rows, heads)
    assert_close(a[rows, heads], ref, "bf16", "candidate-only long user, sampled")


def test_wide_equals_narrow_cached_request():
    """The layer stack's cached request (every layer candidate-only over the history keys and
    values) for a user with 2100 candidates: alone (wide tiles) and in a batch of short
    users (narrow tiles) give the same candidate states bit for bit."""
    H, d, n_layers, nco = 4, 64, 3, 1
    D = H * d
    rng = np.random.default_rng(77)

    def request(prefix, hist, cand, seed):
        L = np.asarray(prefix) + np.asarray(hist) + np.asarray(cand)
        off = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
        cs = (off[:-1] + np.asarray(prefix) + np.asarray(hist)).astype(np.int32)
        x, layers = W.ranker_inputs(seed, int(off[-1]), n_layers, D)
        return x, off, cs, layers

    xl, offl, csl, layers = request([4], [1500], [2100], 5)
    xs, offs, css, _ = request(rng.integers(0, 3, 40), rng.integers(0, 50, 40), rng.integers(1, 15, 40), 6)
    dl = [(to_dev(g), to_dev(wq, torch.bfloat16), to_dev(wo, torch.bfloat16)) for g, wq, wo in layers]
    R = rr()

    def full(x, off, cs):
        Tc = int((off[1:] - cs).sum())
        xd = to_dev(x.copy())
        xc, _, cache = R.rr_ranker_fwd(xd, dl, nco, to_dev(off), to_dev(cs), Tc, H, d)
        return xc, cache

    xc_l, cache_l = full(xl, offl, csl)
    _, cache_s = full(xs, offs, css)
    torch.cuda.synchronize()

    def offsets_of(off, cs):
        hl, cl = cs - off[:-1], off[1:] - cs
        return (np.concatenate([[0], np.cumsum(hl)]).astype(np.int32),
                np.concatenate([[0], np.cumsum(cl)]).astype(np.int32))
    hoff_l, coff_l = offsets_of(offl, csl)
    hoff_s, coff_s = offsets_of(offs, css)
    cand_l = np.concatenate([xl[csl[0]:offl[1]]]).astype(np.float32)
    cand_s = np.concatenate([xs[css[b]:offs[b + 1]] for b in range(len(css))]).astype(np.float32)
    assert len(cand_l) >= WIDE_ROWS and len(cand_l) + len(cand_s) < WIDE_ROWS * (1 + len(css))
    alone = R.rr_ranker_cached_fwd(to_dev(cand_l), dl, cache_l, to_dev(hoff_l), to_dev(coff_l), H, d)
    cache_b = torch.cat([cache_l, cache_s], dim=2).contiguous()
    hoff_b = np.concatenate([hoff_l, hoff_l[-1] + hoff_s[1:]]).astype(np.int32)
    coff_b = np.concatenate([coff_l, coff_l[-1] + coff_s[1:]]).astype(np.int32)
    mixed = R.rr_ranker_cached_fwd(to_dev(np.concatenate([cand_l, cand_s])), dl, cache_b, to_dev(hoff_b),
                                   to_dev(coff_b), H, d)
    torch.cuda.synchronize()
    _log(f"[tiles cached request] candidates alone {len(cand_l)}, in the batch {len(cand_l) + len(cand_s)}")
    assert torch.equal(alone, mixed[:len(cand_l)]), "cached request: narrow and wide tiles differ"
    assert torch.equal(alone, xc_l), "cached request differs from the full request"


# ---------------------------------------------------------------- sentinels


def _poisoned_full(seed, d, pad, flag, H=2):
    """Four long users (wide tiles); users 1 and 3 have every value = 1e3, and every
    candidate's value (and, with flag False, every padding row's) is 1e3 too."""
    rng = np.random.default_rng(seed)
    fb = W.make_full_batch(rng, "sentinel-wide", prefix=[4, 2, 0, 3], hist=[2600, 3000, 1500, 2200],
                           cand=[400, 900, 2100, 300], pad=pad, H=H, d=d, attend_padded_history=flag, seed=seed)
    v = fb.v.copy()
    for b in range(fb.B):
        lo, cs, hi = int(fb.offsets[b]), int(fb.cand_start[b]), int(fb.offsets[b + 1])
        v[cs:hi] = 1000.0
        if b in (1, 3):
            v[lo:hi] = 1000.0
    if fb.valid is not None and not flag:
        v[fb.valid == 0] = 1000.0
    return W.FullBatch(**{**fb.__dict__, "v": v})


@pytest.mark.parametrize("pad,flag", [(None, False), ([100, 0, 300, 50], False), ([100, 0, 300, 50], True)])
def test_sentinel_wide_tiles(pad, flag):
    fb = _poisoned_full(4200 + (pad is not None) + 2 * flag, 64, pad, flag)
    assert fb.T >= WIDE_ROWS * fb.B
    _log(f"[sentinel wide] T={fb.T} padded={pad is not None} flag={flag}")
    got = run_full(fb)
    ref = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, fb.valid, fb.attend_padded_history)
    assert_close(got, ref, "bf16", f"sentinel wide padded={pad is not None} flag={flag}")


@pytest.mark.parametrize("wide", [False, True])
def test_sentinel_candidate_only(wide):
    """Candidate-only layers: the frozen rows of users 1 and 3 and every candidate's own value
    are 1e3; narrow and wide tiles."""
    rng = np.random.default_rng(4300 + wide)
    if wide:
        hist, cand = [2000, 2600, 700, 3100], [2300, 2100, 2500, 2200]
    else:
        hist, cand = [900, 40, 300, 1200, 0, 77], [130, 20, 64, 300, 5, 1]
    cb = W.make_cand_only_batch(rng, "sentinel-co", hist=hist, cand=cand, H=2, d=128, seed=4310 + wide)
    assert (cb.Tc >= WIDE_ROWS * cb.B) == wide
    vh, vc = cb.v_hist.copy(), np.full_like(cb.v_cand, 1000.0)
    for b in (1, 3):
        vh[int(cb.hist_offsets[b]):int(cb.hist_offsets[b + 1])] = 1000.0
    cb = W.CandOnlyBatch(**{**cb.__dict__, "v_hist": vh, "v_cand": vc})
    _log(f"[sentinel cand-only] wide={wide} Th={cb.Th} Tc={cb.Tc}")
    got = run_cand_only(cb)
    ref = A.cand_only_attention(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand, cb.hist_offsets,
                                cb.cand_offsets)
    assert_close(got, ref, "bf16", f"sentinel candidate-only wide={wide}")


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("d,scale", [(32, None), (64, None), (128, None), (128, 0.3)])
def test_key_bound_settling(d, scale):
    """Planned wide-tile launches bound every row's scores by |q| max|k| (a pass over the
    keys) and stop forming tile maxima once no tile can move a row's reference.  The long
    user's heads are built so that waves settle at different points: head 0 holds the
    standard draw (every wave settles after its first trip), in head 1 the first 200
    queries are near one direction q0 and key row 1300 is a large multiple of q0 (their
    reference moves at that key's tile, about 19 log2 units up, and they settle after it,
    while the other waves of the same query tiles never do), and head 2 has features of
    scale 2 (bounds far above every reference: no wave settles).  The planned wide-tile
    output (with the bound) must equal, bit for bit, the self-planned wide tile and both
    narrow-tile runs (without it), and match the oracle on sampled rows; also with a softmax
    scale of 0.3 instead of 1/sqrt(d) (the bound scales with it)."""
    alone, batch, L = _long_and_short(d, 3, 1200 + d, (4, 2500, 700))
    rng = np.random.default_rng(1250 + d)
    q, k, v = alone.q.copy(), alone.k.copy(), alone.v.copy()
    q0 = rng.standard_normal(d) / np.sqrt(d)
    q[:200, 1] = q0 + 0.02 * rng.standard_normal((200, d)) / np.sqrt(d)
    alpha = 19.0 / (np.log2(np.e) / np.sqrt(d)) / float(q0 @ q0)
    k[1300, 1] = alpha * q0
    q[:, 2] *= 2.0 * np.sqrt(d)
    k[:, 2] *= 2.0 * np.sqrt(d)
    q, k = _bf16(q), _bf16(k)
    alone = W.FullBatch(**{**alone.__dict__, "q": q, "k": k, "v": v})
    batch = W.FullBatch(**{**batch.__dict__, "q": np.concatenate([q, batch.q[L:]]),
                           "k": np.concatenate([k, batch.k[L:]]), "v": np.concatenate([v, batch.v[L:]])})
    _log(f"[tiles key bound] d={d} alone T={alone.T} batch B={batch.B} T={batch.T} alpha={alpha:.1f}")
    da, db = full_dev(alone), full_dev(batch)
    kw = {} if scale is None else {"scale": scale}
    outs = [_planned(alone, da, scale), run_full(alone, da, **kw), run_full(batch, db, **kw)[:L],
            _planned(batch, db, scale)[:L]]
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(o, outs[0]), f"variant {i} differs from the bounded wide-tile output"
    rows = np.r_[0:6, 195:205, 1298:1302, 2500:2504, alone.T - 6:alone.T]
    for h in range(3):
        hs = np.full(len(rows), h)
        ref = A.full_attention_rows(alone.q, alone.k, alone.v, alone.offsets, alone.cand_start, rows, hs, **kw)
        assert_close(outs[0][rows, hs], ref, "bf16", f"key bound, head {h}, sampled")


@pytest.mark.parametrize("flag", [False, True])
def test_key_bound_settling_padded(flag):
    """The key-norm bound on padded batches: a long user with 50 padding rows between its
    prefix and its history, the heads built as in test_key_bound_settling (waves settling
    early, late and never).  Attended padding (flag True) keeps the keys one row range;
    excluded padding (flag False) lists them through the compacted rows, and the bound then
    spans the first to the last listed key.  The planned wide-tile output must equal, bit
    for bit, the same user's rows in a batch of short users on the narrow tile, and match
    the oracle on sampled rows (padding rows excluded from the keys read 0)."""
    d, H, P = 128, 3, 50
    rng = np.random.default_rng(1300 + flag)
    alone = W.make_full_batch(rng, "pad-long", prefix=[4], hist=[2500], cand=[700], pad=[P], H=H, d=d,
                              attend_padded_history=flag, seed=1310 + flag)
    q, k, v = alone.q.copy(), alone.k.copy(), alone.v.copy()
    q0 = rng.standard_normal(d) / np.sqrt(d)
    q[:200, 1] = q0 + 0.02 * rng.standard_normal((200, d)) / np.sqrt(d)
    k[1300, 1] = 19.0 / (np.log2(np.e) / np.sqrt(d)) / float(q0 @ q0) * q0
    q[:, 2] *= 2.0 * np.sqrt(d)
    k[:, 2] *= 2.0 * np.sqrt(d)
    q, k = _bf16(q), _bf16(k)
    alone = W.FullBatch(**{**alone.__dict__, "q": q, "k": k, "v": v})
    n_short = 40
    sp, sh, sc = rng.integers(0, 4, n_short), rng.integers(0, 60, n_short), rng.integers(0, 12, n_short)
    short = W.make_full_batch(rng, "short", prefix=sp, hist=sh, cand=sc, pad=rng.integers(0, 3, n_short), H=H,
                              d=d, attend_padded_history=flag, seed=1320 + flag)
    L = alone.T
    off = np.concatenate([alone.offsets, short.offsets[1:] + L]).astype(np.int32)
    cst = np.concatenate([alone.cand_start, short.cand_start + L]).astype(np.int32)
    valid = np.concatenate([alone.valid, short.valid]).astype(np.uint8)
    batch = W.FullBatch(**{**short.__dict__, "name": "pad-mixed", "prefix": np.r_[alone.prefix, short.prefix],
                           "hist": np.r_[alone.hist, short.hist], "cand": np.r_[alone.cand, short.cand],
                           "pad": np.r_[alone.pad, short.pad], "offsets": off, "cand_start": cst, "valid": valid,
                           "q": np.concatenate([q, short.q]), "k": np.concatenate([k, short.k]),
                           "v": np.concatenate([v, short.v])})
    assert alone.T >= WIDE_ROWS * alone.B and batch.T < WIDE_ROWS * batch.B
    _log(f"[tiles key bound padded] flag={flag} alone T={alone.T} batch B={batch.B} T={batch.T}")
    da, db = full_dev(alone), full_dev(batch)
    outs = [_planned(alone, da), run_full(alone, da), run_full(batch, db)[:L], _planned(batch, db)[:L]]
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(o, outs[0]), f"variant {i} differs from the bounded wide-tile output"
    rows = np.r_[0:6, 50:56, 195:205, 1298:1302, 2550:2556, alone.T - 6:alone.T]
    for h in range(H):
        hs = np.full(len(rows), h)
        ref = A.full_attention_rows(alone.q, alone.k, alone.v, alone.offsets, alone.cand_start, rows, hs,
                                    valid=alone.valid, attend_padded_history=flag)
        assert_close(outs[0][rows, hs], ref, "bf16", f"padded key bound, flag {flag}, head {h}, sampled")
