"""GPU tests of the layer stack (rr_linear, rr_rms_norm, rr_ranker_fwd, rr_ranker_cached_fwd)
against the oracle (oracle/ranker.py) and the page's invariants."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from _gpu import gpu, needs_gpu, rr, to_dev
from oracle import ranker as RK

pytestmark = [gpu, needs_gpu]
U = 2.0 ** -8          # bf16 unit roundoff (8 significant bits)
F32 = 2.0 ** -24


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _layout(prefix, hist, cand):
    L = np.asarray(prefix) + np.asarray(hist) + np.asarray(cand)
    off = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cs = (off[:-1] + np.asarray(prefix) + np.asarray(hist)).astype(np.int32)
    return off, cs


# users: a long history, no history at all (candidates read only themselves), no
# candidates, a single candidate, a prefix-only history
SHAPES = dict(prefix=[4, 0, 0, 3, 1, 2], hist=[300, 0, 45, 700, 129, 0], cand=[37, 6, 0, 128, 1, 5])


def _setup(H, d, n_layers, seed, shapes=SHAPES):
    off, cs = _layout(**shapes)
    T = int(off[-1])
    x, layers = W.ranker_inputs(seed, T, n_layers, H * d)
    dev_layers = [(to_dev(g), to_dev(wq, torch.bfloat16), to_dev(wo, torch.bfloat16)) for g, wq, wo in layers]
    or_layers = [RK.Layer(g.astype(np.float64), wq.astype(np.float64), wo.astype(np.float64))
                 for g, wq, wo in layers]
    return x, off, cs, dev_layers, or_layers


def _run(x, off, cs, dev_layers, n_cand_only, H, d, user_tokens=None):
    Tc = int((off[1:] - cs).sum())
    xd = to_dev(x.copy())
    ut = None if user_tokens is None else to_dev(np.asarray(user_tokens, np.int32))
    Tp = 0 if user_tokens is None else int(np.sum(user_tokens))
    xc, xh, cache = rr().rr_ranker_fwd(xd, dev_layers, n_cand_only, to_dev(off), to_dev(cs), Tc, H, d,
                                       user_tokens=ut, Tp=Tp)
    torch.cuda.synchronize()
    return xd, xc, xh, cache


def test_linear_bounds_and_rows():
    rng = np.random.default_rng(1)
    for M, N, K in ((1, 128, 64), (129, 384, 256), (300, 256, 512)):
        a = W.round_to_bf16(rng.standard_normal((M, K)).astype(np.float32)).astype(np.float64)
        w = W.round_to_bf16((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)).astype(np.float64)
        ad, wd = to_dev(a, torch.bfloat16), to_dev(w, torch.bfloat16)
        got = _np(rr().rr_linear(ad, wd))
        ref = a @ w.T
        mag = np.abs(a) @ np.abs(w).T
        # exact bf16 products summed in fp32 (at most K roundings), then one rounding to bf16
        assert np.all(np.abs(got - ref) <= U * np.abs(ref) + (K + 2) * F32 * mag), (M, N, K)
        res0 = rng.standard_normal((M, N)).astype(np.float32)
        res = to_dev(res0.copy())
        rr().rr_linear(ad, wd, residual=res)
        got_r = _np(res)
        assert np.all(np.abs(got_r - (res0 + ref)) <= (K + 2) * F32 * (mag + np.abs(res0))), (M, N, K)
        # a row's result does not depend on the other rows of the launch
        r = M // 2
        one = rr().rr_linear(ad[r:r + 1].contiguous(), wd)
        torch.cuda.synchronize()
        assert np.array_equal(_np(one)[0], got[r])


def test_linear_large_tile_rows():
    """A product large enough for the 256 x 256 tiles: sampled rows within the rounding
    bound, and every row bit-identical to the same row computed in a small launch (the
    128 x 128 tiles), plus a slice of rows at an offset that is not a tile multiple."""
    rng = np.random.default_rng(3)
    M, N, K = 65536, 512, 256
    a = W.round_to_bf16(rng.standard_normal((M, K)).astype(np.float32)).astype(np.float64)
    w = W.round_to_bf16((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)).astype(np.float64)
    ad, wd = to_dev(a, torch.bfloat16), to_dev(w, torch.bfloat16)
    big = rr().rr_linear(ad, wd)
    rows = np.sort(rng.choice(M, 300, replace=False))
    got = _np(big[torch.from_numpy(rows).to(big.device)])
    ref = a[rows] @ w.T
    mag = np.abs(a[rows]) @ np.abs(w).T
    assert np.all(np.abs(got - ref) <= U * np.abs(ref) + (K + 2) * F32 * mag)
    for lo, n in ((0, 1), (777, 130), (M - 40, 40)):
        part = rr().rr_linear(ad[lo:lo + n].contiguous(), wd)
        torch.cuda.synchronize()
        assert torch.equal(part, big[lo:lo + n]), (lo, n)
    res0 = to_dev(rng.standard_normal((M, N)).astype(np.float32))
    res = res0.clone()
    rr().rr_linear(ad, wd, residual=res)
    part = res0[777:907].clone()
    rr().rr_linear(ad[777:907].contiguous(), wd, residual=part)
    torch.cuda.synchronize()
    assert torch.equal(part, res[777:907])


def test_rms_norm_bounds():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((37, 256)) * rng.uniform(0.01, 20, (37, 1))).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(256)).astype(np.float32)
    got = _np(rr().rr_rms_norm(to_dev(x), to_dev(g)))
    ref = RK.rms_norm(x, g)
    # float32 evaluation (relative 2^-20 covers its few roundings), one rounding to bf16
    assert np.all(np.abs(got - ref) <= (U + 2.0 ** -20) * np.abs(ref) + 1e-30)


# Element by element: the layer's update against the oracle's, within 10 standard deviations
# of the probabilistic rounding model at the bf16 rounding points of the layer (the oracle's
# full_layer_rounding_sigma / cand_only_layer_rounding_sigma, 64 seeded draws: the estimate
# is within about 25% of the true spread for almost every element) plus float32-level terms.
SIGMA_K, SIGMA_SAMPLES = 10.0, 64


def _elementwise(got, ref, base, sigma, slack, what):
    err = np.abs((got - base) - (ref - base))
    bound = SIGMA_K * sigma + slack
    excess = err - bound
    if np.max(excess) > 0:
        i = np.unravel_index(int(np.argmax(excess / np.maximum(bound, 1e-300))), err.shape)
        raise AssertionError(f"{what}: error {err[i]:.3e} over the bound {bound[i]:.3e} at {i} "
                             f"(sigma {sigma[i]:.3e})")


def _cand_only_slack(x_cand, x_hist, layer, hoff, coff, H, d):
    x, off, cs, rows = RK._fallback_layout(x_hist, x_cand, hoff, coff)
    return RK.f32_slack(x, layer, off, cs, H, d)[rows]


def _frob(got, ref, base, what):
    """Relative Frobenius error of a layer's update (got - base against ref - base)."""
    e = np.linalg.norm(got - ref) / max(np.linalg.norm(ref - base), 1e-30)
    # about five bf16 roundings on the update's path (norm, projections, rotation, attention
    # weights and output), independent errors of relative size u / sqrt(3) each: ~1.3 u;
    # bound 4 u
    assert e <= 4 * U, f"{what}: relative error {e:.4f} > {4 * U:.4f}"


@pytest.mark.parametrize("H,d", [(4, 32), (4, 64), (4, 128)])
def test_each_layer_against_oracle(H, d):
    """The stack run with its first l layers, l = 1..L: layer l's update against the oracle's
    layer applied to the GPU's state before it (no error carried between layers), element by
    element within the rounding model's spread and, as a second check, in Frobenius norm."""
    n_layers, n_cand_only = 4, 2
    x, off, cs, dl, ol = _setup(H, d, n_layers, seed=40 + d)
    xh0, xc0, hoff, coff = RK.split_history_and_candidates(x, off, cs)
    prev_full, prev_c, prev_h = x.astype(np.float64), None, None
    n_full = n_layers - n_cand_only
    for l in range(1, n_layers + 1):
        nco = max(0, l - n_full)
        xd, xc, xh, _ = _run(x, off, cs, dl[:l], nco, H, d)
        if l <= n_full:
            got = _np(xd)
            ref = RK.block_full(prev_full, ol[l - 1], off, cs, H, d)
            sg = RK.full_layer_rounding_sigma(prev_full, ol[l - 1], off, cs, H, d, samples=SIGMA_SAMPLES, seed=l)
            _elementwise(got, ref, prev_full, sg, RK.f32_slack(prev_full, ol[l - 1], off, cs, H, d),
                         f"full layer {l}")
            _frob(got, ref, prev_full, f"full layer {l}")
            prev_full = got
            prev_h, prev_c = RK.split_history_and_candidates(got, off, cs)[:2]
            assert np.array_equal(_np(xc), prev_c) and np.array_equal(_np(xh), prev_h)
        else:
            assert np.array_equal(_np(xh), prev_h), "the history moved in a candidate-only layer"
            kh, vh = RK.history_kv(prev_h, ol[l - 1], hoff, H, d)
            ref = RK.block_cand_only(prev_c, kh, vh, ol[l - 1], hoff, coff, H, d)
            got = _np(xc)
            sg = RK.cand_only_layer_rounding_sigma(prev_c, prev_h, ol[l - 1], hoff, coff, H, d,
                                                   samples=SIGMA_SAMPLES, seed=l)
            _elementwise(got, ref, prev_c, sg, _cand_only_slack(prev_c, prev_h, ol[l - 1], hoff, coff, H, d),
                         f"candidate-only layer {l}")
            _frob(got, ref, prev_c, f"candidate-only layer {l}")
            prev_c = got


def test_stack_is_the_composition_of_its_parts():
    """rr_ranker_fwd equals, bit for bit, the same layers written out with the separately
    tested entry points (rr_rms_norm, rr_linear, rr_rope_qk, rr_attn_fwd,
    rr_cand_only_attn_fwd) and plain row gathers for the split and the cache."""
    H, d, n_layers, nco = 4, 64, 3, 1
    x, off, cs, dl, _ = _setup(H, d, n_layers, seed=50)
    xd, xc, xh, cache = _run(x, off, cs, dl, nco, H, d)
    R = rr()
    D = H * d
    offd, csd = to_dev(off), to_dev(cs)
    hist_rows = np.concatenate([np.arange(off[b], cs[b]) for b in range(len(cs))]).astype(np.int64)
    cand_rows = np.concatenate([np.arange(cs[b], off[b + 1]) for b in range(len(cs))]).astype(np.int64)
    hi, ci = to_dev(hist_rows), to_dev(cand_rows)
    hoff = to_dev(np.concatenate([[0], np.cumsum(cs - off[:-1])]).astype(np.int32))
    coff = to_dev(np.concatenate([[0], np.cumsum(off[1:] - cs)]).astype(np.int32))
    hlen = to_dev((cs - off[:-1]).astype(np.int32))
    s = to_dev(x.copy())
    T = s.shape[0]
    for l, (g, wq, wo) in enumerate(dl[:n_layers - nco]):
        qkv = R.rr_linear(R.rr_rms_norm(s, g), wq)
        q, k, v = (qkv[:, i * D:(i + 1) * D].contiguous().view(T, H, d) for i in range(3))
        q, k = R.rr_rope_qk(q, k, offd, csd)
        assert torch.equal(cache[l, 0], k[hi]) and torch.equal(cache[l, 1], v[hi]), l
        o = R.rr_attn_fwd(q, k, v, offd, csd)
        R.rr_linear(o.view(T, D), wo, residual=s)
    torch.cuda.synchronize()
    assert torch.equal(s, xd)
    sh, sc = s[hi].contiguous(), s[ci].contiguous()
    for l in range(n_layers - nco, n_layers):
        g, wq, wo = dl[l]
        kv = R.rr_linear(R.rr_rms_norm(sh, g), wq[D:].contiguous())
        kh, vh = (kv[:, i * D:(i + 1) * D].contiguous().view(-1, H, d) for i in range(2))
        _, kh = R.rr_rope_qk(None, kh, hoff, hoff[1:].contiguous())
        assert torch.equal(cache[l, 0], kh) and torch.equal(cache[l, 1], vh), l
        qkv = R.rr_linear(R.rr_rms_norm(sc, g), wq)
        Tc = sc.shape[0]
        q, k, v = (qkv[:, i * D:(i + 1) * D].contiguous().view(Tc, H, d) for i in range(3))
        q, k = R.rr_rope_qk(q, k, coff, coff[:-1].contiguous(), pos_base=hlen)
        o = R.rr_cand_only_attn_fwd(q, kh, vh, k, v, hoff, coff)
        R.rr_linear(o.view(Tc, D), wo, residual=sc)
    torch.cuda.synchronize()
    assert torch.equal(sc, xc) and torch.equal(sh, xh)


def test_cached_request_bit_identical():
    """A later request with the same users: the cached pass reproduces the full pass's
    candidates bit for bit, also for a new set of candidates."""
    H, d, n_layers, nco = 4, 128, 4, 2
    x, off, cs, dl, _ = _setup(H, d, n_layers, seed=60)
    _, xc, xh, cache = _run(x, off, cs, dl, nco, H, d)
    xh0, xc0, hoff, coff = RK.split_history_and_candidates(x, off, cs)
    again = rr().rr_ranker_cached_fwd(to_dev(xc0.astype(np.float32)), dl, cache, to_dev(hoff.astype(np.int32)),
                                      to_dev(coff.astype(np.int32)), H, d)
    torch.cuda.synchronize()
    assert torch.equal(again, xc)
    # new candidates for the same users (other counts): the full pass on the new layout
    rng = np.random.default_rng(61)
    newc = np.array([3, 0, 9, 1, 4, 2])
    prefix, hist = np.array(SHAPES["prefix"]), np.array(SHAPES["hist"])
    off2, cs2 = _layout(prefix, hist, newc)
    x2 = np.concatenate([np.concatenate([x[off[b]:cs[b]], rng.standard_normal((newc[b], x.shape[1]))])
                         for b in range(len(newc))]).astype(np.float32)
    _, xc2, xh2, cache2 = _run(x2, off2, cs2, dl, nco, H, d)
    assert torch.equal(xh2, xh) and torch.equal(cache2, cache)
    c2 = RK.split_history_and_candidates(x2, off2, cs2)
    cached = rr().rr_ranker_cached_fwd(to_dev(c2[1].astype(np.float32)), dl, cache,
                                       to_dev(hoff.astype(np.int32)), to_dev(c2[3].astype(np.int32)), H, d)
    torch.cuda.synchronize()
    assert torch.equal(cached, xc2)


def test_many_users_cached_request_bit_identical():
    """2200 users (more than the plans sort in LDS, several passes of the split's per-user
    scan): the cached request still reproduces the full request bit for bit."""
    rng = np.random.default_rng(62)
    B = 2200
    shapes = dict(prefix=rng.integers(0, 3, B), hist=rng.integers(0, 40, B) * (rng.random(B) > 0.1),
                  cand=rng.integers(0, 6, B) * (rng.random(B) > 0.1))
    shapes["hist"][::97] = 130
    shapes["cand"][::89] = 131
    H, d, n_layers, nco = 2, 64, 2, 1
    x, off, cs, dl, _ = _setup(H, d, n_layers, seed=63, shapes=shapes)
    print(f"[ranker, many users] B={B} T={int(off[-1])}", flush=True)
    _, xc, xh, cache = _run(x, off, cs, dl, nco, H, d)
    xh0, xc0, hoff, coff = RK.split_history_and_candidates(x, off, cs)
    again = rr().rr_ranker_cached_fwd(to_dev(xc0.astype(np.float32)), dl, cache, to_dev(hoff.astype(np.int32)),
                                      to_dev(coff.astype(np.int32)), H, d)
    torch.cuda.synchronize()
    assert torch.equal(again, xc)
    assert np.all(np.isfinite(_np(xc))) and np.all(np.isfinite(_np(xh)))


def test_long_users_cached_request_bit_identical():
    """Users of about 4000 rows: the full layers run on 256-row query tiles with the
    key-norm bound (their tiles stop forming maxima once no key can move a row's
    reference), while the cached request's candidate-only layers run on 128-row tiles
    without it.  The cached request still reproduces the full request's candidates bit
    for bit."""
    shapes = dict(prefix=[4, 2], hist=[3000, 2600], cand=[900, 1500])
    H, d, n_layers, nco = 4, 128, 4, 2
    x, off, cs, dl, _ = _setup(H, d, n_layers, seed=64, shapes=shapes)
    T, B = int(off[-1]), len(shapes["hist"])
    assert T >= 2048 * B, "the full layers must take the wide tile"
    print(f"[ranker, long users] B={B} T={T}", flush=True)
    _, xc, xh, cache = _run(x, off, cs, dl, nco, H, d)
    xh0, xc0, hoff, coff = RK.split_history_and_candidates(x, off, cs)
    again = rr().rr_ranker_cached_fwd(to_dev(xc0.astype(np.float32)), dl, cache, to_dev(hoff.astype(np.int32)),
                                      to_dev(coff.astype(np.int32)), H, d)
    torch.cuda.synchronize()
    assert torch.equal(again, xc)
    assert np.all(np.isfinite(_np(xc))) and np.all(np.isfinite(_np(xh)))


def test_candidate_order_bit_identical():
    H, d, n_layers, nco = 4, 64, 3, 1
    x, off, cs, dl, _ = _setup(H, d, n_layers, seed=70)
    _, xc, xh, _ = _run(x, off, cs, dl, nco, H, d)
    b = 3
    perm = np.arange(len(x))
    perm[cs[b]:off[b + 1]] = cs[b] + np.random.default_rng(7).permutation(off[b + 1] - cs[b])
    _, xc2, xh2, _ = _run(x[perm], off, cs, dl, nco, H, d)
    coff = np.concatenate([[0], np.cumsum(off[1:] - cs)])
    cperm = np.arange(int(coff[-1]))
    cperm[coff[b]:coff[b + 1]] = coff[b] + (perm[cs[b]:off[b + 1]] - cs[b])
    assert torch.equal(xh2, xh)
    assert torch.equal(xc2, xc[to_dev(cperm)])


def test_user_token_attention():
    """rr_user_token_attn: each query of a user reads exactly that user's keys, no self-term;
    a user without keys gives 0; against the oracle's masked softmax attention."""
    from oracle.attention import masked_softmax_attention
    rng = np.random.default_rng(80)
    H, d = 3, 64
    nk, nq = np.array([5, 0, 300, 1, 70]), np.array([2, 3, 0, 4, 9])
    koff = np.concatenate([[0], np.cumsum(nk)]).astype(np.int32)
    qoff = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q, k, v = (W.round_to_bf16(rng.standard_normal((n, H, d)).astype(np.float32)) for n in (qoff[-1], koff[-1],
                                                                                          koff[-1]))
    got = _np(rr().rr_user_token_attn(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16),
                                      to_dev(v, torch.bfloat16), to_dev(koff), to_dev(qoff)))
    ref = np.zeros(q.shape)
    for b in range(len(nk)):
        qs, ks = slice(qoff[b], qoff[b + 1]), slice(koff[b], koff[b + 1])
        if nk[b] == 0 or nq[b] == 0:
            continue
        for h in range(H):
            ref[qs, h] = masked_softmax_attention(q[qs, h].astype(np.float64), k[ks, h].astype(np.float64),
                                                  v[ks, h].astype(np.float64), np.ones((nq[b], nk[b]), bool),
                                                  1.0 / np.sqrt(d))
    from _gpu import assert_close
    assert_close(got, ref, "bf16", "user-token attention")
    assert not got[qoff[1]:qoff[2]].any(), "a user with no keys must give 0"


def _user_token_layout(cur_h, frozen_h, cur_c, is_p, p, hoff, coff):
    """Per user [user tokens (current) | rest of the history (frozen) | candidates] as one
    full-sequence batch, with the rows of the user tokens and of the candidates in it."""
    parts, offs, cst, rows_p, rows_c = [], [0], [], [], []
    for b in range(len(p)):
        blk_h = np.where(is_p[hoff[b]:hoff[b + 1], None], cur_h[hoff[b]:hoff[b + 1]], frozen_h[hoff[b]:hoff[b + 1]])
        parts += [blk_h, cur_c[coff[b]:coff[b + 1]]]
        rows_p += range(offs[-1], offs[-1] + int(p[b]))
        cst.append(offs[-1] + len(blk_h))
        rows_c += range(cst[-1], cst[-1] + int(coff[b + 1] - coff[b]))
        offs.append(cst[-1] + int(coff[b + 1] - coff[b]))
    return np.concatenate(parts), np.asarray(offs), np.asarray(cst), np.asarray(rows_p), np.asarray(rows_c)


@pytest.mark.parametrize("d", [64, 128])
def test_user_token_layers_against_oracle(d):
    """candidate_only_layers_update_user_token: each candidate-only layer's update of the
    user tokens and of the candidates against the oracle's layer on the GPU's own state
    (element by element within the rounding model's spread, and in Frobenius norm); the
    other rows before the candidate start stay frozen bit for bit."""
    H, n_layers, n_cand_only = 4, 4, 2
    x, off, cs, dl, ol = _setup(H, d, n_layers, seed=90 + d)
    p = np.array(SHAPES["prefix"])
    n_full = n_layers - n_cand_only
    _, xc, xh, _ = _run(x, off, cs, dl[:n_full], 0, H, d)
    prev_c, prev_h = _np(xc), _np(xh)
    frozen_h = prev_h.copy()
    hoff = np.concatenate([[0], np.cumsum(cs - off[:-1])])
    coff = np.concatenate([[0], np.cumsum(off[1:] - cs)])
    is_p = np.zeros(len(prev_h), bool)
    for b in range(len(p)):
        is_p[hoff[b]:hoff[b] + p[b]] = True
    for l in range(n_full + 1, n_layers + 1):
        _, xc, xh, _ = _run(x, off, cs, dl[:l], l - n_full, H, d, user_tokens=p)
        got_c, got_h = _np(xc), _np(xh)
        assert np.array_equal(got_h[~is_p], frozen_h[~is_p]), "a history row moved"
        ref_p, ref_c, _, _ = RK.block_user_token_layer(prev_h[is_p], frozen_h, prev_c, ol[l - 1], p, hoff, coff,
                                                       H, d, 10000.0, None)
        # the layer is the full layer over each user's [user tokens | frozen history | candidates]
        X, offs, cst, rows_p, rows_c = _user_token_layout(prev_h, frozen_h, prev_c, is_p, p, hoff, coff)
        sg = RK.full_layer_rounding_sigma(X, ol[l - 1], offs, cst, H, d, samples=SIGMA_SAMPLES, seed=l)
        sl = RK.f32_slack(X, ol[l - 1], offs, cst, H, d)
        _elementwise(got_c, ref_c, prev_c, sg[rows_c], sl[rows_c], f"candidates, layer {l}")
        _elementwise(got_h[is_p], ref_p, prev_h[is_p], sg[rows_p], sl[rows_p], f"user tokens, layer {l}")
        _frob(got_c, ref_c, prev_c, f"candidates, layer {l}")
        _frob(got_h[is_p], ref_p, prev_h[is_p], f"user tokens, layer {l}")
        prev_c, prev_h = got_c, got_h


def test_user_token_cached_request_bit_identical():
    H, d, n_layers, nco = 4, 64, 4, 2
    x, off, cs, dl, _ = _setup(H, d, n_layers, seed=95)
    p = np.array(SHAPES["prefix"])
    _, xc, xh, cache = _run(x, off, cs, dl, nco, H, d, user_tokens=p)
    _, xc_plain, xh_plain, _ = _run(x, off, cs, dl, nco, H, d)
    assert not torch.equal(xc, xc_plain), "updating the user tokens changed nothing"
    _, xc0, hoff, coff = RK.split_history_and_candidates(x, off, cs)
    again = rr().rr_ranker_cached_fwd(to_dev(xc0.astype(np.float32)), dl, cache, to_dev(hoff.astype(np.int32)),
                                      to_dev(coff.astype(np.int32)), H, d)
    torch.cuda.synchronize()
    assert torch.equal(again, xc)


N_STACK_CASES = 12


def _random_stack_case(i):
    """Layout and stack shape of random case i: up to 12 users (empty histories, users without
    candidates, single candidates, prefix-only histories; at least one candidate), H and d
    with H d a multiple of 128, 2-3 layers of which 0 to all are candidate-only."""
    rng = np.random.default_rng(7700 + i)
    B = int(rng.integers(1, 13))
    shapes = dict(prefix=rng.integers(0, 4, B), hist=rng.integers(0, 300, B) * (rng.random(B) > 0.15),
                  cand=rng.integers(1, 40, B) * (rng.random(B) > 0.15))
    if shapes["cand"].sum() == 0:
        shapes["cand"][0] = 1
    H, d = [(1, 128), (2, 64), (2, 128), (4, 32), (4, 64), (4, 128)][int(rng.integers(0, 6))]
    n_layers = int(rng.integers(2, 4))
    nco = int(rng.integers(0, n_layers + 1))
    return rng, shapes, H, d, n_layers, nco


def test_random_stack_sweep():
    """Random layouts and stack shapes: each layer's update against the oracle's layer on the
    GPU's state before it, in relative Frobenius norm; the cached request equal to the full
    request's candidates bit for bit; a permutation of one user's candidates permuting their
    outputs bit for bit."""
    for i in range(N_STACK_CASES):
        rng, shapes, H, d, n_layers, nco = _random_stack_case(i)
        B = len(shapes["cand"])
        what = f"stack sweep {i} (B={B} H={H} d={d} layers={n_layers} candidate-only={nco})"
        print(what, flush=True)
        x, off, cs, dl, ol = _setup(H, d, n_layers, seed=7800 + i, shapes=shapes)
        hoff = np.concatenate([[0], np.cumsum(cs - off[:-1])])
        coff = np.concatenate([[0], np.cumsum(off[1:] - cs)])
        prev_full, prev_c, prev_h = x.astype(np.float64), None, None
        n_full = n_layers - nco
        for l in range(1, n_layers + 1):
            xd, xc, xh, cache = _run(x, off, cs, dl[:l], max(0, l - n_full), H, d)
            if l <= n_full:
                got = _np(xd)
                _frob(got, RK.block_full(prev_full, ol[l - 1], off, cs, H, d), prev_full, f"{what}, full layer {l}")
                prev_full = got
                prev_h, prev_c = RK.split_history_and_candidates(got, off, cs)[:2]
            else:
                if prev_c is None:
                    prev_h, prev_c = RK.split_history_and_candidates(prev_full, off, cs)[:2]
                assert np.array_equal(_np(xh), prev_h), f"{what}: the history moved"
                kh, vh = RK.history_kv(prev_h, ol[l - 1], hoff, H, d)
                got = _np(xc)
                _frob(got, RK.block_cand_only(prev_c, kh, vh, ol[l - 1], hoff, coff, H, d), prev_c,
                      f"{what}, candidate-only layer {l}")
                prev_c = got
        xc0 = RK.split_history_and_candidates(x, off, cs)[1]
        again = rr().rr_ranker_cached_fwd(to_dev(xc0.astype(np.float32)), dl, cache, to_dev(hoff.astype(np.int32)),
                                          to_dev(coff.astype(np.int32)), H, d)
        torch.cuda.synchronize()
        assert torch.equal(again, xc), f"{what}: cached request"
        b = int(np.argmax(off[1:] - cs))
        perm = np.arange(len(x))
        perm[cs[b]:off[b + 1]] = cs[b] + rng.permutation(off[b + 1] - cs[b])
        _, xc2, xh2, _ = _run(x[perm], off, cs, dl, nco, H, d)
        cperm = np.arange(int(coff[-1]))
        cperm[coff[b]:coff[b + 1]] = coff[b] + (perm[cs[b]:off[b + 1]] - cs[b])
        assert torch.equal(xh2, xh) and torch.equal(xc2, xc[to_dev(cperm)]), f"{what}: candidate order"


def test_random_user_token_sweep():
    """The same random layouts with each user's prefix rows as its user tokens, updated in the
    candidate-only layers (at least one such layer per case): per candidate-only layer the
    update of the candidates and of the user tokens against the oracle's layer on the GPU's
    own state, in relative Frobenius norm, and the other history rows frozen bit for bit;
    then the cached request equal to the full request's candidates bit for bit."""
    for i in range(N_STACK_CASES):
        _, shapes, H, d, n_layers, nco = _random_stack_case(i)
        nco = max(nco, 1)
        p = np.asarray(shapes["prefix"])
        what = f"user-token sweep {i} (B={len(p)} H={H} d={d} layers={n_layers} candidate-only={nco})"
        print(what, flush=True)
        x, off, cs, dl, ol = _setup(H, d, n_layers, seed=7900 + i, shapes=shapes)
        hoff = np.concatenate([[0], np.cumsum(cs - off[:-1])])
        coff = np.concatenate([[0], np.cumsum(off[1:] - cs)])
        n_full = n_layers - nco
        if n_full:
            _, xc, xh, _ = _run(x, off, cs, dl[:n_full], 0, H, d)
            prev_c, prev_h = _np(xc), _np(xh)
        else:
            prev_h, prev_c = RK.split_history_and_candidates(x.astype(np.float64), off, cs)[:2]
        frozen_h = prev_h.copy()
        is_p = np.zeros(len(prev_h), bool)
        for b in range(len(p)):
            is_p[hoff[b]:hoff[b] + p[b]] = True
        for l in range(n_full + 1, n_layers + 1):
            _, xc, xh, cache = _run(x, off, cs, dl[:l], l - n_full, H, d, user_tokens=p)
            got_c, got_h = _np(xc), _np(xh)
            assert np.array_equal(got_h[~is_p], frozen_h[~is_p]), f"{what}: a history row moved"
            ref_p, ref_c, _, _ = RK.block_user_token_layer(prev_h[is_p], frozen_h, prev_c, ol[l - 1], p, hoff, coff,
                                                           H, d, 10000.0, None)
            _frob(got_c, ref_c, prev_c, f"{what}, candidates, layer {l}")
            if is_p.any():
                _frob(got_h[is_p], ref_p, prev_h[is_p], f"{what}, user tokens, layer {l}")
            prev_c, prev_h = got_c, got_h
        xc0 = RK.split_history_and_candidates(x, off, cs)[1]
        again = rr().rr_ranker_cached_fwd(to_dev(xc0.astype(np.float32)), dl, cache, to_dev(hoff.astype(np.int32)),
                                          to_dev(coff.astype(np.int32)), H, d)
        torch.cuda.synchronize()
        assert torch.equal(again, xc), f"{what}: cached request"


@pytest.mark.parametrize("cfg", [3, 5])
def test_stack_full_size_sampled_users(cfg):
    """The stack as the benchmark runs it (8 layers, the last 2 candidate-only, the benchmark's
    random inputs of width D = H d) on the lognormal-history and skew batches at full size,
    with its first l layers for l = 1..8: for sampled users (the shortest and median
    histories, and on the lognormal batch the longest), each layer's update of that user's
    rows against the oracle's layer on the GPU's state of those rows before it, in relative
    Frobenius norm, and the frozen history unchanged through the candidate-only layers.
    Users never read each other's rows, so the oracle runs each sampled user alone."""
    fb = W.make_config(cfg)
    H, d = fb.H, fb.d
    n_layers, nco = 8, 2
    n_full = n_layers - nco
    x, layers = W.ranker_inputs(fb.seed + 99, fb.T, n_layers, H * d)
    dl = [(to_dev(g), to_dev(wq, torch.bfloat16), to_dev(wo, torch.bfloat16)) for g, wq, wo in layers]
    ol = [RK.Layer(g.astype(np.float64), wq.astype(np.float64), wo.astype(np.float64)) for g, wq, wo in layers]
    off, cs = fb.offsets, fb.cand_start
    hoff = np.concatenate([[0], np.cumsum(cs - off[:-1])])
    coff = np.concatenate([[0], np.cumsum(off[1:] - cs)])
    order = np.argsort(fb.hist, kind="stable")
    picks = sorted({int(order[0]), int(order[len(order) // 2])} | ({int(order[-1])} if cfg == 3 else set()))
    state = {b: x[off[b]:off[b + 1]].astype(np.float64) for b in picks}
    hist, cand = {}, {}
    for l in range(1, n_layers + 1):
        xd, xc, xh, _ = _run(x, off, cs, dl[:l], max(0, l - n_full), H, d)
        for b in picks:
            lo, hi, c = int(off[b]), int(off[b + 1]), int(cs[b])
            what = f"config {cfg} user {b} ({c - lo} history, {hi - c} candidates), layer {l}"
            if l <= n_full:
                got = _np(xd[lo:hi])
                ref = RK.block_full(state[b], ol[l - 1], np.array([0, hi - lo]), np.array([c - lo]), H, d)
                _frob(got, ref, state[b], what)
                state[b] = got
                hist[b], cand[b] = got[:c - lo], got[c - lo:]
            else:
                assert np.array_equal(_np(xh[hoff[b]:hoff[b + 1]]), hist[b]), f"{what}: the history moved"
                hb, cb = np.array([0, c - lo]), np.array([0, hi - c])
                kh, vh = RK.history_kv(hist[b], ol[l - 1], hb, H, d)
                got = _np(xc[coff[b]:coff[b + 1]])
                _frob(got, RK.block_cand_only(cand[b], kh, vh, ol[l - 1], hb, cb, H, d), cand[b], what)
                cand[b] = got
        del xd, xc, xh


@pytest.mark.parametrize("cfg", [3, 5])
def test_user_token_stack_full_size_sampled_users(cfg):
    """The benchmarked stack with each user's prefix rows as its user tokens, on the
    lognormal-history and skew batches at full size: after the full layers (checked in the
    test above), each candidate-only layer's update of a sampled user's candidates and user
    tokens against the oracle's layer on the GPU's own state of that user's rows, in
    relative Frobenius norm, and the user's other history rows frozen bit for bit."""
    fb = W.make_config(cfg)
    H, d = fb.H, fb.d
    n_layers, nco = 8, 2
    n_full = n_layers - nco
    x, layers = W.ranker_inputs(fb.seed + 99, fb.T, n_layers, H * d)
    dl = [(to_dev(g), to_dev(wq, torch.bfloat16), to_dev(wo, torch.bfloat16)) for g, wq, wo in layers]
    ol = [RK.Layer(g.astype(np.float64), wq.astype(np.float64), wo.astype(np.float64)) for g, wq, wo in layers]
    off, cs, p = fb.offsets, fb.cand_start, np.asarray(fb.prefix)
    hoff = np.concatenate([[0], np.cumsum(cs - off[:-1])])
    coff = np.concatenate([[0], np.cumsum(off[1:] - cs)])
    order = np.argsort(fb.hist, kind="stable")
    picks = sorted({int(order[0]), int(order[len(order) // 2])} | ({int(order[-1])} if cfg == 3 else set()))
    _, xc, xh, _ = _run(x, off, cs, dl[:n_full], 0, H, d)
    hist = {b: _np(xh[hoff[b]:hoff[b + 1]]) for b in picks}
    cand = {b: _np(xc[coff[b]:coff[b + 1]]) for b in picks}
    frozen = {b: hist[b].copy() for b in picks}
    del xc, xh
    for l in range(n_full + 1, n_layers + 1):
        _, xc, xh, _ = _run(x, off, cs, dl[:l], l - n_full, H, d, user_tokens=p)
        for b in picks:
            nh, nc, pb = int(cs[b] - off[b]), int(off[b + 1] - cs[b]), int(p[b])
            what = f"config {cfg} user {b} ({pb} user tokens, {nh} history, {nc} candidates), layer {l}"
            got_h, got_c = _np(xh[hoff[b]:hoff[b + 1]]), _np(xc[coff[b]:coff[b + 1]])
            assert np.array_equal(got_h[pb:], frozen[b][pb:]), f"{what}: a history row moved"
            ref_p, ref_c, _, _ = RK.block_user_token_layer(hist[b][:pb], frozen[b], cand[b], ol[l - 1], np.array([pb]),
                                                           np.array([0, nh]), np.array([0, nc]), H, d, 10000.0, None)
            _frob(got_c, ref_c, cand[b], f"{what}, candidates")
            if pb:
                _frob(got_h[:pb], ref_p, hist[b][:pb], f"{what}, user tokens")
            hist[b], cand[b] = got_h, got_c
        del xc, xh
