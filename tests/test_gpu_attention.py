"""Attention parity on the GPU: the HIP path (through the C ABI) against the float64 oracle.

Small cases compare every output element; the full-size workloads compare stratified
samples of (row, head) outputs that the oracle computes one by one, plus properties that
hold at any size (candidate isolation and cross-user independence bit for bit,
determinism, candidate-only == full-mode candidate rows)."""
import numpy as np
import pytest
import torch

import workloads as W
from _gpu import (assert_close, cand_only_dev, full_dev, gpu, needs_gpu, run_cand_only, run_full,
                  sample_cand_rows, sample_full_rows)
from oracle import attention as A

pytestmark = [gpu, needs_gpu]


def _oracle_full(fb):
    return A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, fb.valid,
                            fb.attend_padded_history)


def _log(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- small cases, every element

def test_config1_fp32():
    fb = W.config1()
    got = run_full(fb)
    assert_close(got, _oracle_full(fb), "f32", "config1")


def _fuzz_batch(seed, dtype, d, H, holes, flag):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(2, 9))
    P = rng.integers(0, 5, B)
    h = rng.integers(0, 330, B) * (rng.random(B) > 0.15)
    c = rng.integers(0, 150, B) * (rng.random(B) > 0.15)
    h[0] = 257   # spans several key tiles with a ragged tail
    c[0] = 131   # spans two query tiles with a ragged tail
    if B > 2:
        P[1] = h[1] = c[1] = 0          # an empty user
        P[2], h[2] = 0, 0               # candidates only: each reads just itself
    lens = P + h + c
    valid = None
    if holes:
        valid = (rng.random(int(lens.sum())) > 0.25).astype(np.uint8)
    return W.make_full_batch(rng, f"fuzz{seed}", prefix=P, hist=h, cand=c, H=H, d=d, dtype=dtype,
                             scaled=(dtype == "bf16"), valid=valid, attend_padded_history=flag,
                             seed=5000 + seed)


CASES = [(dtype, d, holes, flag)
         for dtype in ("f32", "bf16") for d in (16, 32, 64, 128)
         for holes, flag in ((False, False), (True, False), (True, True))]


@pytest.mark.parametrize("dtype,d,holes,flag", CASES)
def test_fuzz_every_element(dtype, d, holes, flag):
    fb = _fuzz_batch(CASES.index((dtype, d, holes, flag)), dtype, d, 2, holes, flag)
    _log(f"[fuzz] dtype={dtype} d={d} holes={holes} flag={flag} B={fb.B} T={fb.T}")
    got = run_full(fb)
    assert_close(got, _oracle_full(fb), dtype, f"fuzz {dtype} d={d}")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128), ("bf16", 32)])
def test_cand_only_every_element(dtype, d):
    rng = np.random.default_rng(77 + d)
    hist = np.array([0, 1, 63, 64, 65, 300, 129, 5])
    cand = np.array([3, 0, 130, 1, 64, 128, 7, 257])
    cb = W.make_cand_only_batch(rng, "co", hist=hist, cand=cand, H=3, d=d, dtype=dtype,
                                scaled=(dtype == "bf16"), seed=900 + d)
    _log(f"[cand-only] dtype={dtype} d={d} Th={cb.Th} Tc={cb.Tc}")
    got = run_cand_only(cb)
    ref = A.cand_only_attention(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand,
                                cb.hist_offsets, cb.cand_offsets)
    assert_close(got, ref, dtype, f"cand-only {dtype} d={d}")


def test_config2_every_element():
    fb = W.config2()
    _log(f"[config2] T={fb.T}")
    got = run_full(fb)
    assert_close(got, _oracle_full(fb), "bf16", "config2")


# ---------------------------------------------------------------- full sizes, sampled

@pytest.mark.parametrize("cfg", [3, 5])
def test_full_size_sampled(cfg):
    fb = W.make_config(cfg)
    _log(f"[config{cfg}] B={fb.B} T={fb.T} H={fb.H} d={fb.d}")
    got = run_full(fb)
    rows, heads = sample_full_rows(fb, 6, seed=cfg)
    ref = A.full_attention_rows(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, rows, heads)
    assert_close(got[rows, heads], ref, "bf16", f"config{cfg} sampled")


@pytest.mark.parametrize("flag", [True, False])
def test_config5_padded_sampled(flag):
    fb = W.config5_padded(attend_padded_history=flag)
    _log(f"[config5-pad] flag={flag} T={fb.T}")
    got = run_full(fb)
    rows, heads = sample_full_rows(fb, 6, seed=11)
    ref = A.full_attention_rows(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, rows, heads,
                                fb.valid, flag)
    assert_close(got[rows, heads], ref, "bf16", f"config5-pad flag={flag}")
    if not flag:
        assert np.all(got[fb.valid == 0] == 0.0)


def test_config4_cand_only_sampled():
    cb = W.config4()
    _log(f"[config4] Th={cb.Th} Tc={cb.Tc}")
    got = run_cand_only(cb)
    rows, heads = sample_cand_rows(cb, 3, seed=4)
    ref = A.cand_only_attention_rows(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand,
                                     cb.hist_offsets, cb.cand_offsets, rows, heads)
    assert_close(got[rows, heads], ref, "bf16", "config4 sampled")


# ---------------------------------------------------------------- properties, bit for bit

def _property_batch(dtype="bf16", d=128):
    rng = np.random.default_rng(31)
    return W.make_full_batch(rng, "prop", prefix=[4, 2, 0, 3], hist=[700, 90, 0, 260],
                             cand=[300, 40, 5, 129], H=4, d=d, dtype=dtype, seed=3131)


@pytest.mark.parametrize("d", [64, 128])
def test_candidate_isolation_bit_identical(d):
    fb = _property_batch(d=d)
    base = run_full(fb)
    b = 0
    cs, hi = int(fb.cand_start[b]), int(fb.offsets[b + 1])
    rng = np.random.default_rng(5)
    perm = np.arange(fb.T)
    perm[cs:hi] = cs + rng.permutation(hi - cs)
    fb2 = W.FullBatch(**{**fb.__dict__, "q": fb.q[perm], "k": fb.k[perm], "v": fb.v[perm]})
    got = run_full(fb2)
    assert np.array_equal(got, base[perm]), "candidate permutation changed outputs"
    # remove all but 3 candidates of user 0
    keep = np.r_[0:cs + 3, hi:fb.T]
    drop = hi - cs - 3
    off = fb.offsets.copy(); off[b + 1:] -= drop
    cst = fb.cand_start.copy(); cst[b + 1:] -= drop
    fb3 = W.FullBatch(**{**fb.__dict__, "q": fb.q[keep], "k": fb.k[keep], "v": fb.v[keep],
                         "offsets": off, "cand_start": cst})
    got3 = run_full(fb3)
    assert np.array_equal(got3, base[keep]), "removing candidates changed other outputs"


def test_history_and_cross_user_bit_identical():
    fb = _property_batch()
    base = run_full(fb)
    q, k, v = fb.q.copy(), fb.k.copy(), fb.v.copy()
    for b in range(fb.B):                     # change every candidate
        s = slice(int(fb.cand_start[b]), int(fb.offsets[b + 1]))
        q[s] = W.round_to_bf16(q[s] * 2 + 0.5); k[s] = W.round_to_bf16(-k[s]); v[s] = v[s] + 64
    got = run_full(W.FullBatch(**{**fb.__dict__, "q": q, "k": k, "v": v}))
    for b in range(fb.B):
        s = slice(int(fb.offsets[b]), int(fb.cand_start[b]))
        assert np.array_equal(got[s], base[s]), f"history of user {b} depends on candidates"
    q, k, v = fb.q.copy(), fb.k.copy(), fb.v.copy()
    s3 = slice(int(fb.offsets[3]), int(fb.offsets[4]))
    q[s3] = W.round_to_bf16(q[s3] * 3); v[s3] = 100.0
    got = run_full(W.FullBatch(**{**fb.__dict__, "q": q, "k": k, "v": v}))
    s012 = slice(0, int(fb.offsets[3]))
    assert np.array_equal(got[s012], base[s012]), "users 0-2 depend on user 3"


@pytest.mark.parametrize("d", [64, 128])
def test_deterministic_repeat(d):
    """Run-to-run bit identity (scores may be cached; a hazard or race shows up here)."""
    fb = _property_batch(d=d)
    dev = full_dev(fb)
    a = run_full(fb, dev)
    for i in range(7):
        assert np.array_equal(run_full(fb, dev), a), f"run {i + 1} differs"
    fb3 = W.config3()
    dev3 = full_dev(fb3)
    a3 = run_full(fb3, dev3)
    for _ in range(2):
        assert np.array_equal(run_full(fb3, dev3), a3)


@pytest.mark.parametrize("d", [64, 128])
def test_cand_only_equals_full_mode_rows(d):
    fb = _property_batch(d=d)
    full = run_full(fb)
    cb = W.split_to_cand_only(fb)
    co = run_cand_only(cb)
    assert np.array_equal(co, full[cb.meta["cand_rows"]])


# ---------------------------------------------------------------- random small batches

def test_random_batches_both_modes():
    """Twenty-four random small batches (users, lengths, heads, head width, padding holes
    and flag drawn per batch): every element of the full-sequence output against the
    oracle, and for unpadded bf16 batches the candidate-only layer against the oracle and
    bit for bit against the full mode's candidate rows."""
    rng = np.random.default_rng(2024)
    for i in range(24):
        B = int(rng.integers(1, 12))
        d = int(rng.choice([16, 32, 64, 128]))
        dtype = "f32" if d == 16 or rng.random() < 0.25 else "bf16"
        H = int(rng.integers(1, 5))
        P = rng.integers(0, 4, B)
        h = rng.integers(0, 200, B) * (rng.random(B) > 0.2)
        c = rng.integers(0, 140, B) * (rng.random(B) > 0.2)
        holes = bool(rng.random() < 0.3)
        flag = bool(holes and rng.random() < 0.5)
        lens = P + h + c
        valid = (rng.random(int(lens.sum())) > 0.3).astype(np.uint8) if holes else None
        fb = W.make_full_batch(rng, f"rand{i}", prefix=P, hist=h, cand=c, H=H, d=d, dtype=dtype,
                               scaled=(dtype == "bf16"), valid=valid, attend_padded_history=flag,
                               seed=9300 + i)
        _log(f"[random {i}] B={B} T={fb.T} H={H} d={d} {dtype} holes={holes} flag={flag}")
        full = run_full(fb)
        assert_close(full, _oracle_full(fb), dtype, f"random batch {i}")
        if not holes and dtype == "bf16":
            cb = W.split_to_cand_only(fb)
            co = run_cand_only(cb)
            ref = A.cand_only_attention(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand,
                                        cb.hist_offsets, cb.cand_offsets)
            assert_close(co, ref, dtype, f"random batch {i}, candidate-only")
            assert np.array_equal(co, full[cb.meta["cand_rows"]]), f"random batch {i}"


# ---------------------------------------------------------------- more users than the in-LDS sort

# The work-list builder sorts up to 2048 users in LDS; larger batches keep the user order
# and read the per-user counts back from global memory.
MANY_USERS = 3000


def _many_users_batch(seed, holes=False, flag=False, d=64):
    rng = np.random.default_rng(seed)
    B = MANY_USERS
    P = rng.integers(0, 3, B)
    h = rng.integers(0, 40, B) * (rng.random(B) > 0.1)
    c = rng.integers(0, 6, B) * (rng.random(B) > 0.1)
    h[::97] = 130   # some users span three key tiles
    c[::89] = 131   # and some two query tiles
    lens = P + h + c
    valid = (rng.random(int(lens.sum())) > 0.2).astype(np.uint8) if holes else None
    return W.make_full_batch(rng, f"many{seed}", prefix=P, hist=h, cand=c, H=2, d=d, valid=valid,
                             attend_padded_history=flag, seed=7000 + seed)


@pytest.mark.parametrize("holes,flag", [(False, False), (True, False), (True, True)])
def test_more_users_than_the_lds_sort(holes, flag):
    fb = _many_users_batch(1 + 2 * holes + flag, holes, flag)
    _log(f"[many users] B={fb.B} T={fb.T} holes={holes} flag={flag}")
    assert fb.B > 2048
    assert_close(run_full(fb), _oracle_full(fb), "bf16", f"{fb.B} users holes={holes} flag={flag}")


def test_cand_only_more_users_than_the_lds_sort():
    fb = _many_users_batch(9, d=128)
    _log(f"[many users, candidate-only] B={fb.B} T={fb.T}")
    full = run_full(fb)
    cb = W.split_to_cand_only(fb)
    co = run_cand_only(cb)
    ref = A.cand_only_attention(cb.q_cand, cb.k_hist, cb.v_hist, cb.k_cand, cb.v_cand,
                                cb.hist_offsets, cb.cand_offsets)
    assert_close(co, ref, "bf16", f"candidate-only, {cb.B} users")
    assert np.array_equal(co, full[cb.meta["cand_rows"]])


# ---------------------------------------------------------------- sentinels and edge cases

@pytest.mark.parametrize("flag", [False, True])
def test_sentinel_forbidden_values(flag):
    """Forbidden keys (other candidates, padding under flag False) carry V = +1e3 (bf16)."""
    rng = np.random.default_rng(41)
    fb = W.make_full_batch(rng, "sentinel", prefix=[2, 1, 3], hist=[200, 40, 500], cand=[150, 9, 64],
                           pad=[30, 0, 77], H=2, d=64, dtype="bf16", attend_padded_history=flag,
                           seed=4141)
    v = fb.v.copy()
    for b in range(fb.B):
        v[int(fb.cand_start[b]):int(fb.offsets[b + 1])] = 1000.0
    if not flag:
        v[fb.valid == 0] = 1000.0
    fb = W.FullBatch(**{**fb.__dict__, "v": v})
    assert_close(run_full(fb), _oracle_full(fb), "bf16", f"sentinel flag={flag}")


def test_no_history_candidates_read_themselves():
    rng = np.random.default_rng(8)
    fb = W.make_full_batch(rng, "self-only", prefix=[0, 0], hist=[0, 0], cand=[200, 3], H=2, d=128,
                           seed=808)
    got = run_full(fb)
    assert np.array_equal(got, fb.v.astype(np.float64))
    cb = W.make_cand_only_batch(rng, "co-self", hist=[0, 0], cand=[130, 1], H=2, d=64, seed=809)
    assert np.array_equal(run_cand_only(cb), cb.v_cand.astype(np.float64))


def test_empty_and_degenerate_batches():
    rng = np.random.default_rng(9)
    fb = W.make_full_batch(rng, "empties", prefix=[0, 1, 0], hist=[0, 0, 0], cand=[0, 0, 0], H=1,
                           d=64, seed=909)
    got = run_full(fb)
    assert np.array_equal(got, fb.v.astype(np.float64))   # one single-row user: reads itself
    import torch as _t
    from _gpu import rr as _rr
    q = _t.zeros((0, 2, 64), dtype=_t.bfloat16, device="cuda")
    off = _t.zeros(4, dtype=_t.int32, device="cuda")
    cs = _t.zeros(3, dtype=_t.int32, device="cuda")
    out = _rr().rr_attn_fwd(q, q, q, off, cs)
    _t.cuda.synchronize()
    assert out.shape == (0, 2, 64)


def test_scale_argument():
    fb = _fuzz_batch(3, "f32", 32, 2, False, False)
    got = run_full(fb, scale=0.37)
    ref = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, scale=0.37)
    assert_close(got, ref, "f32", "scale 0.37")


@pytest.mark.parametrize("cfg", [2, "ragged64", "ragged128"])
def test_self_planned_equals_planned(cfg):
    """rr_attn_fwd on a small unpadded batch builds the work list inside the attention
    kernel; the outputs equal, bit for bit, those of the separate plan + run (and the
    oracle, on config 2: test_config2_every_element)."""
    from _gpu import rr
    if cfg == 2:
        fb = W.config2()
    else:
        d = 64 if cfg.endswith("64") else 128
        rng = np.random.default_rng(d)
        fb = W.make_full_batch(rng, "self-plan", prefix=[4, 0, 2, 0, 3], hist=[900, 0, 17, 0, 250],
                               cand=[32, 5, 0, 0, 129], H=3, d=d, seed=9000 + d)
    dev = full_dev(fb)
    fused = run_full(fb, dev)
    T, H, d = fb.q.shape
    ws = rr().rr_attn_plan(dev["offsets"], dev["cand_start"], T, H, d, dev["q"].dtype)
    out = rr().rr_attn_run(dev["q"], dev["k"], dev["v"], fb.B, ws)
    torch.cuda.synchronize()
    planned = out.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(fused, planned)
    if cfg != 2:
        assert_close(fused, _oracle_full(fb), "bf16", f"self-planned {cfg}")


@pytest.mark.parametrize("B", [1, 17, 64, 65, 100, 256])
def test_self_planned_random_batches(B):
    """In-kernel planning on random small batches (many users in one key-count bucket,
    empty users, users with no history): bit-identical to plan + run."""
    from _gpu import rr
    rng = np.random.default_rng(B)
    P = rng.integers(0, 4, B)
    h = np.where(rng.random(B) < 0.5, 37, rng.integers(0, 200 if B <= 100 else 60, B)) * (rng.random(B) > 0.1)
    c = rng.integers(0, 40, B) * (rng.random(B) > 0.1)
    H = 2 if B <= 100 else 1
    fb = W.make_full_batch(rng, f"selfplan{B}", prefix=P, hist=h, cand=c, H=H, d=64, seed=9100 + B)
    # the library plans in-kernel for at most 256 users and a grid of at most 1024 workgroups
    grid = -(-(H + 1) * (-(-fb.T // 128) + B) // 256) * 256
    assert fb.T < 2048 * B and grid <= 1024, "the batch must take the in-kernel planning path"
    dev = full_dev(fb)
    fused = run_full(fb, dev)
    ws = rr().rr_attn_plan(dev["offsets"], dev["cand_start"], fb.T, fb.H, fb.d, dev["q"].dtype)
    out = rr().rr_attn_run(dev["q"], dev["k"], dev["v"], fb.B, ws)
    torch.cuda.synchronize()
    assert np.array_equal(fused, out.float().cpu().numpy().astype(np.float64))
    rows, heads = sample_full_rows(fb, per_user=1, seed=B)
    assert_close(fused[rows, heads], A.full_attention_rows(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, rows,
                                                           heads), "bf16", f"self-planned B={B}")


@pytest.mark.parametrize("d", [64, 128])
def test_maximum_heads(d):
    """H = 1023, the largest head count a work item can carry: full-sequence and
    candidate-only attention on a small batch, every head of sampled rows against the
    oracle, and the head past the limit rejected."""
    from _gpu import rr
    rng = np.random.default_rng(d)
    H = 1023
    fb = W.make_full_batch(rng, "max-heads", prefix=[1, 0], hist=[40, 3], cand=[5, 2], H=H, d=d,
                           seed=9300 + d)
    got = run_full(fb)
    rows = np.array([0, 20, 40, 41, 45, 46, 49, 50], dtype=np.int64)
    rows = rows[rows < fb.T]
    for h in (0, 511, 1022):
        ref = A.full_attention_rows(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, rows,
                                    np.full(len(rows), h))
        assert_close(got[rows, h], ref, "bf16", f"H=1023 head {h}")
    cb = W.split_to_cand_only(fb)
    co = run_cand_only(cb)
    assert np.array_equal(co, got[cb.meta["cand_rows"]])
    q = torch.zeros((4, H + 1, d), dtype=torch.bfloat16, device="cuda")
    off = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    with pytest.raises(rr().RRError):
        rr().rr_attn_fwd(q, q, q, off, torch.tensor([2], dtype=torch.int32, device="cuda"))


def test_user_keys_past_2_gib():
    """One user whose key rows span more than 2 GiB (H = 1023, d = 128: 262 KB a row, 8304
    keys), so its full key tiles leave the 32-bit buffer ranges for 64-bit addresses, and
    a second user whose rows start past 2 GiB: sampled rows and heads against the oracle
    (only those rows of the 2.2 GB output come back to the host)."""
    from _gpu import rr
    H, d = 1023, 128
    fb = W.make_full_batch(np.random.default_rng(5), "keys-past-2gib", prefix=[4, 2], hist=[8300, 60],
                           cand=[16, 9], H=H, d=d, seed=9500)
    assert (int(fb.cand_start[0]) - int(fb.offsets[0])) * H * d * 2 > 2 ** 31
    _log(f"[keys past 2 GiB] B={fb.B} T={fb.T} H={H} d={d}")
    dev = full_dev(fb)
    out = rr().rr_attn_fwd(dev["q"], dev["k"], dev["v"], dev["offsets"], dev["cand_start"])
    lo2 = int(fb.offsets[1])
    rows = np.array([0, 3, 4, 4150, 8303, 8304, 8312, 8319, lo2, lo2 + 61, fb.T - 1], dtype=np.int64)
    heads = np.array([0, 1022, 511, 7, 1000, 300, 0, 1022, 5, 600, 1022], dtype=np.int64)
    got = out[torch.from_numpy(rows).cuda(), torch.from_numpy(heads).cuda()].float().cpu().numpy()
    del out, dev
    torch.cuda.empty_cache()
    ref = A.full_attention_rows(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, rows, heads)
    assert_close(got.astype(np.float64), ref, "bf16", "keys past 2 GiB")


def test_one_long_user():
    """A single user of 60,000 rows (one long key chain per query tile, offsets far past
    16 bits): sampled rows against the oracle, and candidates read only history + self."""
    fb = W.make_full_batch(np.random.default_rng(3), "long-user", prefix=[4], hist=[59000], cand=[996],
                           H=2, d=128, seed=9400)
    got = run_full(fb)
    rows, heads = sample_full_rows(fb, per_user=24, seed=4)
    assert_close(got[rows, heads], A.full_attention_rows(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, rows,
                                                         heads), "bf16", "one long user")
