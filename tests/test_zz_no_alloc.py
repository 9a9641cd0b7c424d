"""The entry point that allocates nothing (rr_attn_fwd_noalloc) against rr_attn_fwd with a
workspace, through the C ABI: identical outputs on consecutive calls that share the
library's static array, each later call with a smaller batch, on the separate-plan path
of long users (wide tiles, whose key-norm bounds also live in the array), on the
in-kernel-plan path and on the separate-plan path with a padding mask; and the size limit
refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from _gpu import assert_close, full_dev, gpu, needs_gpu, rr
from oracle import attention as A

pytestmark = [gpu, needs_gpu]


def _batches():
    rng = np.random.default_rng(515)
    # users averaging >= 2048 rows (wide tiles) and a grid above the in-kernel-plan limit
    wide = W.make_full_batch(rng, "noalloc-wide", prefix=[4, 2, 0], hist=[3000, 2500, 3500], cand=[1000, 1400, 600],
                             H=24, d=128, seed=5150)
    big = W.make_full_batch(rng, "noalloc-big", prefix=[4, 0, 2, 3, 1], hist=[900, 0, 333, 1500, 70],
                            cand=[40, 7, 129, 300, 2], pad=[20, 0, 5, 100, 0], H=3, d=64,
                            attend_padded_history=False, seed=5151)
    small = W.make_full_batch(rng, "noalloc-small", prefix=[2, 1], hist=[120, 0], cand=[9, 33], H=2, d=128,
                              seed=5152)
    padded_small = W.make_full_batch(rng, "noalloc-small-pad", prefix=[1], hist=[60], cand=[5], pad=[7], H=2,
                                     d=64, attend_padded_history=True, seed=5153)
    return wide, big, small, padded_small


def test_no_alloc_equals_workspace_path():
    R = rr()
    for fb in _batches():           # consecutive calls share the static plan; later ones are smaller
        dev = full_dev(fb)
        print(f"[no-alloc] {fb.name} B={fb.B} T={fb.T} H={fb.H} d={fb.d} padded={fb.valid is not None}", flush=True)
        ref = R.rr_attn_fwd(dev["q"], dev["k"], dev["v"], dev["offsets"], dev["cand_start"], dev["valid"],
                            fb.attend_padded_history)
        out = torch.full_like(dev["q"], float("nan"))
        got = R.rr_attn_fwd_noalloc(dev["q"], dev["k"], dev["v"], dev["offsets"], dev["cand_start"], out,
                                    dev["valid"], fb.attend_padded_history)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(out, ref), f"{fb.name}: no-alloc output differs from the workspace path"
        got_np = out.float().cpu().numpy()
        if fb.name == "noalloc-wide":   # sampled rows (the dense oracle on the whole batch is slow)
            rows = np.concatenate([np.r_[lo:lo + 3, cs - 2:cs + 2, hi - 3:hi] for lo, cs, hi in
                                   zip(fb.offsets[:-1], fb.cand_start, fb.offsets[1:])])
            heads = np.arange(len(rows)) % fb.H
            want = A.full_attention_rows(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, rows, heads)
            assert_close(got_np[rows, heads], want, "bf16", fb.name)
            continue
        want = A.full_attention(fb.q, fb.k, fb.v, fb.offsets, fb.cand_start, fb.valid, fb.attend_padded_history)
        assert_close(got_np, want, "bf16", fb.name)


def test_no_alloc_limit_refused_on_the_host():
    R = rr()
    lib = R._lib
    cap = lib.rr_attn_fwd_noalloc_max_bytes()
    assert cap == 16 << 20
    # the smallest row count whose plan does not fit: nothing is launched for it
    T = 1
    while lib.rr_attn_workspace_bytes(1, T, 8, 64) <= cap:
        T *= 2
    fake = ctypes.c_void_p(0x1000)
    st = lib.rr_attn_fwd_noalloc(fake, fake, fake, fake, fake, fake, None, 0, 1, T, 8, 64, R.RR_BF16, 0.0, None)
    assert st == R.RR_EUNSUPPORTED
    assert lib.rr_attn_fwd_noalloc(None, None, None, None, None, None, None, 0, 0, 0, 8, 64, R.RR_BF16, 0.0,
                                   None) == R.RR_OK
