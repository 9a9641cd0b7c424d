"""Segment IDs and bounds on the GPU, bit-exact against the oracle (integer work)."""
import numpy as np
import pytest
import torch

import workloads as W
from _gpu import gpu, needs_gpu, rr, to_dev
from oracle import jagged as J

pytestmark = [gpu, needs_gpu]


def _check(offsets, cand_start, valid, flag):
    offsets = np.asarray(offsets, np.int32)
    cand_start = np.asarray(cand_start, np.int32)
    T = int(offsets[-1])
    d_off, d_cs = to_dev(offsets), to_dev(cand_start)
    d_valid = None if valid is None else to_dev(np.asarray(valid, np.uint8))
    seg = rr().rr_segment_ids(d_off, d_cs, d_valid, flag, T=T)
    bnd = rr().rr_bounds(d_off, seg)
    torch.cuda.synchronize()
    ref_seg = J.segment_ids(offsets, cand_start, valid, flag)
    ref_bnd = J.bounds(offsets, ref_seg)
    assert np.array_equal(seg.cpu().numpy(), ref_seg)
    assert np.array_equal(bnd.cpu().numpy().astype(np.int64), ref_bnd)


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_configs(cfg):
    fb = W.make_config(cfg)
    print(f"[segments] config {cfg} B={fb.B} T={fb.T}", flush=True)
    _check(fb.offsets, fb.cand_start, fb.valid, False)


@pytest.mark.parametrize("flag", [False, True])
def test_config5_padded(flag):
    fb = W.config5_padded(attend_padded_history=flag)
    print(f"[segments] config 5 padded flag={flag} T={fb.T}", flush=True)
    _check(fb.offsets, fb.cand_start, fb.valid, flag)


@pytest.mark.parametrize("seed", range(6))
def test_fuzz(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 40))
    P = rng.integers(0, 4, B)
    h = rng.integers(0, 300, B) * (rng.random(B) > 0.2)
    c = rng.integers(0, 70, B) * (rng.random(B) > 0.2)
    lens = P + h + c
    offsets = np.zeros(B + 1, np.int64)
    np.cumsum(lens, out=offsets[1:])
    cand_start = offsets[:-1] + P + h
    T = int(offsets[-1])
    valid = (rng.random(T) > 0.3).astype(np.uint8) if seed % 2 else None
    for flag in (False, True):
        _check(offsets, cand_start, valid, flag)


def test_validate_jagged():
    off = to_dev(np.array([0, 3, 3, 9], np.int32))
    assert rr().rr_validate_jagged(off, to_dev(np.array([1, 3, 9], np.int32)), T=9) == 0
    assert rr().rr_validate_jagged(off, to_dev(np.array([1, 4, 9], np.int32)), T=9) == 8
    bad = to_dev(np.array([1, 5, 3, 8], np.int32))
    assert rr().rr_validate_jagged(bad, None, T=9) == 1 | 2 | 4
