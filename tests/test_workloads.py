"""The seeded generators produce the configured structure (CPU only)."""
import numpy as np

import workloads as W


def test_config1_structure():
    fb = W.config1()
    assert fb.offsets.tolist() == [0, 6, 14, 20] and fb.cand_start.tolist() == [3, 12, 16]
    assert fb.q.shape == (20, 2, 16) and fb.valid is None and fb.dtype == "f32"


def test_config2_3_structure():
    fb = W.config2()
    assert fb.B == 64 and fb.H == 4 and fb.d == 64
    assert fb.hist.min() >= 10 and fb.hist.max() <= 1000 and np.all(fb.cand == 32)
    fb = W.config3()
    assert fb.B == 256 and fb.H == 8 and fb.d == 64
    assert (fb.hist == 0).sum() >= 5 and fb.hist.max() <= 2048 and np.all(fb.cand == 128)
    assert 200 <= np.median(fb.hist) <= 360


def test_bf16_rounding_exact():
    fb = W.config2()
    bits = fb.q.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5e-3], dtype=np.float32)
    r = W.round_to_bf16(x)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == np.float32(1.015625)   # ties to even


def test_config5_padded_layout():
    fb = W.config5()
    fp = W.config5_padded()
    assert np.array_equal(fb.hist, fp.hist) and fp.meta["hcap"] == fb.hist.max()
    assert int(fp.valid.sum()) == int(fb.T)      # every real row valid, every pad row not
    b = int(np.argmin(fp.hist))
    lo = int(fp.offsets[b])
    assert fp.valid[lo + 4: lo + 4 + int(fp.pad[b])].sum() == 0


def test_split_to_cand_only_is_a_gather():
    fb = W.config1()
    cb = W.split_to_cand_only(fb)
    assert cb.hist_offsets.tolist() == [0, 3, 9, 11] and cb.cand_offsets.tolist() == [0, 3, 5, 9]
    assert np.array_equal(cb.k_hist, fb.k[cb.meta["hist_rows"]])
