"""Helpers for the GPU parity tests: move seeded batches to the device, run the HIP path
through the C ABI, compare with the oracle at the stated tolerances."""
from __future__ import annotations

import numpy as np
import pytest
import torch

# fp32: max |err| <= 1e-5.  bf16 (fp32 accumulation): |gpu - ref| <= 2e-2 + 1e-2 * |ref|
# elementwise, against the float64 oracle on the same bf16-rounded inputs.
F32_ATOL = 1e-5
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2

gpu = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def device():
    return torch.device("cuda:0")


def torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def to_dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x)).to(device())
    return t if dtype is None else t.to(dtype)


def rr():
    from jagged_candidate_isolated_amd import rr as _rr
    return _rr


def full_dev(fb):
    dt = torch_dtype(fb.dtype)
    return dict(q=to_dev(fb.q, dt), k=to_dev(fb.k, dt), v=to_dev(fb.v, dt),
                offsets=to_dev(fb.offsets), cand_start=to_dev(fb.cand_start),
                valid=None if fb.valid is None else to_dev(fb.valid))


def run_full(fb, dev_inputs=None, **kw) -> np.ndarray:
    d = dev_inputs or full_dev(fb)
    out = rr().rr_attn_fwd(d["q"], d["k"], d["v"], d["offsets"], d["cand_start"], d["valid"],
                           fb.attend_padded_history, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def cand_only_dev(cb):
    dt = torch_dtype(cb.dtype)
    return dict(q_cand=to_dev(cb.q_cand, dt), k_hist=to_dev(cb.k_hist, dt), v_hist=to_dev(cb.v_hist, dt),
                k_cand=to_dev(cb.k_cand, dt), v_cand=to_dev(cb.v_cand, dt),
                hist_offsets=to_dev(cb.hist_offsets), cand_offsets=to_dev(cb.cand_offsets))


def run_cand_only(cb, dev_inputs=None, **kw) -> np.ndarray:
    d = dev_inputs or cand_only_dev(cb)
    out = rr().rr_cand_only_attn_fwd(d["q_cand"], d["k_hist"], d["v_hist"], d["k_cand"], d["v_cand"],
                                     d["hist_offsets"], d["cand_offsets"], **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, dtype: str, what: str = ""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if dtype == "f32":
        err = float(np.max(np.abs(got - ref))) if got.size else 0.0
        assert err <= F32_ATOL, f"{what}: fp32 max|err| {err:.3e} > {F32_ATOL}"
    else:
        excess = np.abs(got - ref) - (BF16_ATOL + BF16_RTOL * np.abs(ref))
        worst = float(excess.max()) if got.size else -1.0
        if worst > 0:
            i = np.unravel_index(int(np.argmax(excess)), excess.shape)
            raise AssertionError(f"{what}: bf16 tolerance exceeded at {i}: got {got[i]} ref {ref[i]}")


# bf16 gradients: P and dS enter their products rounded to bf16 and o, dq, dk, dv are
# stored in bf16 (unit roundoff u = 2^-8), with fp32 accumulation.  Rounding-error
# analysis bounds each element by u (E + |grad|), E the oracle's gradient_error_scale;
# the factor 1.25 covers fp32 accumulation over up to 2^14 terms (2^14 * 2^-24 = u / 4)
# and P's fp32 evaluation (about 1e-6 relative).
GRAD_U, GRAD_C = 2.0 ** -8, 1.25


def assert_close_grad(got, ref, escale, what: str = ""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape == np.shape(escale), (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    if not got.size:
        return
    excess = np.abs(got - ref) - GRAD_C * GRAD_U * (np.asarray(escale) + np.abs(ref))
    worst = float(excess.max())
    if worst > 0:
        i = np.unravel_index(int(np.argmax(excess)), excess.shape)
        raise AssertionError(f"{what}: gradient bound exceeded at {i}: got {got[i]} ref {ref[i]} "
                             f"scale {np.asarray(escale)[i]}")


def sample_full_rows(fb, per_user: int, seed: int):
    """Stratified (row, head) samples: every user's first and last row, first and last
    candidate, last history row, plus ``per_user`` random rows, each with a random head."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(fb.B):
        lo, cs, hi = int(fb.offsets[b]), int(fb.cand_start[b]), int(fb.offsets[b + 1])
        if hi == lo:
            continue
        pick = {lo, hi - 1}
        if cs < hi:
            pick |= {cs, hi - 1}
        if cs > lo:
            pick.add(cs - 1)
        pick |= set(int(x) for x in rng.integers(lo, hi, per_user))
        rows.extend(sorted(pick))
    rows = np.array(rows, dtype=np.int64)
    heads = rng.integers(0, fb.H, len(rows))
    return rows, heads


def sample_cand_rows(cb, per_user: int, seed: int):
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(cb.B):
        lo, hi = int(cb.cand_offsets[b]), int(cb.cand_offsets[b + 1])
        if hi == lo:
            continue
        pick = {lo, hi - 1} | set(int(x) for x in rng.integers(lo, hi, per_user))
        rows.extend(sorted(pick))
    rows = np.array(rows, dtype=np.int64)
    heads = rng.integers(0, cb.H, len(rows))
    return rows, heads
