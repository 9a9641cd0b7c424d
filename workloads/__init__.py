"""Seeded synthetic jagged batches for the candidate-isolated attention path.

This module only draws inputs: lengths, offsets, candidate starts, padding
masks and q/k/v values.  It holds none of the method's arithmetic (no segment
rule, no mask, no softmax), so both the oracle and the HIP path can take their
inputs from it without sharing any computation.

Layout (jagged values + offsets, as in the HSTU scaling notes, section on
hand-computing padding waste and offsets): the rows of all users are
concatenated; user b owns rows ``[offsets[b], offsets[b+1])`` and, in full
sequence mode, lays them out as ``[prefix | history | candidates]`` (Candidate
isolation attention mask page, section "why it is needed").  ``cand_start[b]``
is the absolute row of user b's first candidate.  Tensors are token-major
``[rows, H, d]``.

Recipe (stated once, used by every config):
  * RNG: ``numpy.random.Generator(PCG64(seed))``; the seed of config ``i`` is
    ``1000 + i``.
  * Draw order: lengths first, from that generator; then the value tensors
    q, k, v (candidate-only mode: q_cand, k_hist, v_hist, k_cand, v_cand), the
    t-th of them (t = 0, 1, ...) a float32 standard normal of shape
    ``[rows, H, d]`` filled in C order in chunks of 2**22 values, chunk j drawn
    from ``Generator(PCG64(SeedSequence([seed, t, j])))`` (so large tensors can
    be drawn on several threads with the same result), multiplied by
    ``1/sqrt(d)`` (config 1 stays unscaled).
  * bf16 configs round every value to bf16 with round-to-nearest-even; the
    arrays stay float32 but hold only bf16-representable values, so the oracle
    (float64) and the GPU (bf16) see the same numbers.
  * Integer lengths use ``rint`` then ``clip``.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "FullBatch", "CandOnlyBatch", "round_to_bf16", "layout_full", "make_full_batch",
    "make_cand_only_batch", "config1", "config2", "config3", "config4", "config5",
    "config5_padded", "make_config", "CONFIG_NAMES", "split_to_cand_only",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bf16 value (ties to even).

    Input preparation only (finite values; NaN/inf are not produced here)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    shape = x.shape
    u = x.reshape(-1).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(shape)


@dataclass
class FullBatch:
    """A full-sequence jagged batch: every user is ``[prefix | history | candidates]``."""
    name: str
    H: int
    d: int
    dtype: str                       # "f32" or "bf16"
    prefix: np.ndarray               # [B] prefix rows per user
    hist: np.ndarray                 # [B] real history rows per user
    cand: np.ndarray                 # [B] candidate rows per user
    pad: np.ndarray                  # [B] padding rows placed before the history
    offsets: np.ndarray              # int32 [B+1]
    cand_start: np.ndarray           # int32 [B], absolute row
    valid: Optional[np.ndarray]      # uint8 [T] or None (= every row valid)
    attend_padded_history: bool
    q: np.ndarray                    # float32 [T, H, d]
    k: np.ndarray
    v: np.ndarray
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.offsets.shape[0] - 1)

    @property
    def T(self) -> int:
        return int(self.offsets[-1])


@dataclass
class CandOnlyBatch:
    """A candidate-only-layer batch: candidate q/k/v plus frozen history K/V per user."""
    name: str
    H: int
    d: int
    dtype: str
    hist_offsets: np.ndarray         # int32 [B+1] into k_hist / v_hist
    cand_offsets: np.ndarray         # int32 [B+1] into q_cand / k_cand / v_cand
    q_cand: np.ndarray               # float32 [Tc, H, d]
    k_hist: np.ndarray               # float32 [Th, H, d]
    v_hist: np.ndarray
    k_cand: np.ndarray
    v_cand: np.ndarray
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.cand_offsets.shape[0] - 1)

    @property
    def Th(self) -> int:
        return int(self.hist_offsets[-1])

    @property
    def Tc(self) -> int:
        return int(self.cand_offsets[-1])


_CHUNK = 1 << 22


def _fill_chunk(x, seed, t, j, mult, bf16):
    lo = j * _CHUNK
    part = x[lo:lo + _CHUNK]
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, t, j])))
    g.standard_normal(out=part, dtype=np.float32)
    if mult is not None:
        part *= mult
    if bf16:
        part[:] = round_to_bf16(part)


def _draw(seed: int, t: int, rows: int, H: int, d: int, scaled: bool, dtype: str) -> np.ndarray:
    n = rows * H * d
    x = np.empty(n, dtype=np.float32)
    mult = np.float32(1.0 / math.sqrt(d)) if scaled else None
    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 2:
        for j in range(nchunks):
            _fill_chunk(x, seed, t, j, mult, dtype == "bf16")
    else:
        from concurrent.futures import ThreadPoolExecutor
        workers = min(16, os.cpu_count() or 1, nchunks)
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda j: _fill_chunk(x, seed, t, j, mult, dtype == "bf16"), range(nchunks)))
    return x.reshape(rows, H, d)


def _value_seed(rng: np.random.Generator, seed: int) -> int:
    """The config's seed when given; ad-hoc batches (seed 0) take one from their generator."""
    return int(seed) if seed else int(rng.integers(1, 2**31))


def _exclusive_cumsum(lengths: np.ndarray) -> np.ndarray:
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=out[1:])
    return out


def layout_full(prefix, hist, cand, pad=None):
    """Offsets, candidate starts and the valid mask of ``[prefix | pad | history | candidates]``.

    Padding rows (if any) sit right before the history, so the newest history row
    stays right-anchored at the end of the history block (Candidate isolation
    attention mask page, section on positions shared by candidates).  Returns
    ``(offsets int32[B+1], cand_start int32[B], valid uint8[T] or None)``."""
    prefix = np.asarray(prefix, dtype=np.int64)
    hist = np.asarray(hist, dtype=np.int64)
    cand = np.asarray(cand, dtype=np.int64)
    pad = np.zeros_like(hist) if pad is None else np.asarray(pad, dtype=np.int64)
    lengths = prefix + pad + hist + cand
    offsets = _exclusive_cumsum(lengths)
    cand_start = offsets[:-1] + prefix + pad + hist
    valid = None
    if pad.any():
        valid = np.ones(int(offsets[-1]), dtype=np.uint8)
        for b in range(len(lengths)):
            p0 = offsets[b] + prefix[b]
            valid[p0:p0 + pad[b]] = 0
    if offsets[-1] > np.iinfo(np.int32).max:
        raise ValueError("row count exceeds int32 offsets")
    return offsets.astype(np.int32), cand_start.astype(np.int32), valid


def make_full_batch(rng, name, prefix, hist, cand, H, d, dtype="bf16", scaled=True,
                    pad=None, attend_padded_history=False, valid=None, seed=0, meta=None) -> FullBatch:
    """Lay out the users and draw q, k, v (in that order) for every row, padding included.

    ``valid`` (uint8 [T]) overrides the padding mask derived from ``pad``; tests use
    it to punch arbitrary holes."""
    prefix = np.broadcast_to(np.asarray(prefix, dtype=np.int64), np.shape(hist)).copy()
    hist = np.asarray(hist, dtype=np.int64)
    cand = np.broadcast_to(np.asarray(cand, dtype=np.int64), hist.shape).copy()
    padv = np.zeros_like(hist) if pad is None else np.asarray(pad, dtype=np.int64)
    offsets, cand_start, vmask = layout_full(prefix, hist, cand, padv)
    if valid is not None:
        vmask = np.asarray(valid, dtype=np.uint8)
        assert vmask.shape == (int(offsets[-1]),)
    T = int(offsets[-1])
    vseed = _value_seed(rng, seed)
    q = _draw(vseed, 0, T, H, d, scaled, dtype)
    k = _draw(vseed, 1, T, H, d, scaled, dtype)
    v = _draw(vseed, 2, T, H, d, scaled, dtype)
    return FullBatch(name=name, H=H, d=d, dtype=dtype, prefix=prefix, hist=hist, cand=cand,
                     pad=padv, offsets=offsets, cand_start=cand_start, valid=vmask,
                     attend_padded_history=attend_padded_history, q=q, k=k, v=v, seed=seed,
                     meta=dict(meta or {}))


def make_cand_only_batch(rng, name, hist, cand, H, d, dtype="bf16", scaled=True, seed=0,
                         meta=None) -> CandOnlyBatch:
    """Draw a candidate-only batch: q_cand, k_hist, v_hist, k_cand, v_cand in that order."""
    hist = np.asarray(hist, dtype=np.int64)
    cand = np.broadcast_to(np.asarray(cand, dtype=np.int64), hist.shape).copy()
    hoff = _exclusive_cumsum(hist).astype(np.int32)
    coff = _exclusive_cumsum(cand).astype(np.int32)
    Th, Tc = int(hoff[-1]), int(coff[-1])
    vseed = _value_seed(rng, seed)
    q_cand = _draw(vseed, 0, Tc, H, d, scaled, dtype)
    k_hist = _draw(vseed, 1, Th, H, d, scaled, dtype)
    v_hist = _draw(vseed, 2, Th, H, d, scaled, dtype)
    k_cand = _draw(vseed, 3, Tc, H, d, scaled, dtype)
    v_cand = _draw(vseed, 4, Tc, H, d, scaled, dtype)
    return CandOnlyBatch(name=name, H=H, d=d, dtype=dtype, hist_offsets=hoff, cand_offsets=coff,
                         q_cand=q_cand, k_hist=k_hist, v_hist=v_hist, k_cand=k_cand, v_cand=v_cand,
                         seed=seed, meta=dict(meta or {}))


def draw_output_grad(seed: int, T: int, H: int, d: int, dtype: str = "bf16",
                     scaled: bool = False) -> np.ndarray:
    """An upstream gradient dO [T, H, d] for the backward pass: N(0, 1) entries (N(0, 1/d) when
    ``scaled``), rounded to bf16 for bf16 batches; stream 3 of ``seed``."""
    return _draw(int(seed), 3, T, H, d, scaled, dtype)


def ranker_inputs(seed: int, T: int, n_layers: int, D: int):
    """Inputs of a layer stack: states x ~ N(0, 1) float32 [T, D], and per layer a norm gain
    1 + 0.1 N(0, 1) (float32 [D]) and projections W_qkv [3D, D], W_o [D, D] ~ N(0, 1/D) rounded
    to bf16 (held as float32).  Streams 10.. of ``seed``."""
    x = _draw(int(seed), 10, T, 1, D, False, "f32").reshape(T, D)
    layers = []
    for l in range(n_layers):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), 11, l])))
        gain = (1.0 + 0.1 * g.standard_normal(D)).astype(np.float32)
        w_qkv = round_to_bf16((g.standard_normal((3 * D, D)) / math.sqrt(D)).astype(np.float32))
        w_o = round_to_bf16((g.standard_normal((D, D)) / math.sqrt(D)).astype(np.float32))
        layers.append((gain, w_qkv, w_o))
    return x, layers


def split_to_cand_only(fb: FullBatch) -> CandOnlyBatch:
    """Re-express a full batch without padding as candidate-only inputs.

    Frozen history = every prefix and history row of a user (Candidate isolation
    attention mask page, section on candidate-only tail layers: the prefix and
    history states are the ones frozen); candidate rows keep their own q/k/v.
    Pure gathering of rows; no arithmetic."""
    if fb.valid is not None:
        raise ValueError("split_to_cand_only expects a batch without padding")
    B = fb.B
    hist_rows, cand_rows = [], []
    for b in range(B):
        lo, cs, hi = int(fb.offsets[b]), int(fb.cand_start[b]), int(fb.offsets[b + 1])
        hist_rows.append(np.arange(lo, cs))
        cand_rows.append(np.arange(cs, hi))
    hidx = np.concatenate(hist_rows) if hist_rows else np.zeros(0, np.int64)
    cidx = np.concatenate(cand_rows) if cand_rows else np.zeros(0, np.int64)
    hoff = _exclusive_cumsum(np.array([len(r) for r in hist_rows], dtype=np.int64)).astype(np.int32)
    coff = _exclusive_cumsum(np.array([len(r) for r in cand_rows], dtype=np.int64)).astype(np.int32)
    return CandOnlyBatch(name=fb.name + "/cand-only", H=fb.H, d=fb.d, dtype=fb.dtype,
                         hist_offsets=hoff, cand_offsets=coff, q_cand=fb.q[cidx],
                         k_hist=fb.k[hidx], v_hist=fb.v[hidx], k_cand=fb.k[cidx], v_cand=fb.v[cidx],
                         seed=fb.seed, meta={"hist_rows": hidx, "cand_rows": cidx})


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _log_uniform(rng, lo, hi, n):
    return np.clip(np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), n))), lo, hi).astype(np.int64)


def config1(seed: int = 1001) -> FullBatch:
    """Tiny fp32: B=3, prefix 1, history [2,5,1], candidates [3,2,4], H=2, d=16, q/k/v ~ N(0,1)."""
    rng = _rng(seed)
    return make_full_batch(rng, "tiny-fp32", prefix=1, hist=[2, 5, 1], cand=[3, 2, 4], H=2, d=16,
                           dtype="f32", scaled=False, seed=seed)


def config2(seed: int = 1002) -> FullBatch:
    """bf16: B=64, prefix 4, history log-uniform in [10,1000], 32 candidates, H=4, d=64."""
    rng = _rng(seed)
    hist = _log_uniform(rng, 10, 1000, 64)
    return make_full_batch(rng, "short-history-bf16", prefix=4, hist=hist, cand=32, H=4, d=64, seed=seed)


def config3(seed: int = 1003) -> FullBatch:
    """bf16: B=256, prefix 8, history lognormal(median 280, sigma 0.8) clipped to [0,2048],
    exactly round(0.02*B) users with an empty history, 128 candidates, H=8, d=64."""
    rng = _rng(seed)
    B = 256
    hist = np.clip(np.rint(rng.lognormal(math.log(280.0), 0.8, B)), 0, 2048).astype(np.int64)
    n_empty = int(round(0.02 * B))
    hist[rng.choice(B, n_empty, replace=False)] = 0
    return make_full_batch(rng, "lognormal-history-bf16", prefix=8, hist=hist, cand=128, H=8, d=64,
                           seed=seed, meta={"n_empty": n_empty})


def config4(seed: int = 1004) -> CandOnlyBatch:
    """bf16 candidate-only layer: B=512, frozen history log-uniform in [50,4000], 512 candidates,
    H=8, d=128."""
    rng = _rng(seed)
    hist = _log_uniform(rng, 50, 4000, 512)
    return make_cand_only_batch(rng, "cand-only-bf16", hist=hist, cand=512, H=8, d=128, seed=seed)


def _config5_lengths(rng):
    return rng.choice(np.array([0, 10, 100, 1000, 8192], dtype=np.int64), 32)


def config5(seed: int = 1005) -> FullBatch:
    """bf16 skew stress: B=32, history from {0,10,100,1000,8192}, prefix 4, 2048 candidates,
    H=16, d=128, no padding."""
    rng = _rng(seed)
    hist = _config5_lengths(rng)
    return make_full_batch(rng, "skew-bf16", prefix=4, hist=hist, cand=2048, H=16, d=128, seed=seed)


def config5_padded(seed: int = 1005, attend_padded_history: bool = True) -> FullBatch:
    """Config 5's length draw, each history right-anchored and padded to the batch's longest
    history (pad rows have valid=0 and q/k/v drawn like real rows)."""
    rng = _rng(seed)
    hist = _config5_lengths(rng)
    hcap = int(hist.max())
    return make_full_batch(rng, "skew-padded-bf16", prefix=4, hist=hist, cand=2048, H=16, d=128,
                           pad=hcap - hist, attend_padded_history=attend_padded_history, seed=seed,
                           meta={"hcap": hcap})


CONFIG_NAMES = {1: "tiny-fp32", 2: "short-history-bf16", 3: "lognormal-history-bf16",
                4: "cand-only-bf16", 5: "skew-bf16", 6: "skew-padded-bf16"}


def make_config(i: int, **kw):
    """Config by index: 1..5 as listed, 6 = config 5 padded (``attend_padded_history`` kwarg)."""
    return {1: config1, 2: config2, 3: config3, 4: config4, 5: config5, 6: config5_padded}[i](**kw)
