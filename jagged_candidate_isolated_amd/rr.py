"""Python binding of librr: the C ABI's calls under the same names.

Argument marshalling only -- every step of the computation runs in librr's HIP
kernels.  PyTorch supplies device memory and the current stream.  Importing this
module fails loudly when librr.so has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librr.so")

RR_OK, RR_EINVAL, RR_EDTYPE, RR_EUNSUPPORTED, RR_EWORKSPACE, RR_EHIP = 0, -1, -2, -3, -4, -5
RR_F32, RR_BF16 = 0, 1

_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "rr_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "rr_abi_version": (ctypes.c_int, []),
    "rr_forward_fingerprint": (ctypes.c_char_p, []),
    "rr_segment_ids": (ctypes.c_int, [_P, _P, _P, ctypes.c_int, _I, _I, _P, _P]),
    "rr_bounds": (ctypes.c_int, [_P, _P, _I, _I, _P, _P]),
    "rr_attn_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "rr_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_int, _I, _I, _I, _I,
                                   ctypes.c_int, ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "rr_cand_only_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "rr_cand_only_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                             ctypes.c_int, ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "rr_validate_jagged": (ctypes.c_int, [_P, _P, _I, _I, _P, _P]),
    "rr_rope_positions": (ctypes.c_int, [_P, _P, _P, _I, _I, _P, _P]),
    "rr_rope_qk": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int,
                                  ctypes.c_float, _P]),
    "rr_attn_plan": (ctypes.c_int, [_P, _P, _P, ctypes.c_int, _I, _I, _I, _I, ctypes.c_int, _P,
                                    ctypes.c_size_t, _P]),
    "rr_attn_run": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, ctypes.c_float, _P,
                                   ctypes.c_size_t, _P]),
    "rr_attn_run_lse": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, ctypes.c_float,
                                       _P, ctypes.c_size_t, _P]),
    "rr_attn_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "rr_attn_bwd_run": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int,
                                       ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "rr_attn_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int, _I, _I,
                                   _I, _I, ctypes.c_int, ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "rr_rms_norm": (ctypes.c_int, [_P, _P, _P, _I, _I, ctypes.c_float, _P]),
    "rr_linear": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _P]),
    "rr_ranker_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I]),
    "rr_ranker_fwd": (ctypes.c_int, [_P, _P, _I, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P,
                                     _P, _P, _P, ctypes.c_size_t, _P]),
    "rr_user_token_attn_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "rr_user_token_attn_plan": (ctypes.c_int, [_P, _P, _I, _I, _I, _I, _I, ctypes.c_int, _P, ctypes.c_size_t,
                                               _P]),
    "rr_user_token_attn_run": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int, ctypes.c_float,
                                              _P, ctypes.c_size_t, _P]),
    "rr_ranker_cached_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "rr_ranker_cached_fwd": (ctypes.c_int, [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _P,
                                            ctypes.c_size_t, _P]),
    "rr_cand_only_run_lse": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int,
                                            ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "rr_cand_only_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "rr_cand_only_bwd_run": (ctypes.c_int, [_P] * 15 + [_I, _I, _I, _I, _I, ctypes.c_int, ctypes.c_float, _P,
                                                        ctypes.c_size_t, _P]),
    "rr_cand_only_plan": (ctypes.c_int, [_P, _P, _I, _I, _I, _I, _I, ctypes.c_int, _P,
                                         ctypes.c_size_t, _P]),
    "rr_cand_only_run": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int,
                                        ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "rr_attn_fwd_rope": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "rr_cand_only_attn_fwd_rope": (ctypes.c_int, [_P] * 8 + [_I, _I, _I, _I, _I, ctypes.c_int, ctypes.c_float,
                                                             ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "rr_attn_fwd_noalloc_max_bytes": (ctypes.c_size_t, []),
    "rr_attn_fwd_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_int, _I, _I, _I, _I, ctypes.c_int,
                                           ctypes.c_float, _P]),
}


def load_library(path: str = _LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m jagged_candidate_isolated_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = load_library()
LIBRARY_PATH = _LIB_PATH


class RRError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {_lib.rr_status_string(status).decode()} (status {status})")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != RR_OK:
        raise RRError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _rr_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RR_F32
    if t.dtype == torch.bfloat16:
        return RR_BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def rr_segment_ids(offsets, cand_start, valid=None, attend_padded_history=False, out=None,
                   T: Optional[int] = None, stream=None) -> torch.Tensor:
    """Per-row segment IDs (int8 [T]).  ``T`` defaults to ``valid.numel()`` or ``out.numel()``;
    otherwise it must be given (the library never reads sizes back from the device)."""
    dev = offsets.device
    _need(offsets, "offsets", torch.int32)
    _need(cand_start, "cand_start", torch.int32, dev)
    if valid is not None:
        _need(valid, "valid", torch.uint8, dev)
    if T is None:
        T = valid.numel() if valid is not None else (out.numel() if out is not None else None)
    if T is None:
        raise ValueError("T is required")
    B = offsets.numel() - 1
    if out is None:
        out = torch.empty(T, dtype=torch.int8, device=dev)
    _need(out, "out", torch.int8, dev)
    _check("rr_segment_ids", _lib.rr_segment_ids(_ptr(offsets), _ptr(cand_start), _ptr(valid),
                                                 int(bool(attend_padded_history)), B, T, _ptr(out),
                                                 _stream(stream, dev)))
    return out


def rr_bounds(offsets, seg, out=None, stream=None) -> torch.Tensor:
    """Per-user [hist_lo, hist_hi, cand_lo, cand_hi] as int32 [4, B]."""
    dev = offsets.device
    _need(offsets, "offsets", torch.int32)
    _need(seg, "seg", torch.int8, dev)
    B = offsets.numel() - 1
    if out is None:
        out = torch.empty((4, B), dtype=torch.int32, device=dev)
    _need(out, "out", torch.int32, dev)
    _check("rr_bounds", _lib.rr_bounds(_ptr(offsets), _ptr(seg), B, seg.numel(), _ptr(out),
                                       _stream(stream, dev)))
    return out


def rr_attn_workspace_bytes(B: int, T: int, H: int, d: int) -> int:
    return int(_lib.rr_attn_workspace_bytes(B, T, H, d))


def rr_cand_only_workspace_bytes(B: int, Th: int, Tc: int, H: int, d: int) -> int:
    return int(_lib.rr_cand_only_workspace_bytes(B, Th, Tc, H, d))


def _workspace(nbytes: int, workspace, dev) -> torch.Tensor:
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    return workspace


def rr_attn_fwd(q, k, v, offsets, cand_start, valid=None, attend_padded_history=False, scale=None,
                out=None, workspace=None, stream=None) -> torch.Tensor:
    """Full-sequence candidate-isolated attention.  q, k, v: [T, H, d] float32 or bfloat16."""
    dev = q.device
    _need(q, "q")
    dt = _rr_dtype(q)
    for name, t in (("k", k), ("v", v)):
        _need(t, name, q.dtype, dev)
        if t.shape != q.shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != q shape {tuple(q.shape)}")
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d]")
    _need(offsets, "offsets", torch.int32, dev)
    _need(cand_start, "cand_start", torch.int32, dev)
    if valid is not None:
        _need(valid, "valid", torch.uint8, dev)
    T, H, d = q.shape
    B = offsets.numel() - 1
    if cand_start.numel() != B:
        raise ValueError("cand_start must have B entries")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev)
    ws_bytes = rr_attn_workspace_bytes(B, T, H, d)
    ws = _workspace(ws_bytes, workspace, dev)
    _check("rr_attn_fwd", _lib.rr_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(offsets), _ptr(cand_start), _ptr(valid),
        int(bool(attend_padded_history)), B, T, H, d, dt, float(scale or 0.0), _ptr(ws),
        ws.numel(), _stream(stream, dev)))
    return out


def rr_attn_fwd_rope(q, k, v, offsets, cand_start, theta_base=None, scale=None, out=None, workspace=None,
                     stream=None) -> torch.Tensor:
    """Full-sequence attention with the queries rotated inside the kernel: q unrotated, k
    already rotated (rr_rope_qk with q=None); bf16, no padding mask."""
    dev = q.device
    _need(q, "q")
    dt = _rr_dtype(q)
    for name, t in (("k", k), ("v", v)):
        _need(t, name, q.dtype, dev)
        if t.shape != q.shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != q shape {tuple(q.shape)}")
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d]")
    _need(offsets, "offsets", torch.int32, dev)
    _need(cand_start, "cand_start", torch.int32, dev)
    T, H, d = q.shape
    B = offsets.numel() - 1
    if cand_start.numel() != B:
        raise ValueError("cand_start must have B entries")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev)
    ws = _workspace(rr_attn_workspace_bytes(B, T, H, d), workspace, dev)
    _check("rr_attn_fwd_rope", _lib.rr_attn_fwd_rope(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(offsets), _ptr(cand_start), B, T, H, d, dt,
        float(scale or 0.0), float(theta_base or 0.0), _ptr(ws), ws.numel(), _stream(stream, dev)))
    return out


def rr_cand_only_attn_fwd_rope(q_cand, k_hist, v_hist, k_cand, v_cand, hist_offsets, cand_offsets,
                               theta_base=None, scale=None, out=None, workspace=None, stream=None) -> torch.Tensor:
    """Candidate-only attention with the candidates' queries rotated inside the kernel (at
    their user's history length); k_hist and k_cand already rotated."""
    dev = q_cand.device
    _need(q_cand, "q_cand")
    dt = _rr_dtype(q_cand)
    Tc, H, d = q_cand.shape
    for name, t in (("k_cand", k_cand), ("v_cand", v_cand)):
        _need(t, name, q_cand.dtype, dev)
        if t.shape != q_cand.shape:
            raise ValueError(f"{name} must match q_cand")
    for name, t in (("k_hist", k_hist), ("v_hist", v_hist)):
        _need(t, name, q_cand.dtype, dev)
        if t.dim() != 3 or tuple(t.shape[1:]) != (H, d):
            raise ValueError(f"{name} must be [Th, H, d]")
    if k_hist.shape != v_hist.shape:
        raise ValueError("k_hist and v_hist must have the same shape")
    _need(hist_offsets, "hist_offsets", torch.int32, dev)
    _need(cand_offsets, "cand_offsets", torch.int32, dev)
    B = cand_offsets.numel() - 1
    if hist_offsets.numel() != B + 1:
        raise ValueError("hist_offsets and cand_offsets must both have B+1 entries")
    Th = k_hist.shape[0]
    if out is None:
        out = torch.empty_like(q_cand)
    _need(out, "out", q_cand.dtype, dev)
    ws = _workspace(rr_cand_only_workspace_bytes(B, Th, Tc, H, d), workspace, dev)
    _check("rr_cand_only_attn_fwd_rope", _lib.rr_cand_only_attn_fwd_rope(
        _ptr(q_cand), _ptr(k_hist), _ptr(v_hist), _ptr(k_cand), _ptr(v_cand), _ptr(out), _ptr(hist_offsets),
        _ptr(cand_offsets), B, Th, Tc, H, d, dt, float(scale or 0.0), float(theta_base or 0.0), _ptr(ws),
        ws.numel(), _stream(stream, dev)))
    return out


def rr_attn_fwd_noalloc(q, k, v, offsets, cand_start, out, valid=None, attend_padded_history=False, scale=None,
                        stream=None) -> torch.Tensor:
    """rr_attn_fwd with no workspace: the library keeps the plan in a static device array
    (rr_attn_fwd_noalloc_max_bytes() bytes per GPU) and allocates nothing; ``out`` is the
    caller's output tensor [T, H, d] of q's dtype.  Calls that overlap on one GPU race."""
    dev = q.device
    _need(q, "q")
    dt = _rr_dtype(q)
    for name, t in (("k", k), ("v", v), ("out", out)):
        _need(t, name, q.dtype, dev)
        if t.shape != q.shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != q shape {tuple(q.shape)}")
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d]")
    _need(offsets, "offsets", torch.int32, dev)
    _need(cand_start, "cand_start", torch.int32, dev)
    if valid is not None:
        _need(valid, "valid", torch.uint8, dev)
    T, H, d = q.shape
    B = offsets.numel() - 1
    if cand_start.numel() != B:
        raise ValueError("cand_start must have B entries")
    _check("rr_attn_fwd_noalloc", _lib.rr_attn_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(offsets), _ptr(cand_start), _ptr(valid),
        int(bool(attend_padded_history)), B, T, H, d, dt, float(scale or 0.0), _stream(stream, dev)))
    return out


def rr_attn_fwd_noalloc_max_bytes() -> int:
    return int(_lib.rr_attn_fwd_noalloc_max_bytes())


def rr_cand_only_attn_fwd(q_cand, k_hist, v_hist, k_cand, v_cand, hist_offsets, cand_offsets,
                          scale=None, out=None, workspace=None, stream=None) -> torch.Tensor:
    """Candidate-only layer attention.  Candidate tensors [Tc, H, d], history K/V [Th, H, d]."""
    dev = q_cand.device
    _need(q_cand, "q_cand")
    dt = _rr_dtype(q_cand)
    if q_cand.dim() != 3:
        raise ValueError("q_cand must be [Tc, H, d]")
    Tc, H, d = q_cand.shape
    for name, t in (("k_cand", k_cand), ("v_cand", v_cand)):
        _need(t, name, q_cand.dtype, dev)
        if t.shape != q_cand.shape:
            raise ValueError(f"{name} shape mismatch")
    for name, t in (("k_hist", k_hist), ("v_hist", v_hist)):
        _need(t, name, q_cand.dtype, dev)
        if t.dim() != 3 or t.shape[1:] != q_cand.shape[1:]:
            raise ValueError(f"{name} must be [Th, H, d]")
    if k_hist.shape != v_hist.shape:
        raise ValueError("k_hist and v_hist differ in shape")
    Th = k_hist.shape[0]
    _need(hist_offsets, "hist_offsets", torch.int32, dev)
    _need(cand_offsets, "cand_offsets", torch.int32, dev)
    B = cand_offsets.numel() - 1
    if hist_offsets.numel() != B + 1:
        raise ValueError("hist_offsets and cand_offsets must both have B+1 entries")
    if out is None:
        out = torch.empty_like(q_cand)
    _need(out, "out", q_cand.dtype, dev)
    ws_bytes = rr_cand_only_workspace_bytes(B, Th, Tc, H, d)
    ws = _workspace(ws_bytes, workspace, dev)
    _check("rr_cand_only_attn_fwd", _lib.rr_cand_only_attn_fwd(
        _ptr(q_cand), _ptr(k_hist), _ptr(v_hist), _ptr(k_cand), _ptr(v_cand), _ptr(out),
        _ptr(hist_offsets), _ptr(cand_offsets), B, Th, Tc, H, d, dt, float(scale or 0.0),
        _ptr(ws), ws.numel(), _stream(stream, dev)))
    return out


def rr_attn_plan(offsets, cand_start, T: int, H: int, d: int, dtype, valid=None,
                 attend_padded_history=False, workspace=None, stream=None,
                 backward=False) -> torch.Tensor:
    """Plan a full-sequence call (lengths only); returns the workspace holding the plan.
    ``backward`` sizes a new workspace for rr_attn_bwd_run as well."""
    dev = offsets.device
    _need(offsets, "offsets", torch.int32)
    _need(cand_start, "cand_start", torch.int32, dev)
    if valid is not None:
        _need(valid, "valid", torch.uint8, dev)
    B = offsets.numel() - 1
    dt = _rr_dtype(torch.empty(0, dtype=dtype))
    need = rr_attn_bwd_workspace_bytes(B, T, H, d) if backward else rr_attn_workspace_bytes(B, T, H, d)
    ws = _workspace(need, workspace, dev)
    _check("rr_attn_plan", _lib.rr_attn_plan(_ptr(offsets), _ptr(cand_start), _ptr(valid),
                                             int(bool(attend_padded_history)), B, T, H, d, dt,
                                             _ptr(ws), ws.numel(), _stream(stream, dev)))
    return ws


def rr_attn_run(q, k, v, B: int, workspace, scale=None, out=None, stream=None) -> torch.Tensor:
    """Attention with the plan in ``workspace`` (same sizes as the plan)."""
    dev = q.device
    _need(q, "q")
    dt = _rr_dtype(q)
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    T, H, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev)
    _check("rr_attn_run", _lib.rr_attn_run(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, T, H, d, dt,
                                           float(scale or 0.0), _ptr(workspace), workspace.numel(),
                                           _stream(stream, dev)))
    return out


def rr_attn_run_lse(q, k, v, B: int, workspace, scale=None, out=None, lse=None, stream=None):
    """rr_attn_run that also returns each row's log-sum-exp: (out, lse float32 [T, H])."""
    dev = q.device
    _need(q, "q")
    dt = _rr_dtype(q)
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    T, H, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(out, "out", q.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    _check("rr_attn_run_lse", _lib.rr_attn_run_lse(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, T, H, d, dt, float(scale or 0.0),
        _ptr(workspace), workspace.numel(), _stream(stream, dev)))
    return out, lse


def rr_attn_bwd_workspace_bytes(B: int, T: int, H: int, d: int) -> int:
    return int(_lib.rr_attn_bwd_workspace_bytes(B, T, H, d))


def _bwd_tensors(q, k, v, o, dout, lse, dq, dk, dv):
    dev = q.device
    _need(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d]")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, name, q.dtype, dev)
        if t.shape != q.shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != q shape {tuple(q.shape)}")
    _need(lse, "lse", torch.float32, dev)
    if tuple(lse.shape) != tuple(q.shape[:2]):
        raise ValueError("lse must be [T, H]")
    outs = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        t = torch.empty_like(q) if t is None else t
        _need(t, name, q.dtype, dev)
        outs.append(t)
    return outs


def rr_attn_bwd_run(q, k, v, o, dout, lse, B: int, workspace, scale=None, dq=None, dk=None, dv=None,
                    stream=None):
    """Gradients (dq, dk, dv) with the plan in ``workspace``: one from rr_attn_plan in a
    workspace of rr_attn_bwd_workspace_bytes (``rr_attn_plan(..., backward=True)``)."""
    dq, dk, dv = _bwd_tensors(q, k, v, o, dout, lse, dq, dk, dv)
    _need(workspace, "workspace", torch.uint8, q.device)
    T, H, d = q.shape
    _check("rr_attn_bwd_run", _lib.rr_attn_bwd_run(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, T, H, d,
        _rr_dtype(q), float(scale or 0.0), _ptr(workspace), workspace.numel(), _stream(stream, q.device)))
    return dq, dk, dv


def rr_attn_bwd(q, k, v, o, dout, lse, offsets, cand_start, valid=None, attend_padded_history=False,
                scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Plan and backward in one call: (dq, dk, dv), each [T, H, d] like q."""
    dq, dk, dv = _bwd_tensors(q, k, v, o, dout, lse, dq, dk, dv)
    dev = q.device
    _need(offsets, "offsets", torch.int32, dev)
    _need(cand_start, "cand_start", torch.int32, dev)
    if valid is not None:
        _need(valid, "valid", torch.uint8, dev)
    T, H, d = q.shape
    B = offsets.numel() - 1
    if cand_start.numel() != B:
        raise ValueError("cand_start must have B entries")
    ws = _workspace(rr_attn_bwd_workspace_bytes(B, T, H, d), workspace, dev)
    _check("rr_attn_bwd", _lib.rr_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(offsets), _ptr(cand_start), _ptr(valid), int(bool(attend_padded_history)), B, T, H, d,
        _rr_dtype(q), float(scale or 0.0), _ptr(ws), ws.numel(), _stream(stream, dev)))
    return dq, dk, dv


def rr_cand_only_plan(hist_offsets, cand_offsets, Th: int, Tc: int, H: int, d: int, dtype,
                      workspace=None, stream=None) -> torch.Tensor:
    dev = cand_offsets.device
    _need(hist_offsets, "hist_offsets", torch.int32, dev)
    _need(cand_offsets, "cand_offsets", torch.int32, dev)
    B = cand_offsets.numel() - 1
    dt = _rr_dtype(torch.empty(0, dtype=dtype))
    ws = _workspace(rr_cand_only_workspace_bytes(B, Th, Tc, H, d), workspace, dev)
    _check("rr_cand_only_plan", _lib.rr_cand_only_plan(_ptr(hist_offsets), _ptr(cand_offsets), B, Th,
                                                       Tc, H, d, dt, _ptr(ws), ws.numel(),
                                                       _stream(stream, dev)))
    return ws


def rr_cand_only_run(q_cand, k_hist, v_hist, k_cand, v_cand, B: int, workspace, scale=None, out=None,
                     stream=None) -> torch.Tensor:
    dev = q_cand.device
    _need(q_cand, "q_cand")
    dt = _rr_dtype(q_cand)
    for name, t in (("k_hist", k_hist), ("v_hist", v_hist), ("k_cand", k_cand), ("v_cand", v_cand)):
        _need(t, name, q_cand.dtype, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    Tc, H, d = q_cand.shape
    Th = k_hist.shape[0]
    if out is None:
        out = torch.empty_like(q_cand)
    _need(out, "out", q_cand.dtype, dev)
    _check("rr_cand_only_run", _lib.rr_cand_only_run(
        _ptr(q_cand), _ptr(k_hist), _ptr(v_hist), _ptr(k_cand), _ptr(v_cand), _ptr(out), B, Th, Tc, H,
        d, dt, float(scale or 0.0), _ptr(workspace), workspace.numel(), _stream(stream, dev)))
    return out


def rr_validate_jagged(offsets, cand_start, T: int, stream=None) -> int:
    """Debug: data-contract bit flags (0 = fine).  Synchronises the stream to read them."""
    dev = offsets.device
    _need(offsets, "offsets", torch.int32)
    if cand_start is not None:
        _need(cand_start, "cand_start", torch.int32, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    s = _stream(stream, dev)
    _check("rr_validate_jagged", _lib.rr_validate_jagged(_ptr(offsets), _ptr(cand_start),
                                                         offsets.numel() - 1, T, _ptr(err), s))
    return int(err.item())


def rr_rope_positions(offsets, cand_start, T: int, pos_base=None, out=None, stream=None) -> torch.Tensor:
    """Right-anchored position of every row (int32 [T])."""
    dev = offsets.device
    _need(offsets, "offsets", torch.int32)
    _need(cand_start, "cand_start", torch.int32, dev)
    if pos_base is not None:
        _need(pos_base, "pos_base", torch.int32, dev)
    B = offsets.numel() - 1
    if out is None:
        out = torch.empty(T, dtype=torch.int32, device=dev)
    _need(out, "out", torch.int32, dev)
    _check("rr_rope_positions", _lib.rr_rope_positions(_ptr(offsets), _ptr(cand_start), _ptr(pos_base),
                                                       B, T, _ptr(out), _stream(stream, dev)))
    return out


def rr_rope_qk(q, k, offsets, cand_start, pos_base=None, theta_base=None, q_out=None, k_out=None,
               in_place=False, stream=None):
    """Rotary encoding of q and k ([T, H, d], either may be None) at right-anchored positions.

    Returns (q_out, k_out); with ``in_place`` the inputs are overwritten and returned."""
    x = q if q is not None else k
    if x is None:
        return None, None
    dev = x.device
    _need(x, "q" if q is not None else "k")
    dt = _rr_dtype(x)
    if x.dim() != 3:
        raise ValueError("q and k must be [T, H, d]")
    T, H, d = x.shape
    _need(offsets, "offsets", torch.int32, dev)
    _need(cand_start, "cand_start", torch.int32, dev)
    if pos_base is not None:
        _need(pos_base, "pos_base", torch.int32, dev)
    outs = []
    for name, t, o in (("q", q, q_out), ("k", k, k_out)):
        if t is None:
            outs.append(None)
            continue
        _need(t, name, x.dtype, dev)
        if t.shape != x.shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(x.shape)}")
        if o is None:
            o = t if in_place else torch.empty_like(t)
        _need(o, f"{name}_out", x.dtype, dev)
        if o.shape != x.shape:
            raise ValueError(f"{name}_out shape {tuple(o.shape)} != {tuple(x.shape)}")
        outs.append(o)
    B = offsets.numel() - 1
    _check("rr_rope_qk", _lib.rr_rope_qk(_ptr(q), _ptr(k), _ptr(outs[0]), _ptr(outs[1]), _ptr(offsets),
                                         _ptr(cand_start), _ptr(pos_base), B, T, H, d, dt,
                                         float(theta_base or 0.0), _stream(stream, dev)))
    return outs[0], outs[1]


class RRLayer(ctypes.Structure):
    """rr_layer: device pointers of one layer's norm gain, W_qkv and W_o."""
    _fields_ = [("norm_gain", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p)]


def rr_rms_norm(x, gain, eps=None, out=None, stream=None) -> torch.Tensor:
    """bf16 rows x / sqrt(mean(x^2) + eps) * gain; x float32 [M, D]."""
    _need(x, "x", torch.float32)
    _need(gain, "gain", torch.float32, x.device)
    M, D = x.shape
    if out is None:
        out = torch.empty((M, D), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, x.device)
    _check("rr_rms_norm", _lib.rr_rms_norm(_ptr(x), _ptr(gain), _ptr(out), M, D, float(eps or 0.0),
                                           _stream(stream, x.device)))
    return out


def rr_linear(a, w, out=None, residual=None, stream=None) -> torch.Tensor:
    """a W^T for a bf16 [M, K] and W bf16 [N, K]: into a new or given bf16 ``out``, or added
    to a float32 ``residual`` [M, N] (returned)."""
    _need(a, "a", torch.bfloat16)
    _need(w, "w", torch.bfloat16, a.device)
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N, K]")
    if residual is not None:
        _need(residual, "residual", torch.float32, a.device)
    elif out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if out is not None:
        _need(out, "out", torch.bfloat16, a.device)
    _check("rr_linear", _lib.rr_linear(_ptr(a), _ptr(w), _ptr(out), _ptr(residual), M, N, K,
                                       _stream(stream, a.device)))
    return residual if residual is not None else out


def _layer_array(layers, D, dev):
    arr = (RRLayer * len(layers))()
    for i, (gain, w_qkv, w_o) in enumerate(layers):
        _need(gain, "norm_gain", torch.float32, dev)
        _need(w_qkv, "w_qkv", torch.bfloat16, dev)
        _need(w_o, "w_o", torch.bfloat16, dev)
        if gain.numel() != D or tuple(w_qkv.shape) != (3 * D, D) or tuple(w_o.shape) != (D, D):
            raise ValueError(f"layer {i}: expected gain [D], w_qkv [3D, D], w_o [D, D] with D = {D}")
        arr[i] = RRLayer(gain.data_ptr(), w_qkv.data_ptr(), w_o.data_ptr())
    return arr


def rr_ranker_fwd(x, layers, n_cand_only, offsets, cand_start, Tc: int, H: int, d: int, theta_base=None,
                  keep_cache=True, x_cand_out=None, x_hist_out=None, kv_cache=None, workspace=None,
                  stream=None, user_tokens=None, Tp: int = 0):
    """The layer stack over x float32 [T, H*d] (updated in place by the full layers).
    ``layers``: list of (norm_gain float32 [D], w_qkv bf16 [3D, D], w_o bf16 [D, D]).
    ``user_tokens`` (int32 [B] on the device, Tp = their sum): the user tokens keep being
    updated in the candidate-only layers.
    Returns (x_cand [Tc, D], x_hist [T-Tc, D], kv_cache bf16 [L, 2, T-Tc, H, d] or None)."""
    dev = x.device
    _need(x, "x", torch.float32)
    T, D = x.shape
    if D != H * d:
        raise ValueError("x must be [T, H*d]")
    _need(offsets, "offsets", torch.int32, dev)
    _need(cand_start, "cand_start", torch.int32, dev)
    B = offsets.numel() - 1
    arr = _layer_array(layers, D, dev)
    Th = T - Tc
    if x_cand_out is None:
        x_cand_out = torch.empty((Tc, D), dtype=torch.float32, device=dev)
    if x_hist_out is None:
        x_hist_out = torch.empty((Th, D), dtype=torch.float32, device=dev)
    if kv_cache is None and keep_cache:
        kv_cache = torch.empty((len(layers), 2, Th, H, d), dtype=torch.bfloat16, device=dev)
    for name, t in (("x_cand_out", x_cand_out), ("x_hist_out", x_hist_out)):
        _need(t, name, torch.float32, dev)
    if kv_cache is not None:
        _need(kv_cache, "kv_cache", torch.bfloat16, dev)
        if kv_cache.numel() != len(layers) * 2 * Th * D:
            raise ValueError("kv_cache must be [n_layers, 2, T - Tc, H, d]")
    if user_tokens is not None:
        _need(user_tokens, "user_tokens", torch.int32, dev)
        if user_tokens.numel() != B:
            raise ValueError("user_tokens must have B entries")
    else:
        Tp = 0
    ws = _workspace(int(_lib.rr_ranker_workspace_bytes(B, T, Tc, Tp, H, d)), workspace, dev)
    _check("rr_ranker_fwd", _lib.rr_ranker_fwd(
        _ptr(x), ctypes.cast(arr, ctypes.c_void_p), len(layers), int(n_cand_only), _ptr(offsets),
        _ptr(cand_start), _ptr(user_tokens), B, T, Tc, int(Tp), H, d, float(theta_base or 0.0),
        _ptr(x_cand_out), _ptr(x_hist_out), _ptr(kv_cache), _ptr(ws), ws.numel(), _stream(stream, dev)))
    return x_cand_out, x_hist_out, kv_cache


def rr_ranker_cached_fwd(x_cand, layers, kv_cache, hist_offsets, cand_offsets, H: int, d: int,
                         theta_base=None, workspace=None, stream=None) -> torch.Tensor:
    """A later request: candidates float32 [Tc, H*d] through every layer as a candidate-only
    layer over ``kv_cache`` (from rr_ranker_fwd); updated in place and returned."""
    dev = x_cand.device
    _need(x_cand, "x_cand", torch.float32)
    Tc, D = x_cand.shape
    _need(kv_cache, "kv_cache", torch.bfloat16, dev)
    _need(hist_offsets, "hist_offsets", torch.int32, dev)
    _need(cand_offsets, "cand_offsets", torch.int32, dev)
    B = cand_offsets.numel() - 1
    Th = kv_cache.shape[2]
    if kv_cache.shape[0] != len(layers) or kv_cache.numel() != len(layers) * 2 * Th * D:
        raise ValueError("kv_cache must be [n_layers, 2, Th, H, d]")
    arr = _layer_array(layers, D, dev)
    ws = _workspace(int(_lib.rr_ranker_cached_workspace_bytes(B, Th, Tc, H, d)), workspace, dev)
    _check("rr_ranker_cached_fwd", _lib.rr_ranker_cached_fwd(
        _ptr(x_cand), ctypes.cast(arr, ctypes.c_void_p), len(layers), _ptr(kv_cache), _ptr(hist_offsets),
        _ptr(cand_offsets), B, Th, Tc, H, d, float(theta_base or 0.0), _ptr(ws), ws.numel(),
        _stream(stream, dev)))
    return x_cand


def rr_ranker_workspace_bytes(B: int, T: int, Tc: int, H: int, d: int, Tp: int = 0) -> int:
    return int(_lib.rr_ranker_workspace_bytes(B, T, Tc, Tp, H, d))


def rr_user_token_attn(q, k, v, key_offsets, query_offsets, scale=None, out=None, workspace=None,
                       stream=None) -> torch.Tensor:
    """Every query row of user b reads exactly user b's key rows (no self-term).
    q [Tq, H, d]; k, v [Tk, H, d]; key_offsets, query_offsets int32 [B+1]."""
    dev = q.device
    _need(q, "q")
    dt = _rr_dtype(q)
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    _need(key_offsets, "key_offsets", torch.int32, dev)
    _need(query_offsets, "query_offsets", torch.int32, dev)
    Tq, H, d = q.shape
    Tk = k.shape[0]
    B = query_offsets.numel() - 1
    if out is None:
        out = torch.empty_like(q)
    ws = _workspace(int(_lib.rr_user_token_attn_workspace_bytes(B, Tk, Tq, H, d)), workspace, dev)
    _check("rr_user_token_attn_plan", _lib.rr_user_token_attn_plan(
        _ptr(key_offsets), _ptr(query_offsets), B, Tk, Tq, H, d, dt, _ptr(ws), ws.numel(), _stream(stream, dev)))
    _check("rr_user_token_attn_run", _lib.rr_user_token_attn_run(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Tk, Tq, H, d, dt, float(scale or 0.0), _ptr(ws), ws.numel(),
        _stream(stream, dev)))
    return out


def rr_ranker_cached_workspace_bytes(B: int, Th: int, Tc: int, H: int, d: int) -> int:
    return int(_lib.rr_ranker_cached_workspace_bytes(B, Th, Tc, H, d))


def rr_forward_fingerprint() -> str:
    """Digest of the forward attention kernels' machine code in the loaded library."""
    return _lib.rr_forward_fingerprint().decode()


def rr_cand_only_bwd_workspace_bytes(B: int, Th: int, Tc: int, H: int, d: int) -> int:
    return int(_lib.rr_cand_only_bwd_workspace_bytes(B, Th, Tc, H, d))


def rr_cand_only_train_plan(hist_offsets, cand_offsets, Th: int, Tc: int, H: int, d: int, dtype, stream=None):
    """rr_cand_only_plan into a workspace sized for the backward as well."""
    dev = cand_offsets.device
    B = cand_offsets.numel() - 1
    ws = _workspace(rr_cand_only_bwd_workspace_bytes(B, Th, Tc, H, d), None, dev)
    return rr_cand_only_plan(hist_offsets, cand_offsets, Th, Tc, H, d, dtype, workspace=ws, stream=stream)


def rr_cand_only_run_lse(q_cand, k_hist, v_hist, k_cand, v_cand, B: int, workspace, scale=None, out=None,
                         lse=None, stream=None):
    """rr_cand_only_run that also returns each candidate row's log-sum-exp: (out, lse [Tc, H])."""
    dev = q_cand.device
    _need(q_cand, "q_cand")
    dt = _rr_dtype(q_cand)
    Tc, H, d = q_cand.shape
    Th = k_hist.shape[0]
    for name, t in (("k_hist", k_hist), ("v_hist", v_hist), ("k_cand", k_cand), ("v_cand", v_cand)):
        _need(t, name, q_cand.dtype, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    if out is None:
        out = torch.empty_like(q_cand)
    if lse is None:
        lse = torch.empty((Tc, H), dtype=torch.float32, device=dev)
    _need(out, "out", q_cand.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    _check("rr_cand_only_run_lse", _lib.rr_cand_only_run_lse(
        _ptr(q_cand), _ptr(k_hist), _ptr(v_hist), _ptr(k_cand), _ptr(v_cand), _ptr(out), _ptr(lse), B, Th, Tc, H,
        d, dt, float(scale or 0.0), _ptr(workspace), workspace.numel(), _stream(stream, dev)))
    return out, lse


def rr_cand_only_bwd_run(q_cand, k_hist, v_hist, k_cand, v_cand, o_cand, dout, lse, hist_offsets, cand_offsets,
                         workspace, scale=None, stream=None):
    """Gradients of a candidate-only layer: (dq_cand, dk_hist, dv_hist, dk_cand, dv_cand)."""
    dev = q_cand.device
    _need(q_cand, "q_cand")
    dt = _rr_dtype(q_cand)
    Tc, H, d = q_cand.shape
    Th = k_hist.shape[0]
    for name, t in (("k_cand", k_cand), ("v_cand", v_cand), ("o_cand", o_cand), ("dout", dout)):
        _need(t, name, q_cand.dtype, dev)
        if t.shape != q_cand.shape:
            raise ValueError(f"{name} must be [Tc, H, d]")
    for name, t in (("k_hist", k_hist), ("v_hist", v_hist)):
        _need(t, name, q_cand.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    _need(hist_offsets, "hist_offsets", torch.int32, dev)
    _need(cand_offsets, "cand_offsets", torch.int32, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    B = cand_offsets.numel() - 1
    grads = [torch.empty_like(q_cand), torch.empty_like(k_hist), torch.empty_like(v_hist), torch.empty_like(k_cand),
             torch.empty_like(v_cand)]
    _check("rr_cand_only_bwd_run", _lib.rr_cand_only_bwd_run(
        _ptr(q_cand), _ptr(k_hist), _ptr(v_hist), _ptr(k_cand), _ptr(v_cand), _ptr(o_cand), _ptr(dout), _ptr(lse),
        *[_ptr(g) for g in grads], _ptr(hist_offsets), _ptr(cand_offsets), B, Th, Tc, H, d, dt,
        float(scale or 0.0), _ptr(workspace), workspace.numel(), _stream(stream, dev)))
    return tuple(grads)
