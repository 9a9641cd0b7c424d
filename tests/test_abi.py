"""The C ABI on the host (CPU only): the library loads, exports every declared symbol,
and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rr.h")


def _lib():
    from jagged_candidate_isolated_amd import rr
    return rr, rr._lib


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("rr_segment_ids", "rr_bounds", "rr_attn_fwd", "rr_cand_only_attn_fwd"):
        assert n in names


def test_library_exports_every_declared_symbol():
    _, lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    rr, lib = _lib()
    assert lib.rr_abi_version() == 1
    for st in (rr.RR_OK, rr.RR_EINVAL, rr.RR_EDTYPE, rr.RR_EUNSUPPORTED, rr.RR_EWORKSPACE, rr.RR_EHIP):
        assert lib.rr_status_string(st)
    assert lib.rr_status_string(-99) == b"unknown status"


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case below returns before any launch


def _attn(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, offsets=FAKE, cand_start=FAKE, valid=None, flag=0,
             B=2, T=10, H=2, d=64, dtype=1, scale=0.0, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.rr_attn_fwd(a["q"], a["k"], a["v"], a["o"], a["offsets"], a["cand_start"], a["valid"],
                           a["flag"], a["B"], a["T"], a["H"], a["d"], a["dtype"], a["scale"], a["ws"],
                           a["ws_bytes"], a["stream"])


def test_attn_argument_errors():
    rr, lib = _lib()
    assert _attn(lib, B=-1) == rr.RR_EINVAL
    assert _attn(lib, T=-5) == rr.RR_EINVAL
    assert _attn(lib, dtype=7) == rr.RR_EDTYPE
    for d in (0, 8, 48, 96, 256):
        assert _attn(lib, d=d) == rr.RR_EUNSUPPORTED, d
    assert _attn(lib, H=2000) == rr.RR_EUNSUPPORTED
    assert _attn(lib, q=None) == rr.RR_EINVAL
    assert _attn(lib, offsets=None) == rr.RR_EINVAL
    assert _attn(lib, cand_start=None) == rr.RR_EINVAL
    assert _attn(lib, ws=None) == rr.RR_EWORKSPACE
    need = lib.rr_attn_workspace_bytes(2, 10, 2, 64)
    assert need > 0
    assert _attn(lib, ws_bytes=need - 1) == rr.RR_EWORKSPACE
    # empty calls are valid no-ops, even with NULL tensors
    assert _attn(lib, B=0, q=None, k=None, v=None, o=None, ws=None) == rr.RR_OK
    assert _attn(lib, T=0, q=None, ws=None) == rr.RR_OK


def test_query_tile_index_limit():
    """A work item packs its query tile above 10 head bits of an int32, so the library
    refuses 2^21 or more 64-row query tiles (checked on the host; nothing is launched)."""
    rr, lib = _lib()
    last_ok = (1 << 27) - 64          # 2^21 - 1 tiles of 64 rows
    first_bad = last_ok + 1
    assert _attn(lib, B=1, T=first_bad, H=1) == rr.RR_EUNSUPPORTED
    assert _attn(lib, B=1, T=(1 << 31) - 1, H=1) == rr.RR_EUNSUPPORTED
    assert lib.rr_attn_workspace_bytes(1, first_bad, 1, 64) == 0
    assert lib.rr_attn_workspace_bytes(1, last_ok, 1, 64) > 0
    assert lib.rr_cand_only_workspace_bytes(1, 10, first_bad, 1, 128) == 0
    assert lib.rr_cand_only_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 10, first_bad, 1, 128, 1,
                                     0.0, FAKE, 1 << 40, None) == rr.RR_EUNSUPPORTED
    # the key-major plan of the candidate-only backward tiles the frozen rows the same way
    assert lib.rr_cand_only_bwd_workspace_bytes(1, first_bad, 10, 1, 128) == 0


def test_cand_only_argument_errors():
    rr, lib = _lib()
    f = lib.rr_cand_only_attn_fwd

    def call(**kw):
        a = dict(qc=FAKE, kh=FAKE, vh=FAKE, kc=FAKE, vc=FAKE, oc=FAKE, ho=FAKE, co=FAKE, B=2, Th=10,
                 Tc=6, H=2, d=128, dtype=1, scale=0.0, ws=FAKE, ws_bytes=1 << 30, stream=None)
        a.update(kw)
        return f(a["qc"], a["kh"], a["vh"], a["kc"], a["vc"], a["oc"], a["ho"], a["co"], a["B"],
                 a["Th"], a["Tc"], a["H"], a["d"], a["dtype"], a["scale"], a["ws"], a["ws_bytes"],
                 a["stream"])
    assert call(Th=-1) == rr.RR_EINVAL
    assert call(dtype=5) == rr.RR_EDTYPE
    assert call(d=80) == rr.RR_EUNSUPPORTED
    assert call(kh=None) == rr.RR_EINVAL
    assert call(kh=None, vh=None, Th=0, ws=None) == rr.RR_EWORKSPACE
    assert call(ws=None) == rr.RR_EWORKSPACE
    assert call(co=None) == rr.RR_EINVAL
    assert call(Tc=0, qc=None, ws=None) == rr.RR_OK
    assert lib.rr_cand_only_workspace_bytes(2, 10, 6, 2, 128) > 0
    assert lib.rr_cand_only_workspace_bytes(2, 10, 6, 2, 100) == 0


def test_segment_and_bounds_argument_errors():
    rr, lib = _lib()
    assert lib.rr_segment_ids(FAKE, FAKE, None, 0, -1, 5, FAKE, None) == rr.RR_EINVAL
    assert lib.rr_segment_ids(None, FAKE, None, 0, 2, 5, FAKE, None) == rr.RR_EINVAL
    assert lib.rr_segment_ids(FAKE, FAKE, None, 0, 2, 5, None, None) == rr.RR_EINVAL
    assert lib.rr_segment_ids(None, None, None, 0, 0, 0, None, None) == rr.RR_OK
    assert lib.rr_bounds(FAKE, None, 2, 5, FAKE, None) == rr.RR_EINVAL
    assert lib.rr_bounds(FAKE, FAKE, 2, 5, None, None) == rr.RR_EINVAL
    assert lib.rr_bounds(None, None, 0, 0, None, None) == rr.RR_OK
    assert lib.rr_validate_jagged(None, None, 1, 1, FAKE, None) == rr.RR_EINVAL


def test_rope_argument_errors():
    rr, lib = _lib()
    # (q, k, q_out, k_out, offsets, cand_start, pos_base, B, T, H, d, dtype, base, stream)
    ok = dict(q=FAKE, k=FAKE, qo=FAKE, ko=FAKE, off=FAKE, cs=FAKE, B=2, T=8, H=2, d=64, dt=rr.RR_BF16)

    def call(**kw):
        a = {**ok, **kw}
        return lib.rr_rope_qk(a["q"], a["k"], a["qo"], a["ko"], a["off"], a["cs"], None, a["B"], a["T"],
                              a["H"], a["d"], a["dt"], 0.0, None)
    assert call(d=63) == rr.RR_EUNSUPPORTED
    assert call(d=0) == rr.RR_EUNSUPPORTED
    assert call(d=258) == rr.RR_EUNSUPPORTED
    assert call(dt=7) == rr.RR_EDTYPE
    assert call(B=-1) == rr.RR_EINVAL
    assert call(qo=None) == rr.RR_EINVAL
    assert call(ko=None) == rr.RR_EINVAL
    assert call(off=None) == rr.RR_EINVAL
    assert call(q=None, k=None) == rr.RR_OK          # nothing to rotate: no launch
    assert call(B=0) == rr.RR_OK and call(T=0) == rr.RR_OK
    assert lib.rr_rope_positions(None, FAKE, None, 2, 8, FAKE, None) == rr.RR_EINVAL
    assert lib.rr_rope_positions(FAKE, FAKE, None, 2, 8, None, None) == rr.RR_EINVAL
    assert lib.rr_rope_positions(FAKE, FAKE, None, -1, 8, FAKE, None) == rr.RR_EINVAL
    assert lib.rr_rope_positions(None, None, None, 0, 0, None, None) == rr.RR_OK


def test_backward_argument_errors():
    rr, lib = _lib()

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, off=FAKE,
                 cs=FAKE, B=2, T=10, H=2, d=64, dt=rr.RR_BF16, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return lib.rr_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                               a["off"], a["cs"], None, 0, a["B"], a["T"], a["H"], a["d"], a["dt"], 0.0,
                               a["ws"], a["ws_bytes"], None)
    assert call(B=-1) == rr.RR_EINVAL
    assert call(dt=9) == rr.RR_EDTYPE
    assert call(dt=rr.RR_F32) == rr.RR_EUNSUPPORTED       # the backward is bf16 only
    for d in (16, 32, 48):
        assert call(d=d) == rr.RR_EUNSUPPORTED, d
    assert call(off=None) == rr.RR_EINVAL
    assert call(ws=None) == rr.RR_EWORKSPACE
    need = lib.rr_attn_bwd_workspace_bytes(2, 10, 2, 64)
    assert need > lib.rr_attn_workspace_bytes(2, 10, 2, 64)   # plus rowsum(dO * o) per row and head
    assert call(ws_bytes=need - 1) == rr.RR_EWORKSPACE
    assert lib.rr_attn_bwd_workspace_bytes(2, 10, 2, 32) == 0
    assert call(B=0, q=None, ws=None) == rr.RR_OK
    # the run step checks its tensors before any launch
    run = lib.rr_attn_bwd_run
    args = [FAKE] * 9 + [2, 10, 2, 64, rr.RR_BF16, 0.0, FAKE, 1 << 30, None]
    for i in range(9):
        a = list(args)
        a[i] = None
        assert run(*a) == rr.RR_EINVAL, i
    a = list(args)
    a[16] = need - 1
    assert run(*a) == rr.RR_EWORKSPACE
    # the forward with lse checks like rr_attn_run
    assert lib.rr_attn_run_lse(None, FAKE, FAKE, FAKE, FAKE, 2, 10, 2, 64, 1, 0.0, FAKE, 1 << 30,
                               None) == rr.RR_EINVAL


def test_ranker_argument_errors():
    rr, lib = _lib()
    layer = rr.RRLayer(0x1000, 0x1000, 0x1000)
    arr = (rr.RRLayer * 2)(layer, layer)
    null_layer = (rr.RRLayer * 2)(layer, rr.RRLayer(0x1000, None, 0x1000))

    def call(**kw):
        a = dict(x=FAKE, layers=arr, n=2, nco=1, off=FAKE, cs=FAKE, B=2, T=100, Tc=10, H=4, d=64, xc=FAKE,
                 ws=FAKE, ws_bytes=1 << 40)
        a.update(kw)
        return lib.rr_ranker_fwd(a["x"], ctypes.cast(a["layers"], ctypes.c_void_p) if a["layers"] else None,
                                 a["n"], a["nco"], a["off"], a["cs"], a.get("ut"), a["B"], a["T"], a["Tc"],
                                 a.get("Tp", 0), a["H"], a["d"], 0.0, a["xc"], None, None, a["ws"], a["ws_bytes"],
                                 None)
    assert call(d=16) == rr.RR_EUNSUPPORTED                 # the MFMA attention: d 32, 64, 128
    assert call(H=3) == rr.RR_EUNSUPPORTED                  # D = 192 is not a multiple of 128
    assert call(Tc=101) == rr.RR_EINVAL
    assert call(nco=3) == rr.RR_EINVAL
    assert call(layers=null_layer) == rr.RR_EINVAL
    assert call(layers=None) == rr.RR_EINVAL
    assert call(x=None) == rr.RR_EINVAL
    assert call(xc=None) == rr.RR_EINVAL
    assert call(ws=None) == rr.RR_EWORKSPACE
    assert call(ut=FAKE, Tp=91) == rr.RR_EINVAL             # more user tokens than rows before candidates
    assert call(ut=FAKE, Tp=-1) == rr.RR_EINVAL
    assert call(ut=None, Tp=-1, ws=None) == rr.RR_EWORKSPACE   # Tp is ignored without user tokens
    assert lib.rr_ranker_workspace_bytes(2, 100, 10, 8, 4, 64) > lib.rr_ranker_workspace_bytes(2, 100, 10, 0, 4, 64)
    need = lib.rr_ranker_workspace_bytes(2, 100, 10, 0, 4, 64)
    assert need > lib.rr_attn_workspace_bytes(2, 100, 4, 64)
    assert call(ws_bytes=need - 1) == rr.RR_EWORKSPACE
    assert call(B=0, x=None, ws=None) == rr.RR_OK
    assert lib.rr_ranker_workspace_bytes(2, 100, 10, 0, 4, 16) == 0
    assert lib.rr_ranker_cached_workspace_bytes(2, 90, 10, 4, 64) > 0
    assert lib.rr_ranker_cached_fwd(None, ctypes.cast(arr, ctypes.c_void_p), 2, FAKE, FAKE, FAKE, 2, 90, 10, 4, 64,
                                    0.0, FAKE, 1 << 40, None) == rr.RR_EINVAL
    assert lib.rr_linear(FAKE, FAKE, FAKE, None, 10, 100, 64, None) == rr.RR_EUNSUPPORTED   # N % 128
    assert lib.rr_linear(FAKE, FAKE, FAKE, None, 10, 128, 48, None) == rr.RR_EUNSUPPORTED   # K % 64
    assert lib.rr_linear(FAKE, FAKE, FAKE, FAKE, 10, 128, 64, None) == rr.RR_EINVAL          # both outputs
    assert lib.rr_rms_norm(FAKE, FAKE, FAKE, 3, 6, 0.0, None) == rr.RR_EINVAL                # D % 4
    assert lib.rr_user_token_attn_plan(None, FAKE, 2, 10, 4, 2, 64, 1, FAKE, 1 << 30, None) == rr.RR_EINVAL
    assert lib.rr_user_token_attn_run(None, FAKE, FAKE, FAKE, 2, 10, 4, 2, 64, 1, 0.0, FAKE, 1 << 30,
                                      None) == rr.RR_EINVAL
    assert lib.rr_user_token_attn_run(FAKE, FAKE, FAKE, FAKE, 2, 10, 4, 2, 64, 1, 0.0, None, 0,
                                      None) == rr.RR_EWORKSPACE


def test_workspace_size_grows_with_work():
    _, lib = _lib()
    a = lib.rr_attn_workspace_bytes(64, 16000, 4, 64)
    b = lib.rr_attn_workspace_bytes(64, 32000, 4, 64)
    assert 0 < a < b
    assert lib.rr_attn_workspace_bytes(-1, 10, 1, 64) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    rr, _ = _lib()
    q = torch.zeros(4, 1, 16)
    off = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        rr.rr_attn_fwd(q, q, q, off, torch.tensor([2], dtype=torch.int32))
