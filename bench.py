#!/usr/bin/env python3
"""Throughput of jagged candidate-isolated attention on one MI355X; prints one JSON line.

A step is one pass of the hot path over one batch with its inputs resident in HBM:
``rr_attn_plan`` (segment IDs / bounds / length-sorted work list) then ``rr_attn_run``
(for batches of long users the key-norm pass, then the fused attention kernel) -- or, for
a small unpadded batch such as the short-history workload, ``rr_attn_fwd``, whose
attention kernel builds the work list itself (one launch); for the candidate-only
workload ``rr_cand_only_plan`` + ``rr_cand_only_run``.  The default line times the skew
workload (B=32, prefix 4, history lengths drawn from {0, 10, 100, 1000, 8192}, 2048
candidates per user, H=16, d=128, bf16, no padding) against the bf16 MFMA roofline, and
carries the short-history workload (B=64, prefix 4, history log-uniform in [10, 1000],
32 candidates per user, H=4, d=64, bf16) with its HBM roofline as a secondary object.
Steps rotate over ceil(1 GiB / footprint) copies of the inputs (one for a batch above
1 GiB), so that no step finds its data in the 256 MB Infinity Cache.

metric: effective (non-pad) attention TFLOP/s = 4 * d * H * sum_b [n_b^2 + c_b (n_b + 1)]
per step / step time; candidates/s is reported beside it.

``--ranker`` (full-sequence bf16 workloads) runs the ranker's layer stack instead: 6 full
layers, the split, 2 candidate-only layers (``rr_ranker_fwd``), with random bf16
projections of width D = H d; the line reports candidates/s of a whole request, and of
a later request for the same users that reuses the history's keys and values
(``rr_ranker_cached_fwd``).

``--backward`` (full-sequence bf16 workloads) makes a step one training pass of the
attention: plan, forward with the log-sum-exp (``rr_attn_run_lse``) and the backward
(``rr_attn_bwd_run``: dq, dk, dv).  The backward counts 2.5x the forward's effective
FLOPs (five products of the forward's size against the forward's two).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published
ROTATE_BYTES = 1 << 30
METRIC = "effective non-pad attention TFLOP/s + candidates/s, jagged candidate-isolated attn"


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="timed steps (default: about 1 s of work)")
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--config", type=int, default=None,
                   help="2 short-history, 3 lognormal, 4 candidate-only, 5 skew (the default line, which "
                        "also carries the short-history workload's roofline), 6 skew padded "
                        "(attend_padded_history=True), 7 skew padded (False)")
    p.add_argument("--rope", action="store_true",
                   help="rotate q and k at right-anchored positions (rr_rope_qk) inside every step, "
                        "before the attention")
    p.add_argument("--backward", action="store_true",
                   help="a step is plan + forward with lse + backward (full-sequence bf16, d 64 or 128)")
    p.add_argument("--ranker", action="store_true",
                   help="the layer stack (6 full + 2 candidate-only layers) end to end; candidates/s")
    p.add_argument("--update-user-token", action="store_true",
                   help="with --ranker: the prefix rows (user tokens) keep being updated in the "
                        "candidate-only layers")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="instead of the benchmark, run three plain device copies of this many MiB "
                        "from a cold 4x larger source (reference for FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def source_hash() -> str:
    """Digest of the forward attention kernels' machine code in the loaded library
    (rr_forward_fingerprint): traffic counters taken on other kernels are not reported."""
    from jagged_candidate_isolated_amd import rr
    return rr.rr_forward_fingerprint()


def measured_traffic(workload: str):
    """HBM bytes per launch of the attention kernel from the committed counter summary of
    this workload (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's reading), or
    None when there is none or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"k_attn_mfma_{workload.replace('-', '_')}_traffic.txt")
    try:
        with open(path) as fh:
            for line in fh:
                f = line.split()
                if len(f) == 4 and f[0] == "traffic_bytes_per_launch" and f[2] == "sources":
                    return float(f[1]) if f[3] == source_hash() else None
    except OSError:
        pass
    return None


def calibrate_copy(mib: int) -> None:
    """A plain copy kernel of known size, for scaling the HBM traffic counters."""
    import torch
    n = mib << 20
    src = torch.empty(4 * n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for i in range(3):
        dst.copy_(src[i * n:(i + 1) * n])   # a different, cold slice each time
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_per_copy": n, "copies": 3}), flush=True)


def make_batch(cfg):
    import workloads as W
    if cfg == 6:
        return W.config5_padded(attend_padded_history=True)
    if cfg == 7:
        return W.config5_padded(attend_padded_history=False)
    return W.make_config(cfg)


def describe(cfg, b):
    import numpy as np
    if cfg == 4:
        h = np.diff(b.hist_offsets)
        return {"workload": b.name, "mode": "candidate-only", "B": b.B, "Th": b.Th, "Tc": b.Tc,
                "H": b.H, "d": b.d, "hist_len": [int(h.min()), int(np.median(h)), int(h.max())],
                "cand_per_user": int(b.cand_offsets[1] - b.cand_offsets[0]), "seed": b.seed}
    return {"workload": b.name, "mode": "full-sequence", "B": b.B, "T": b.T, "H": b.H, "d": b.d,
            "prefix": int(b.prefix[0]), "hist_len": [int(b.hist.min()), int(np.median(b.hist)),
                                                      int(b.hist.max())],
            "cand_per_user": int(b.cand[0]), "padded": bool(b.valid is not None),
            "attend_padded_history": bool(b.attend_padded_history), "seed": b.seed}


def work_counts(cfg, b):
    """(effective FLOPs, executed FLOPs, algorithmic bytes, candidates) of one step."""
    from jagged_candidate_isolated_amd import accounting as acc
    es = 2 if b.dtype == "bf16" else 4
    if cfg == 4:
        import numpy as np
        pairs = acc.cand_only_pairs(np.diff(b.hist_offsets), np.diff(b.cand_offsets))
        f = acc.attention_flops(pairs, b.H, b.d)
        return f, f, acc.cand_only_bytes(b.Th, b.Tc, b.H, b.d, es), b.Tc
    eff, ex = acc.full_mode_counts(b.prefix, b.hist, b.cand, b.pad, b.attend_padded_history)
    return (acc.attention_flops(eff, b.H, b.d), acc.attention_flops(ex, b.H, b.d),
            acc.full_mode_bytes(b.T, b.H, b.d, es), int(b.cand.sum()))


def mfma_executed_flops(cfg, b):
    """FLOPs the forward kernel issues on the matrix cores for one step: every query tile
    (128 rows, or 256 when users average 2048 rows or more) runs whole over key blocks of 64
    columns (128 at d = 32), both products (S = K Q^T and O = V^T P^T) at 2 d FLOPs per
    pair; the library's tile rule.  None off the MFMA kernel (fp32, d = 16)."""
    import numpy as np
    from jagged_candidate_isolated_amd import accounting as acc
    if b.dtype != "bf16" or b.d < 32:
        return None
    bn = 128 if b.d == 32 else 64
    if cfg == 4:
        n_q, n_kv, rows = np.diff(b.cand_offsets), np.diff(b.hist_offsets), b.Tc
    else:
        pad = b.pad if b.attend_padded_history else 0
        n_kv = b.prefix + pad + b.hist
        n_q = n_kv + b.cand
        rows = b.T
    bm = 256 if rows >= 2048 * b.B else 128
    return acc.attention_flops(acc.tile_pairs(n_q, n_kv, bm, bn), b.H, b.d)


def self_planned(b) -> bool:
    """Whether rr_attn_fwd plans this batch inside the attention kernel (a small unpadded
    bf16 batch: at most 256 users, at most 1024 workgroups); the library's rule."""
    if b.valid is not None or b.dtype != "bf16" or b.d < 32:
        return False
    bm = 256 if b.T >= 2048 * b.B else 128
    q = 8 * 32           # whole XCD chunks of the forward kernel
    grid = (b.H + 1) * ((b.T + bm - 1) // bm + b.B)
    grid = (grid + q - 1) // q * q
    return b.B <= 256 and b.B <= 2 * bm and grid <= 1024


def key_bound_pass(b, cfg) -> bool:
    """Whether a planned full-sequence call of this batch first runs the key-norm pass
    (k_key_norms, the bound that lets the attention kernel skip tile maxima): bf16 wide
    tiles (users averaging 2048 rows or more) without a padding mask; the library's rule."""
    return (cfg != 4 and b.valid is None and b.dtype == "bf16" and b.d >= 32 and b.T >= 2048 * b.B
            and not self_planned(b))


def gpu_setup(cfg, b, torch, rr, rope=False, backward=False):
    """Device copies of the inputs (rotated), outputs, the workspace and the step calls:
    plan(), run(i) (with the rotary encoding first when ``rope``; forward with lse and then
    the backward when ``backward``), rope_only(i) and bwd_only(i)."""
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if b.dtype == "bf16" else torch.float32

    def up(x, dtype=None):
        t = torch.from_numpy(x).to(dev)
        return t if dtype is None else t.to(dtype)

    if cfg == 4:
        base = [up(b.q_cand, dt), up(b.k_hist, dt), up(b.v_hist, dt), up(b.k_cand, dt), up(b.v_cand, dt)]
        if backward:
            import workloads as W
            base.append(up(W.draw_output_grad(b.seed + 77, b.Tc, b.H, b.d, b.dtype), dt))
        hoff, coff = up(b.hist_offsets), up(b.cand_offsets)
        out_like = base[0]
        Th, Tc, H, d = b.Th, b.Tc, b.H, b.d
        nbytes = (rr.rr_cand_only_bwd_workspace_bytes if backward else rr.rr_cand_only_workspace_bytes)(b.B, Th, Tc,
                                                                                                       H, d)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    else:
        base = [up(b.q, dt), up(b.k, dt), up(b.v, dt)]
        if backward:
            import workloads as W
            base.append(up(W.draw_output_grad(b.seed + 77, b.T, b.H, b.d, b.dtype), dt))
        off, cst = up(b.offsets), up(b.cand_start)
        valid = None if b.valid is None else up(b.valid)
        out_like = base[0]
        nbytes = (rr.rr_attn_bwd_workspace_bytes if backward else rr.rr_attn_workspace_bytes)(b.B, b.T, b.H, b.d)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    n_out = 4 if backward else 1          # o (and dq, dk, dv)
    footprint = (sum(t.numel() * t.element_size() for t in base) +
                 n_out * out_like.numel() * out_like.element_size())
    copies = max(1, min(64, math.ceil(ROTATE_BYTES / footprint)))
    sets = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
    outs = [torch.empty_like(out_like) for _ in range(copies)]
    grads = [[torch.empty_like(out_like) for _ in range(3)] for _ in range(copies)] if backward and cfg != 4 else None
    lse = torch.empty((b.Tc if cfg == 4 else b.T, b.H), dtype=torch.float32, device=dev) if backward else None

    # rotary q / k land in one set of buffers that the attention of the same step reads
    rot = [torch.empty_like(t) for t in base] if rope else None
    bwd_only = rope_only = None
    if cfg == 4:
        hist_len = (hoff[1:] - hoff[:-1]).contiguous()
        hist_end, cand_first = hoff[1:].contiguous(), coff[:-1].contiguous()

        def plan():
            if not rope:      # the rotary step's attention call plans for itself
                rr.rr_cand_only_plan(hoff, coff, Th, Tc, H, d, dt, workspace=ws)

        def rope_only(i):     # the keys' rotary pass (the queries turn inside the attention kernel)
            s = sets[i % copies]
            rr.rr_rope_qk(None, s[1], hoff, hist_end, k_out=rot[1])
            rr.rr_rope_qk(None, s[3], coff, cand_first, pos_base=hist_len, k_out=rot[3])

        def bwd_only(i):
            s = sets[i % copies]
            rr.rr_cand_only_bwd_run(s[0], s[1], s[2], s[3], s[4], outs[i % copies], s[5], lse, hoff, coff, ws)

        def run(i):
            s = sets[i % copies]
            if rope:
                rope_only(i)
                rr.rr_cand_only_attn_fwd_rope(s[0], rot[1], s[2], rot[3], s[4], hoff, coff, out=outs[i % copies],
                                              workspace=ws)
            elif backward:
                rr.rr_cand_only_run_lse(s[0], s[1], s[2], s[3], s[4], b.B, ws, out=outs[i % copies], lse=lse)
                bwd_only(i)
            else:
                rr.rr_cand_only_run(s[0], s[1], s[2], s[3], s[4], b.B, ws, out=outs[i % copies])
    elif self_planned(b) and not rope and not backward:
        # the library plans inside the attention kernel for such a batch: one launch a step
        def plan():
            pass

        def run(i):
            s = sets[i % copies]
            rr.rr_attn_fwd(s[0], s[1], s[2], off, cst, valid, b.attend_padded_history, out=outs[i % copies],
                           workspace=ws)
    else:
        def plan():
            if not rope:      # the rotary step's attention call plans for itself
                rr.rr_attn_plan(off, cst, b.T, b.H, b.d, dt, valid=valid,
                                attend_padded_history=b.attend_padded_history, workspace=ws)

        def rope_only(i):     # the keys' rotary pass (the queries turn inside the attention kernel)
            s = sets[i % copies]
            rr.rr_rope_qk(None, s[1], off, cst, k_out=rot[1])

        def bwd_only(i):
            s, g = sets[i % copies], grads[i % copies]
            rr.rr_attn_bwd_run(s[0], s[1], s[2], outs[i % copies], s[3], lse, b.B, ws, dq=g[0], dk=g[1],
                               dv=g[2])

        def run(i):
            s = sets[i % copies]
            if rope:
                rope_only(i)
                rr.rr_attn_fwd_rope(s[0], rot[1], s[2], off, cst, out=outs[i % copies], workspace=ws)
            elif backward:
                rr.rr_attn_run_lse(s[0], s[1], s[2], b.B, ws, out=outs[i % copies], lse=lse)
                bwd_only(i)
            else:
                rr.rr_attn_run(s[0], s[1], s[2], b.B, ws, out=outs[i % copies])
    return plan, run, rope_only, bwd_only, copies, footprint


def host_info() -> dict:
    """The host the CPU baseline ran on: cores available to this process and the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return {"host_cores_available": avail, "cpu_model": model}


def cpu_baseline(cfg, b, budget_s, rope=False, backward=False):
    """The oracle, as it stands, on the host cores: whole batches (or the first users of one)
    repeated until about ``budget_s`` of CPU time; effective TFLOP/s of what it finished
    (forward and backward FLOPs when ``backward``: the forward oracle, then the gradients)."""
    import numpy as np
    from oracle import attention as A
    from oracle import backward as BW
    from oracle import rotary as RO
    full_fn = RO.full_attention_rope if rope else A.full_attention
    cand_fn = RO.cand_only_attention_rope if rope else A.cand_only_attention
    if backward:
        import workloads as W
        dout = W.draw_output_grad(b.seed + 77, b.Tc if cfg == 4 else b.T, b.H, b.d, b.dtype)

        def full_fn(q, k, v, offsets, cand_start, valid, flag, rows=slice(None)):
            A.full_attention(q, k, v, offsets, cand_start, valid, flag)
            BW.full_attention_backward(q, k, v, dout[rows], offsets, cand_start, valid, flag)

        def cand_fn(qc, kh, vh, kc, vc, hoff, coff, rows=slice(None)):
            A.cand_only_attention(qc, kh, vh, kc, vc, hoff, coff)
            BW.cand_only_attention_backward(qc, kh, vh, kc, vc, dout[rows], hoff, coff)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    from jagged_candidate_isolated_amd import accounting as acc
    t0 = time.perf_counter()
    done_flops, done_cands, reps, users = 0, 0, 0, 0
    if cfg == 4:
        hoff, coff = b.hist_offsets, b.cand_offsets
        hl = np.diff(hoff)
        cl = np.diff(coff)
        while time.perf_counter() - t0 < budget_s and users < b.B:
            u = users
            sl = slice(int(coff[u]), int(coff[u + 1]))
            extra = {"rows": sl} if backward else {}
            cand_fn(b.q_cand[sl], b.k_hist[int(hoff[u]):int(hoff[u + 1])],
                    b.v_hist[int(hoff[u]):int(hoff[u + 1])], b.k_cand[sl], b.v_cand[sl],
                    [0, int(hl[u])], [0, int(cl[u])], **extra)
            done_flops += acc.attention_flops(acc.cand_only_pairs([hl[u]], [cl[u]]), b.H, b.d)
            done_cands += int(cl[u])
            users += 1
        sample = (f"first {users} of {b.B} users, candidate-only oracle" + (" with rotary q/k" if rope else "")
                  + (", forward + backward" if backward else ""))
    else:
        eff_all, _ = acc.full_mode_counts(b.prefix, b.hist, b.cand, b.pad, b.attend_padded_history)
        small = b.T <= 40000
        while time.perf_counter() - t0 < budget_s:
            if small:
                full_fn(b.q, b.k, b.v, b.offsets, b.cand_start, b.valid, b.attend_padded_history)
                done_flops += acc.attention_flops(eff_all, b.H, b.d)
                done_cands += int(b.cand.sum())
                reps += 1
            else:
                if users >= b.B:
                    break
                u = users
                lo, hi = int(b.offsets[u]), int(b.offsets[u + 1])
                sl = slice(lo, hi)
                valid = None if b.valid is None else b.valid[sl]
                extra = {"rows": sl} if backward else {}
                full_fn(b.q[sl], b.k[sl], b.v[sl], [0, hi - lo], [int(b.cand_start[u]) - lo],
                        valid, b.attend_padded_history, **extra)
                e, _ = acc.full_mode_counts(b.prefix[u:u + 1], b.hist[u:u + 1], b.cand[u:u + 1],
                                            b.pad[u:u + 1], b.attend_padded_history)
                done_flops += acc.attention_flops(e, b.H, b.d)
                done_cands += int(b.cand[u])
                users += 1
        sample = ((f"whole batch x{reps}" if small else f"first {users} of {b.B} users") + ", float64 oracle"
                  + (" with rotary q/k" if rope else "") + (", forward + backward" if backward else ""))
    dt = time.perf_counter() - t0
    if backward:
        done_flops *= 3.5                 # forward + backward (2.5x), as the GPU figure counts
    return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2), "candidates_per_s": done_cands / dt, **host_info()}


RANKER_LAYERS, RANKER_CAND_ONLY = 8, 2


def ranker_counts(b):
    """(GEMM FLOPs, attention FLOPs) of one full request of the layer stack."""
    import numpy as np
    from jagged_candidate_isolated_amd import accounting as acc
    D = b.H * b.d
    Tc = int(b.cand.sum())
    Th = b.T - Tc
    n_full = RANKER_LAYERS - RANKER_CAND_ONLY
    gemm = n_full * 8.0 * b.T * D * D + RANKER_CAND_ONLY * (4.0 * Th * D * D + 8.0 * Tc * D * D)
    eff, _ = acc.full_mode_counts(b.prefix, b.hist, b.cand, b.pad, b.attend_padded_history)
    hl = b.prefix + b.hist
    pairs = acc.cand_only_pairs(hl, b.cand)
    attn = n_full * acc.attention_flops(eff, b.H, b.d) + RANKER_CAND_ONLY * acc.attention_flops(pairs, b.H, b.d)
    return gemm, attn


def ranker_cached_counts(b):
    from jagged_candidate_isolated_amd import accounting as acc
    D = b.H * b.d
    Tc = int(b.cand.sum())
    pairs = acc.cand_only_pairs(b.prefix + b.hist, b.cand)
    return RANKER_LAYERS * 8.0 * Tc * D * D, RANKER_LAYERS * acc.attention_flops(pairs, b.H, b.d)


def run_ranker(args, b, torch, rr):
    """The layer stack end to end: a full request and a cached request, graph-replayed."""
    import numpy as np
    import workloads as W
    dev = torch.device("cuda:0")
    D = b.H * b.d
    Tc = int(b.cand.sum())
    Th = b.T - Tc
    x0, layers = W.ranker_inputs(b.seed + 99, b.T, RANKER_LAYERS, D)
    dl = [(torch.from_numpy(g).to(dev), torch.from_numpy(wq).to(dev).to(torch.bfloat16),
           torch.from_numpy(wo).to(dev).to(torch.bfloat16)) for g, wq, wo in layers]
    x_src = torch.from_numpy(x0).to(dev)
    x = torch.empty_like(x_src)
    off = torch.from_numpy(b.offsets).to(dev)
    cst = torch.from_numpy(b.cand_start).to(dev)
    xc = torch.empty((Tc, D), dtype=torch.float32, device=dev)
    xh = torch.empty((Th, D), dtype=torch.float32, device=dev)
    cache = torch.empty((RANKER_LAYERS, 2, Th, b.H, b.d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(rr.rr_ranker_workspace_bytes(b.B, b.T, Tc, b.H, b.d), dtype=torch.uint8, device=dev)
    hoff = torch.from_numpy(np.concatenate([[0], np.cumsum(b.cand_start - b.offsets[:-1])]).astype(np.int32)).to(dev)
    coff = torch.from_numpy(np.concatenate([[0], np.cumsum(b.offsets[1:] - b.cand_start)]).astype(np.int32)).to(dev)
    cand_rows = np.concatenate([np.arange(b.cand_start[u], b.offsets[u + 1]) for u in range(b.B)]).astype(np.int64)
    xc_src = x_src[torch.from_numpy(cand_rows).to(dev)].contiguous()
    xc2 = torch.empty_like(xc_src)
    ws2 = torch.empty(rr.rr_ranker_cached_workspace_bytes(b.B, Th, Tc, b.H, b.d), dtype=torch.uint8, device=dev)

    ut, Tp = None, 0
    if args.update_user_token:
        ut = torch.from_numpy(b.prefix.astype(np.int32)).to(dev)
        Tp = int(b.prefix.sum())
        ws = torch.empty(rr.rr_ranker_workspace_bytes(b.B, b.T, Tc, b.H, b.d, Tp=Tp), dtype=torch.uint8,
                         device=dev)

    def full_step():
        x.copy_(x_src)
        rr.rr_ranker_fwd(x, dl, RANKER_CAND_ONLY, off, cst, Tc, b.H, b.d, x_cand_out=xc, x_hist_out=xh,
                         kv_cache=cache, workspace=ws, user_tokens=ut, Tp=Tp)

    def cached_step():
        xc2.copy_(xc_src)
        rr.rr_ranker_cached_fwd(xc2, dl, cache, hoff, coff, b.H, b.d, workspace=ws2)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3

    full_step(); torch.cuda.synchronize()
    t = time.perf_counter(); full_step(); torch.cuda.synchronize()
    est = time.perf_counter() - t
    steps = args.steps or int(min(2000, max(10, 1.0 / max(est, 1e-6))))
    warmup = args.warmup if args.warmup is not None else max(3, steps // 10)
    ms_full = timed(full_step, steps, warmup)
    ms_cached = timed(cached_step, steps, warmup)
    # the cached request reproduces the full request's candidates
    full_step(); cached_step(); torch.cuda.synchronize()
    same = bool(torch.equal(xc, xc2))
    gemm_f, attn_f = ranker_counts(b)
    gemm_c, attn_c = ranker_cached_counts(b)
    out = {
        "metric": "ranker layer stack (6 full + 2 candidate-only layers) end to end, candidates/s",
        "value": Tc / (ms_full / 1e3), "unit": "candidates/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_full, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (random projections)",
        "config": dict(describe(args.config, b), parallelism="none (1 GPU)", layers=RANKER_LAYERS,
                       cand_only_layers=RANKER_CAND_ONLY, D=D, update_user_token=bool(args.update_user_token),
                       step="copy of the input states + rr_ranker_fwd (kv cache written)"),
        "ranker": {
            "full_request": {"ms": ms_full, "candidates_per_s": Tc / (ms_full / 1e3),
                             "gemm_tflop": gemm_f / 1e12, "attention_tflop": attn_f / 1e12,
                             "tflops": (gemm_f + attn_f) / (ms_full / 1e3) / 1e12},
            "cached_request": {"ms": ms_cached, "candidates_per_s": Tc / (ms_cached / 1e3),
                               "gemm_tflop": gemm_c / 1e12, "attention_tflop": attn_c / 1e12,
                               "tflops": (gemm_c + attn_c) / (ms_cached / 1e3) / 1e12,
                               "bit_identical_to_full": same},
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = ranker_cpu_baseline(b, x0, layers, args.cpu_seconds,
                                                  user_tokens=b.prefix if args.update_user_token else None)
    print(json.dumps(out), flush=True)


def ranker_cpu_baseline(b, x0, layers, budget_s, user_tokens=None):
    """The oracle's layer stack on the first users of the batch, one user at a time, until
    about ``budget_s`` of CPU time; candidates/s."""
    import numpy as np
    from oracle import ranker as RK
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    ol = [RK.Layer(g.astype(np.float64), wq.astype(np.float64), wo.astype(np.float64)) for g, wq, wo in layers]
    t0 = time.perf_counter()
    users = cands = 0
    while time.perf_counter() - t0 < budget_s and users < b.B:
        lo, cs, hi = int(b.offsets[users]), int(b.cand_start[users]), int(b.offsets[users + 1])
        RK.ranker_forward(x0[lo:hi], ol, RANKER_CAND_ONLY, [0, hi - lo], [cs - lo], b.H, b.d,
                          user_tokens=None if user_tokens is None else user_tokens[users:users + 1])
        cands += hi - cs
        users += 1
    dt = time.perf_counter() - t0
    return {"value": cands / dt, "unit": "candidates/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {users} of {b.B} users, float64 layer-stack oracle", "seconds": round(dt, 2),
            **host_info()}


SECONDARY_STEPS = 2000   # steps of the secondary (short-history) measurement of the default line


def timed_steps(torch, plan, run, steps, copies):
    """Exactly ``steps`` steps (plan + run, step i on input copy i % copies), replayed from
    captured HIP graphs so the host's launch overhead does not pace the GPU; bracketed by
    device synchronisations.  Returns (seconds, timing mode)."""
    n1 = min(steps, max(copies, 256))
    reps, rem = divmod(steps, n1)

    def capture(n, first):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(first, first + n):
                plan(); run(i % copies)
        g.replay()
        return g
    try:
        g1 = capture(n1, 0)
        g2 = capture(rem, reps * n1) if rem else None
        torch.cuda.synchronize()
    except Exception as e:  # pragma: no cover - depends on the runtime
        print(f"graph capture unavailable ({e}); timing eager launches", file=sys.stderr)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            plan(); run(i % copies)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, "eager launches"
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g1.replay()
    if g2 is not None:
        g2.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, "hip graph replay"


def measure(cfg, args, torch, rr, steps_req, warmup_req, with_cpu):
    """One workload's bench record (the JSON object main prints)."""
    import numpy as np
    b = make_batch(cfg)
    eff_flops, exec_flops, alg_bytes, n_cands = work_counts(cfg, b)
    fwd_eff, fwd_exec = eff_flops, exec_flops
    if args.backward:       # a training step: forward + backward (2.5x the forward)
        eff_flops, exec_flops = 3.5 * eff_flops, 3.5 * exec_flops
    plan, run, rope_only, bwd_only, copies, footprint = gpu_setup(cfg, b, torch, rr, rope=args.rope,
                                                                  backward=args.backward)
    torch.cuda.synchronize()

    # size the run to about a second of GPU work unless told otherwise
    plan(); run(0); torch.cuda.synchronize()
    t = time.perf_counter()
    for i in range(3):
        plan(); run(i)
    torch.cuda.synchronize()
    est = (time.perf_counter() - t) / 3
    steps = steps_req or int(min(5000, max(20, 1.0 / max(est, 1e-6))))
    warmup = warmup_req if warmup_req is not None else max(5, steps // 10)

    for i in range(warmup):
        plan(); run(i % copies)
    torch.cuda.synchronize()

    wall, timing = timed_steps(torch, plan, run, steps, copies)
    ms_per_step = wall / steps * 1e3
    value = eff_flops / (ms_per_step / 1e3) / 1e12
    # One kernel alone: back-to-back launches replayed from a captured graph (no host
    # gaps), bracketed by HIP events recorded on the launch stream.
    stream = torch.cuda.current_stream()
    plan()
    n_run = copies
    reps_k = max(2, math.ceil(max(20, min(steps, 400)) / n_run))

    def time_launches(fn):
        g = None
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n_run):
                    fn(i)
            g.replay()
        except Exception as e:  # pragma: no cover
            print(f"graph capture unavailable ({e}); timing eager launches", file=sys.stderr)
            g = None
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps_k + 1)]
        ev[0].record(stream)
        for r in range(reps_k):
            if g is not None:
                g.replay()
            else:
                for i in range(n_run):
                    fn(i)
            ev[r + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev[r].elapsed_time(ev[r + 1]) / n_run for r in range(reps_k)]
        time_launches.median = float(np.median(per))
        return ev[0].elapsed_time(ev[-1]) / (reps_k * n_run)

    if args.rope:
        rope_ms = time_launches(rope_only)
        kernel_ms = time_launches(run) - rope_ms     # the attention of the rotary step
    elif args.backward:
        bwd_ms = time_launches(bwd_only)
        kernel_ms = time_launches(run) - bwd_ms      # the forward of the training step
    else:
        kernel_ms = time_launches(run)
        kernel_ms_median = time_launches.median
    # the roofline entry covers the forward kernel
    eff_flops_all, exec_flops_all = eff_flops, exec_flops
    eff_flops, exec_flops = fwd_eff, fwd_exec

    flop_per_byte = eff_flops / alg_bytes
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if b.dtype == "f32":
        roof = {"bound": "alu", "achieved": exec_flops / (kernel_ms / 1e3) / 1e12,
                "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s"}
    elif flop_per_byte < ridge:
        roof = {"bound": "hbm", "achieved": alg_bytes / (kernel_ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": exec_flops / (kernel_ms / 1e3) / 1e12,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(b.name)
    roof["kernel"] = "k_attn_mfma" if b.dtype == "bf16" and b.d >= 32 else "k_attn_simple"
    if key_bound_pass(b, cfg):   # the timed call holds both launches
        roof["kernel"] = "k_key_norms + k_attn_mfma"
    roof["self_planned"] = bool(cfg != 4 and self_planned(b) and not args.backward)
    roof["kernel_ms"] = kernel_ms
    if not (args.rope or args.backward):
        roof["kernel_ms_median"] = kernel_ms_median
    roof["alg_bytes"] = alg_bytes
    roof["alg_flops"] = exec_flops

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": b.dtype, "data": "synthetic",
        "config": dict(describe(cfg, b), parallelism="none (1 GPU)"),
        "candidates_per_s": n_cands / (ms_per_step / 1e3),
        "effective_flops_per_step": eff_flops_all, "executed_flops_per_step": exec_flops_all,
        "executed_tflops": exec_flops_all / (ms_per_step / 1e3) / 1e12,
        "input_copies_rotated": copies, "footprint_bytes": footprint,
        "timing": timing,
        "roofline": roof,
        # the forward kernel against both ceilings, whichever bounds it
        "fractions": {"mfma": (exec_flops / (kernel_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS
                               if b.dtype == "bf16" else None),
                      "hbm": alg_bytes / (kernel_ms / 1e3) / 1e9 / HBM_PEAK_GBS},
    }
    mfma_flops = mfma_executed_flops(cfg, b)
    if mfma_flops:
        out["mfma_efficiency"] = {"effective_flops": eff_flops, "mfma_flops": mfma_flops,
                                  "ratio": eff_flops / mfma_flops,
                                  "mfma_tflops": mfma_flops / (kernel_ms / 1e3) / 1e12}
    if args.rope:
        es = 2 if b.dtype == "bf16" else 4
        rows_k = (b.Th + b.Tc) if cfg == 4 else b.T                    # key rows rotated by the pass
        rope_bytes = 2 * rows_k * b.H * b.d * es                      # each read once, written once
        out["rope"] = {"kernel": "k_rope_qk (keys; queries rotate inside k_attn_mfma)", "kernel_ms": rope_ms,
                       "bound": "hbm",
                       "achieved": rope_bytes / (rope_ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": rope_bytes / (rope_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                       "alg_bytes": rope_bytes}
        out["config"]["rope"] = ("right-anchored rotary q/k, base 10000, inside every step: a rotary pass over the "
                                 "keys, the queries rotated in registers by the attention kernel")
    if args.backward:
        bwd_flops = 2.5 * fwd_exec
        out["backward"] = {"kernels": ["k_bwd_dq", "k_bwd_dkdv"], "kernel_ms": bwd_ms, "bound": "mfma",
                           "achieved": bwd_flops / (bwd_ms / 1e3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": bwd_flops / (bwd_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
                           "alg_flops": bwd_flops}
        out["config"]["step"] = "plan + forward with lse + backward (dq, dk, dv)"
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, b, args.cpu_seconds, rope=args.rope, backward=args.backward)
    return out


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): this path shards by "
              "user with no exchange, and no multi-GPU figure is measured here.", file=sys.stderr)
        sys.exit(2)
    import torch
    from jagged_candidate_isolated_amd import rr

    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return
    default_line = args.config is None
    cfg = 5 if default_line else args.config
    args.config = cfg
    if args.ranker:
        b = make_batch(cfg)
        if cfg in (4, 6, 7) or b.dtype != "bf16" or b.d not in (32, 64, 128) or (b.H * b.d) % 128:
            print("--ranker runs the full-sequence bf16 workloads without padding (configs 2, 3, 5)",
                  file=sys.stderr)
            sys.exit(2)
        run_ranker(args, b, torch, rr)
        return
    if args.rope and cfg in (1, 6, 7):
        print("--rope runs the unpadded bf16 workloads (configs 2 to 5): the queries turn inside the attention "
              "kernel, which takes no padding mask", file=sys.stderr)
        sys.exit(2)
    if args.backward and (cfg == 1 or args.rope):
        print("--backward runs the bf16 workloads with d 64 or 128 (configs 2 to 7), without --rope",
              file=sys.stderr)
        sys.exit(2)
    out = measure(cfg, args, torch, rr, args.steps, args.warmup, not args.no_cpu_baseline)
    if default_line and not (args.rope or args.backward):
        # the short-history workload's HBM roofline, measured in the same run
        sec = measure(2, args, torch, rr, SECONDARY_STEPS, None, False)
        out["secondary"] = {sec["config"]["workload"]: {
            k: sec[k] for k in ("value", "unit", "steps", "warmup", "ms_per_step", "candidates_per_s", "roofline",
                                "fractions", "mfma_efficiency", "timing", "input_copies_rotated") if k in sec}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
