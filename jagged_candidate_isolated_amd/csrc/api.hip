// C ABI of librr: argument checks on the host, then stream-ordered launches.
// Nothing here waits for the device or allocates memory.
#include <math.h>

#include "rr_internal.h"

using namespace rr;

namespace {

constexpr int kAbiVersion = 1;

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
int status_of(hipError_t e) { return e == hipSuccess ? RR_OK : RR_EHIP; }

// The MFMA kernel takes bf16 with d >= 32; everything else runs on the VALU kernel.
// Its wide tile (256 query rows, deeper pipeline) pays off when users are long; the
// choice depends on host-known sizes only, so a plan and its run always agree.
bool use_mfma(int dtype, int d) { return dtype == RR_BF16 && d >= 32; }
int tile_rows(int dtype, int d, int64_t B, int64_t rows) {
  if (!use_mfma(dtype, d)) return kBmSimple;
  return rows >= int64_t(kWideMinRows) * B ? kBmMfmaWide : kBmMfmaNarrow;
}

float softmax_scale_log2(float scale, int d) {
  const float s = (scale > 0.f && isfinite(scale)) ? scale : 1.0f / sqrtf(static_cast<float>(d));
  return s * 1.4426950408889634f;  // log2(e)
}

// Sizes shared by both attention modes; returns RR_OK or the error.
int check_sizes(int32_t B, int32_t rows_kv, int32_t rows_q, int32_t H, int32_t d, int dtype) {
  if (B < 0 || rows_kv < 0 || rows_q < 0 || H < 0 || d < 0) return RR_EINVAL;
  if (dtype != RR_F32 && dtype != RR_BF16) return RR_EDTYPE;
  if (!supported_d(d)) return RR_EUNSUPPORTED;
  if (H > kMaxHeads) return RR_EUNSUPPORTED;
  if (item_upper_bound(B, rows_q, H) > 0x7fffffff) return RR_EUNSUPPORTED;
  // a work item packs its query tile above the 10 head bits of an int32: tiles of the
  // smallest height must number below 2^21 (about 134M query rows)
  if ((static_cast<int64_t>(rows_q) + kBmMin - 1) / kBmMin >= kMaxTiles) return RR_EUNSUPPORTED;
  return RR_OK;
}

template <typename T>
T* carve(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

struct Ws {
  PlanHeader* header;
  UserMeta* meta;
  int32_t* start;
  int32_t* idx;
  int2* items;
};

Ws carve_all(void* ws, const WsLayout& w) {
  return Ws{carve<PlanHeader>(ws, w.header), carve<UserMeta>(ws, w.meta), carve<int32_t>(ws, w.start),
            carve<int32_t>(ws, w.idx), carve<int2>(ws, w.items)};
}

int run_attention(const AttnArgs& a, int dtype, int d, int bm, int64_t rows, hipStream_t stream) {
  const int64_t grid = attn_grid(a.B, rows, a.H, bm);
  const hipError_t e = use_mfma(dtype, d) ? launch_attn_mfma(a, d, bm, grid, stream)
                                          : launch_attn_simple(a, d, dtype, grid, stream);
  return status_of(e);
}

// A full-sequence run over the plan in `workspace`.  With the wide tile (long users, many
// key tiles per query tile) the key-norm pass first writes its bounds into the workspace,
// so that the attention kernel can skip forming tile maxima that cannot move a row's
// reference (same bits either way; the pass reads the key rows once).
int run_full(AttnArgs a, int dtype, int d, int bm, int32_t T, void* workspace, hipStream_t stream) {
  if (use_mfma(dtype, d) && bm == kBmMfmaWide) {
    const WsLayout w = ws_layout(a.B, T, T, a.H);
    a.knorm = carve<float>(workspace, w.knorm);
    a.knorm_tiles = static_cast<int32_t>(w.knorm_tiles);
    const hipError_t e = launch_key_norms(a, T, d, stream);
    if (e != hipSuccess) return status_of(e);
  }
  return run_attention(a, dtype, d, bm, T, stream);
}

}  // namespace

extern "C" {

const char* rr_status_string(int status) {
  switch (status) {
    case RR_OK: return "ok";
    case RR_EINVAL: return "invalid argument (NULL pointer, negative or inconsistent size)";
    case RR_EDTYPE: return "unsupported dtype (use RR_F32 or RR_BF16)";
    case RR_EUNSUPPORTED: return "unsupported size (d must be 16, 32, 64 or 128; H <= 1023; rows < 2^27 - 63)";
    case RR_EWORKSPACE: return "workspace missing or too small";
    case RR_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int rr_abi_version(void) { return kAbiVersion; }

int rr_segment_ids(const int32_t* offsets, const int32_t* cand_start, const uint8_t* valid,
                   int attend_padded_history, int32_t B, int32_t T, int8_t* seg_out,
                   hipStream_t stream) {
  if (B < 0 || T < 0) return RR_EINVAL;
  if (B == 0 || T == 0) return RR_OK;
  if (!offsets || !cand_start || !seg_out) return RR_EINVAL;
  return status_of(launch_segment_ids(offsets, cand_start, valid, attend_padded_history ? 1 : 0, B,
                                      T, seg_out, stream));
}

int rr_bounds(const int32_t* offsets, const int8_t* seg, int32_t B, int32_t T, int32_t* bounds_out,
              hipStream_t stream) {
  if (B < 0 || T < 0) return RR_EINVAL;
  if (B == 0) return RR_OK;
  if (!offsets || !bounds_out || (T > 0 && !seg)) return RR_EINVAL;
  return status_of(launch_bounds(offsets, seg, B, T, bounds_out, stream));
}

size_t rr_attn_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t d) {
  if (check_sizes(B, T, T, H, d, RR_BF16) != RR_OK) return 0;
  return ws_layout(B, T, T, H).total;
}

}  // extern "C"

namespace {

// The plan of a full-sequence call for tiles of `bm` query rows, into a workspace the
// caller has checked.
int plan_full(const int32_t* offsets, const int32_t* cand_start, const uint8_t* valid,
              int attend_padded_history, int32_t B, int32_t T, int32_t H, int bm, void* workspace,
              hipStream_t stream) {
  const WsLayout w = ws_layout(B, T, T, H);
  const Ws p = carve_all(workspace, w);
  const int64_t cap = attn_grid(B, T, H, bm);   // <= w.item_bound
  hipError_t e = hipSuccess;
  if (valid) {
    // a padding mask: list each user's valid rows (keys first, then candidates) and its padding
    e = launch_compact(offsets, cand_start, valid, attend_padded_history ? 1 : 0, B, T, p.meta, p.idx,
                       stream);
    if (e == hipSuccess)
      e = launch_worklist(0, offsets, cand_start, 1, B, H, bm, T, T, static_cast<int>(cap), p.meta,
                          p.start, p.items, p.header, stream);
  } else {
    // every row valid: segment IDs and bounds follow from offsets and cand_start directly
    e = launch_worklist(0, offsets, cand_start, 0, B, H, bm, T, T, static_cast<int>(cap), p.meta,
                        p.start, p.items, p.header, stream);
  }
  return status_of(e);
}

// Forward arguments of a full-sequence run over a planned workspace.
AttnArgs full_args(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t T,
                   int32_t H, int32_t d, float scale, const void* workspace) {
  const Ws p = carve_all(const_cast<void*>(workspace), ws_layout(B, T, T, H));
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.k_self = k; a.v_self = v; a.o = o;
  a.plan = p.header; a.meta = p.meta; a.idx = p.idx; a.items = p.items;
  a.B = B; a.H = H; a.mode = 0; a.rows = T;
  a.scale_log2 = softmax_scale_log2(scale, d);
  return a;
}

bool bwd_supported(int dtype, int d) { return dtype == RR_BF16 && (d == 64 || d == 128); }

size_t bwd_delta_offset(int32_t B, int32_t T, int32_t H) { return align256(ws_layout(B, T, T, H).total); }

// Candidate-only backward workspace: the forward's plan, the key-major plan, rowsum(dO * o).
struct CandBwdWs {
  size_t key_plan, delta, total;
};
CandBwdWs cand_bwd_layout(int32_t B, int32_t Th, int32_t Tc, int32_t H) {
  CandBwdWs w{};
  w.key_plan = align256(ws_layout(B, 0, Tc, H).total);
  w.delta = w.key_plan + align256(ws_layout(B, 0, Th, H).total);
  w.total = w.delta + align256(sizeof(float) * size_t(Tc) * size_t(H));
  return w;
}

AttnArgs cand_args(const void* q_cand, const void* k_hist, const void* v_hist, const void* k_cand,
                   const void* v_cand, void* o_cand, int32_t B, int32_t Th, int32_t Tc, int32_t H, int32_t d,
                   float scale, const void* plan_ws, int mode) {
  const Ws p = carve_all(const_cast<void*>(plan_ws), ws_layout(B, 0, mode == 3 ? Th : Tc, H));
  AttnArgs a{};
  a.q = q_cand;
  a.k = Th > 0 ? k_hist : k_cand;   // with no frozen rows the key list is empty for every user
  a.v = Th > 0 ? v_hist : v_cand;
  a.k_self = k_cand; a.v_self = v_cand; a.o = o_cand;
  a.plan = p.header; a.meta = p.meta; a.idx = p.idx; a.items = p.items;
  a.B = B; a.H = H; a.mode = mode; a.rows = Tc;
  a.scale_log2 = softmax_scale_log2(scale, d);
  return a;
}


}  // namespace

extern "C" {

int rr_attn_plan(const int32_t* offsets, const int32_t* cand_start, const uint8_t* valid,
                 int attend_padded_history, int32_t B, int32_t T, int32_t H, int32_t d, int dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_sizes(B, T, T, H, d, dtype);
  if (st != RR_OK) return st;
  if (B == 0 || T == 0 || H == 0) return RR_OK;
  if (!offsets || !cand_start) return RR_EINVAL;
  if (!workspace || workspace_bytes < ws_layout(B, T, T, H).total) return RR_EWORKSPACE;
  return plan_full(offsets, cand_start, valid, attend_padded_history, B, T, H, tile_rows(dtype, d, B, T),
                   workspace, stream);
}

int rr_attn_run(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t T, int32_t H,
                int32_t d, int dtype, float scale, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  return rr_attn_run_lse(q, k, v, o, nullptr, B, T, H, d, dtype, scale, workspace, workspace_bytes,
                         stream);
}

int rr_attn_run_lse(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                    int32_t T, int32_t H, int32_t d, int dtype, float scale, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  const int st = check_sizes(B, T, T, H, d, dtype);
  if (st != RR_OK) return st;
  if (B == 0 || T == 0 || H == 0) return RR_OK;
  if (!q || !k || !v || !o) return RR_EINVAL;
  if (!workspace || workspace_bytes < ws_layout(B, T, T, H).total) return RR_EWORKSPACE;
  AttnArgs a = full_args(q, k, v, o, B, T, H, d, scale, workspace);
  a.lse = lse;
  return run_full(a, dtype, d, tile_rows(dtype, d, B, T), T, workspace, stream);
}

size_t rr_attn_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t d) {
  if (check_sizes(B, T, T, H, d, RR_BF16) != RR_OK || !bwd_supported(RR_BF16, d)) return 0;
  return bwd_delta_offset(B, T, H) + align256(sizeof(float) * size_t(T) * size_t(H));
}

int rr_attn_bwd_run(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, int32_t B, int32_t T, int32_t H,
                    int32_t d, int dtype, float scale, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  const int st = check_sizes(B, T, T, H, d, dtype);
  if (st != RR_OK) return st;
  if (!bwd_supported(dtype, d)) return RR_EUNSUPPORTED;
  if (B == 0 || T == 0 || H == 0) return RR_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return RR_EINVAL;
  if (!workspace || workspace_bytes < rr_attn_bwd_workspace_bytes(B, T, H, d)) return RR_EWORKSPACE;
  const AttnArgs a = full_args(q, k, v, const_cast<void*>(o), B, T, H, d, scale, workspace);
  float* delta = carve<float>(workspace, bwd_delta_offset(B, T, H));
  const float sc = (scale > 0.f && isfinite(scale)) ? scale : 1.0f / sqrtf(static_cast<float>(d));
  const int bm = tile_rows(dtype, d, B, T);   // the plan rr_attn_plan made for these sizes
  const int64_t grid = attn_grid(B, T, H, bm);
  return status_of(launch_attn_bwd(a, bm, grid, a, bm, grid, dout, lse, dq, dk, dv, dk, dv, delta, sc, d, stream));
}

int rr_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, const int32_t* offsets,
                const int32_t* cand_start, const uint8_t* valid, int attend_padded_history, int32_t B,
                int32_t T, int32_t H, int32_t d, int dtype, float scale, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  const int st = check_sizes(B, T, T, H, d, dtype);
  if (st != RR_OK) return st;
  if (!bwd_supported(dtype, d)) return RR_EUNSUPPORTED;
  if (B == 0 || T == 0 || H == 0) return RR_OK;
  if (!offsets || !cand_start) return RR_EINVAL;
  if (!workspace || workspace_bytes < rr_attn_bwd_workspace_bytes(B, T, H, d)) return RR_EWORKSPACE;
  const int r = rr_attn_plan(offsets, cand_start, valid, attend_padded_history, B, T, H, d, dtype,
                             workspace, workspace_bytes, stream);
  if (r != RR_OK) return r;
  return rr_attn_bwd_run(q, k, v, o, dout, lse, dq, dk, dv, B, T, H, d, dtype, scale, workspace,
                         workspace_bytes, stream);
}

}  // extern "C"

namespace {

// rr_attn_fwd, with the queries rotated in the attention kernel when rope_log2_base != 0
// (then the batch has no padding mask and the kernel is the MFMA one).
int attn_fwd(const void* q, const void* k, const void* v, void* o, const int32_t* offsets,
             const int32_t* cand_start, const uint8_t* valid, int attend_padded_history, int32_t B, int32_t T,
             int32_t H, int32_t d, int dtype, float scale, double rope_log2_base, void* workspace,
             size_t workspace_bytes, hipStream_t stream) {
  const int st = check_sizes(B, T, T, H, d, dtype);
  if (st != RR_OK) return st;
  if (B == 0 || T == 0 || H == 0) return RR_OK;
  if (!q || !k || !v || !o) return RR_EINVAL;
  const int bm = tile_rows(dtype, d, B, T);
  const int64_t grid = attn_grid(B, T, H, bm);
  if (!valid && use_mfma(dtype, d) && B <= kSelfPlanUsers && B <= 2 * bm && grid <= kSelfPlanGrid) {
    // a small unpadded batch: every workgroup plans for itself, no planning launch
    if (!offsets || !cand_start) return RR_EINVAL;
    if (!workspace || workspace_bytes < ws_layout(B, T, T, H).total) return RR_EWORKSPACE;
    AttnArgs a = full_args(q, k, v, o, B, T, H, d, scale, workspace);
    a.offsets = offsets;
    a.cand_start = cand_start;
    a.rope_log2_base = rope_log2_base;
    return status_of(launch_attn_mfma_self_planned(a, d, bm, grid, stream));
  }
  const int r = rr_attn_plan(offsets, cand_start, valid, attend_padded_history, B, T, H, d, dtype,
                             workspace, workspace_bytes, stream);
  if (r != RR_OK) return r;
  AttnArgs a = full_args(q, k, v, o, B, T, H, d, scale, workspace);
  a.rope_log2_base = rope_log2_base;
  return run_full(a, dtype, d, bm, T, workspace, stream);
}

double rope_log2(float theta_base) {
  return log2((theta_base > 0.f && isfinite(theta_base)) ? static_cast<double>(theta_base) : 10000.0);
}

}  // namespace

extern "C" {

int rr_attn_fwd(const void* q, const void* k, const void* v, void* o, const int32_t* offsets,
                const int32_t* cand_start, const uint8_t* valid, int attend_padded_history,
                int32_t B, int32_t T, int32_t H, int32_t d, int dtype, float scale,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return attn_fwd(q, k, v, o, offsets, cand_start, valid, attend_padded_history, B, T, H, d, dtype, scale, 0.0,
                  workspace, workspace_bytes, stream);
}

int rr_attn_fwd_rope(const void* q, const void* k, const void* v, void* o, const int32_t* offsets,
                     const int32_t* cand_start, int32_t B, int32_t T, int32_t H, int32_t d, int dtype, float scale,
                     float theta_base, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_sizes(B, T, T, H, d, dtype);
  if (st != RR_OK) return st;
  if (!use_mfma(dtype, d)) return RR_EUNSUPPORTED;
  return attn_fwd(q, k, v, o, offsets, cand_start, nullptr, 0, B, T, H, d, dtype, scale, rope_log2(theta_base),
                  workspace, workspace_bytes, stream);
}

size_t rr_cand_only_workspace_bytes(int32_t B, int32_t Th, int32_t Tc, int32_t H, int32_t d) {
  if (check_sizes(B, Th, Tc, H, d, RR_BF16) != RR_OK) return 0;
  return ws_layout(B, 0, Tc, H).total;
}

int rr_cand_only_plan(const int32_t* hist_offsets, const int32_t* cand_offsets, int32_t B, int32_t Th,
                      int32_t Tc, int32_t H, int32_t d, int dtype, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  const int st = check_sizes(B, Th, Tc, H, d, dtype);
  if (st != RR_OK) return st;
  if (B == 0 || Tc == 0 || H == 0) return RR_OK;
  if (!hist_offsets || !cand_offsets) return RR_EINVAL;
  const WsLayout w = ws_layout(B, 0, Tc, H);
  if (!workspace || workspace_bytes < w.total) return RR_EWORKSPACE;
  const Ws p = carve_all(workspace, w);
  const int bm = tile_rows(dtype, d, B, Tc);
  const int64_t cap = attn_grid(B, Tc, H, bm);   // <= w.item_bound
  return status_of(launch_worklist(1, hist_offsets, cand_offsets, 0, B, H, bm, Tc, Th,
                                   static_cast<int>(cap), p.meta, p.start, p.items, p.header, stream));
}

int rr_cand_only_run(const void* q_cand, const void* k_hist, const void* v_hist, const void* k_cand,
                     const void* v_cand, void* o_cand, int32_t B, int32_t Th, int32_t Tc, int32_t H,
                     int32_t d, int dtype, float scale, const void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  const int st = check_sizes(B, Th, Tc, H, d, dtype);
  if (st != RR_OK) return st;
  if (B == 0 || Tc == 0 || H == 0) return RR_OK;
  if (!q_cand || !k_cand || !v_cand || !o_cand) return RR_EINVAL;
  if (Th > 0 && (!k_hist || !v_hist)) return RR_EINVAL;
  const WsLayout w = ws_layout(B, 0, Tc, H);
  if (!workspace || workspace_bytes < w.total) return RR_EWORKSPACE;
  const Ws p = carve_all(const_cast<void*>(workspace), w);
  AttnArgs a{};
  a.q = q_cand;
  a.k = Th > 0 ? k_hist : k_cand;   // with no frozen rows the key list is empty for every user
  a.v = Th > 0 ? v_hist : v_cand;
  a.k_self = k_cand; a.v_self = v_cand; a.o = o_cand;
  a.plan = p.header; a.meta = p.meta; a.idx = p.idx; a.items = p.items;
  a.B = B; a.H = H; a.mode = 1; a.rows = Tc;
  a.scale_log2 = softmax_scale_log2(scale, d);
  return run_attention(a, dtype, d, tile_rows(dtype, d, B, Tc), Tc, stream);
}

int rr_cand_only_attn_fwd_rope(const void* q_cand, const void* k_hist, const void* v_hist, const void* k_cand,
                               const void* v_cand, void* o_cand, const int32_t* hist_offsets,
                               const int32_t* cand_offsets, int32_t B, int32_t Th, int32_t Tc, int32_t H, int32_t d,
                               int dtype, float scale, float theta_base, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  const int st = check_sizes(B, Th, Tc, H, d, dtype);
  if (st != RR_OK) return st;
  if (!use_mfma(dtype, d)) return RR_EUNSUPPORTED;
  if (B == 0 || Tc == 0 || H == 0) return RR_OK;
  if (!q_cand || !k_cand || !v_cand || !o_cand) return RR_EINVAL;
  if (Th > 0 && (!k_hist || !v_hist)) return RR_EINVAL;
  const int r = rr_cand_only_plan(hist_offsets, cand_offsets, B, Th, Tc, H, d, dtype, workspace,
                                  workspace_bytes, stream);
  if (r != RR_OK) return r;
  AttnArgs a = cand_args(q_cand, k_hist, v_hist, k_cand, v_cand, o_cand, B, Th, Tc, H, d, scale, workspace, 1);
  a.rope_log2_base = rope_log2(theta_base);
  return run_attention(a, dtype, d, tile_rows(dtype, d, B, Tc), Tc, stream);
}

int rr_cand_only_attn_fwd(const void* q_cand, const void* k_hist, const void* v_hist,
                          const void* k_cand, const void* v_cand, void* o_cand,
                          const int32_t* hist_offsets, const int32_t* cand_offsets, int32_t B,
                          int32_t Th, int32_t Tc, int32_t H, int32_t d, int dtype, float scale,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_sizes(B, Th, Tc, H, d, dtype);
  if (st != RR_OK) return st;
  if (B == 0 || Tc == 0 || H == 0) return RR_OK;
  if (!q_cand || !k_cand || !v_cand || !o_cand) return RR_EINVAL;
  if (Th > 0 && (!k_hist || !v_hist)) return RR_EINVAL;
  const int r = rr_cand_only_plan(hist_offsets, cand_offsets, B, Th, Tc, H, d, dtype, workspace,
                                  workspace_bytes, stream);
  if (r != RR_OK) return r;
  return rr_cand_only_run(q_cand, k_hist, v_hist, k_cand, v_cand, o_cand, B, Th, Tc, H, d, dtype,
                          scale, workspace, workspace_bytes, stream);
}

size_t rr_user_token_attn_workspace_bytes(int32_t B, int32_t Tk, int32_t Tq, int32_t H, int32_t d) {
  return rr_cand_only_workspace_bytes(B, Tk, Tq, H, d);
}

int rr_cand_only_run_lse(const void* q_cand, const void* k_hist, const void* v_hist, const void* k_cand,
                         const void* v_cand, void* o_cand, float* lse, int32_t B, int32_t Th, int32_t Tc, int32_t H,
                         int32_t d, int dtype, float scale, const void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  const int st = check_sizes(B, Th, Tc, H, d, dtype);
  if (st != RR_OK) return st;
  if (B == 0 || Tc == 0 || H == 0) return RR_OK;
  if (!q_cand || !k_cand || !v_cand || !o_cand) return RR_EINVAL;
  if (Th > 0 && (!k_hist || !v_hist)) return RR_EINVAL;
  if (!workspace || workspace_bytes < ws_layout(B, 0, Tc, H).total) return RR_EWORKSPACE;
  AttnArgs a = cand_args(q_cand, k_hist, v_hist, k_cand, v_cand, o_cand, B, Th, Tc, H, d, scale, workspace, 1);
  a.lse = lse;
  return run_attention(a, dtype, d, tile_rows(dtype, d, B, Tc), Tc, stream);
}

size_t rr_cand_only_bwd_workspace_bytes(int32_t B, int32_t Th, int32_t Tc, int32_t H, int32_t d) {
  if (check_sizes(B, Th, Tc, H, d, RR_BF16) != RR_OK || check_sizes(B, Tc, Th, H, d, RR_BF16) != RR_OK ||
      !bwd_supported(RR_BF16, d))
    return 0;
  return cand_bwd_layout(B, Th, Tc, H).total;
}

int rr_cand_only_bwd_run(const void* q_cand, const void* k_hist, const void* v_hist, const void* k_cand,
                         const void* v_cand, const void* o_cand, const void* dout, const float* lse, void* dq_cand,
                         void* dk_hist, void* dv_hist, void* dk_cand, void* dv_cand, const int32_t* hist_offsets,
                         const int32_t* cand_offsets, int32_t B, int32_t Th, int32_t Tc, int32_t H, int32_t d,
                         int dtype, float scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_sizes(B, Th, Tc, H, d, dtype);
  if (st == RR_OK) st = check_sizes(B, Tc, Th, H, d, dtype);   // the key-major plan's item bound
  if (st != RR_OK) return st;
  if (!bwd_supported(dtype, d)) return RR_EUNSUPPORTED;
  if (B == 0 || H == 0 || (Th == 0 && Tc == 0)) return RR_OK;
  if (!hist_offsets || !cand_offsets) return RR_EINVAL;
  if (Tc > 0 && (!q_cand || !k_cand || !v_cand || !o_cand || !dout || !lse || !dq_cand || !dk_cand || !dv_cand))
    return RR_EINVAL;
  if (Th > 0 && (!k_hist || !v_hist || !dk_hist || !dv_hist)) return RR_EINVAL;
  if (!workspace || workspace_bytes < rr_cand_only_bwd_workspace_bytes(B, Th, Tc, H, d)) return RR_EWORKSPACE;
  const CandBwdWs w = cand_bwd_layout(B, Th, Tc, H);
  void* key_ws = carve<char>(workspace, w.key_plan);
  float* delta = carve<float>(workspace, w.delta);
  // the key-major plan: items over each user's frozen history keys, 128 per tile
  const Ws kp = carve_all(key_ws, ws_layout(B, 0, Th, H));
  const int64_t grid_k = Th > 0 ? attn_grid(B, Th, H, kBmMfmaNarrow) : 0;
  if (grid_k > 0) {
    const hipError_t e = launch_worklist(3, hist_offsets, cand_offsets, 0, B, H, kBmMfmaNarrow, Tc, Th,
                                         static_cast<int>(grid_k), kp.meta, kp.start, kp.items, kp.header, stream);
    if (e != hipSuccess) return status_of(e);
  }
  const void* q = q_cand ? q_cand : k_hist;   // any rows in bounds: Tc == 0 launches no query-major work
  const void* kc = k_cand ? k_cand : k_hist;
  const void* vc = v_cand ? v_cand : v_hist;
  const AttnArgs aq = cand_args(q, k_hist, v_hist, kc, vc, const_cast<void*>(o_cand), B, Th, Tc, H, d, scale,
                                workspace, 1);
  const AttnArgs ak = cand_args(q, k_hist, v_hist, kc, vc, const_cast<void*>(o_cand), B, Th, Tc, H, d, scale,
                                key_ws, 3);
  const float sc = (scale > 0.f && isfinite(scale)) ? scale : 1.0f / sqrtf(static_cast<float>(d));
  const int bm_q = tile_rows(dtype, d, B, Tc);   // the plan rr_cand_only_plan made for these sizes
  const int64_t grid_q = Tc > 0 ? attn_grid(B, Tc, H, bm_q) : 0;
  return status_of(launch_attn_bwd(aq, bm_q, grid_q, ak, kBmMfmaNarrow, grid_k, dout, lse, dq_cand, dk_hist,
                                   dv_hist, dk_cand, dv_cand, delta, sc, d, stream));
}

int rr_user_token_attn_plan(const int32_t* key_offsets, const int32_t* query_offsets, int32_t B, int32_t Tk,
                            int32_t Tq, int32_t H, int32_t d, int dtype, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  const int st = check_sizes(B, Tk, Tq, H, d, dtype);
  if (st != RR_OK) return st;
  if (B == 0 || Tq == 0 || H == 0) return RR_OK;
  if (!key_offsets || !query_offsets) return RR_EINVAL;
  const WsLayout w = ws_layout(B, 0, Tq, H);
  if (!workspace || workspace_bytes < w.total) return RR_EWORKSPACE;
  const Ws p = carve_all(workspace, w);
  const int bm = tile_rows(dtype, d, B, Tq);
  const int64_t cap = attn_grid(B, Tq, H, bm);
  return status_of(launch_worklist(2, key_offsets, query_offsets, 0, B, H, bm, Tq, Tk, static_cast<int>(cap),
                                   p.meta, p.start, p.items, p.header, stream));
}

int rr_user_token_attn_run(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t Tk,
                           int32_t Tq, int32_t H, int32_t d, int dtype, float scale, const void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  const int st = check_sizes(B, Tk, Tq, H, d, dtype);
  if (st != RR_OK) return st;
  if (B == 0 || Tq == 0 || H == 0) return RR_OK;
  if (!q || !o || (Tk > 0 && (!k || !v))) return RR_EINVAL;
  const WsLayout w = ws_layout(B, 0, Tq, H);
  if (!workspace || workspace_bytes < w.total) return RR_EWORKSPACE;
  const Ws p = carve_all(const_cast<void*>(workspace), w);
  AttnArgs a{};
  a.q = q;
  a.k = Tk > 0 ? k : q;      // with no keys every row's list is empty; never read then
  a.v = Tk > 0 ? v : q;
  a.k_self = q; a.v_self = q;   // in bounds for every query row; no self-term is taken
  a.o = o;
  a.plan = p.header; a.meta = p.meta; a.idx = p.idx; a.items = p.items;
  a.B = B; a.H = H; a.mode = 2; a.rows = Tq;
  a.scale_log2 = softmax_scale_log2(scale, d);
  return run_attention(a, dtype, d, tile_rows(dtype, d, B, Tq), Tq, stream);
}

int rr_rope_positions(const int32_t* offsets, const int32_t* cand_start, const int32_t* pos_base,
                      int32_t B, int32_t T, int32_t* pos_out, hipStream_t stream) {
  if (B < 0 || T < 0) return RR_EINVAL;
  if (B == 0 || T == 0) return RR_OK;
  if (!offsets || !cand_start || !pos_out) return RR_EINVAL;
  return status_of(launch_rope_positions(offsets, cand_start, pos_base, B, T, pos_out, stream));
}

int rr_rope_qk(const void* q, const void* k, void* q_out, void* k_out, const int32_t* offsets,
               const int32_t* cand_start, const int32_t* pos_base, int32_t B, int32_t T, int32_t H,
               int32_t d, int dtype, float theta_base, hipStream_t stream) {
  if (B < 0 || T < 0 || H < 0 || d < 0) return RR_EINVAL;
  if (dtype != RR_F32 && dtype != RR_BF16) return RR_EDTYPE;
  if (d % 2 != 0 || d < 2 || d > 256) return RR_EUNSUPPORTED;
  if (B == 0 || T == 0 || H == 0 || (!q && !k)) return RR_OK;
  if (!offsets || !cand_start || (q && !q_out) || (k && !k_out)) return RR_EINVAL;
  if (static_cast<int64_t>(T) * H * d > (int64_t(1) << 40)) return RR_EUNSUPPORTED;
  const double base = (theta_base > 0.f && isfinite(theta_base)) ? static_cast<double>(theta_base) : 10000.0;
  return status_of(launch_rope_qk(q, k, q_out, k_out, offsets, cand_start, pos_base, B, T, H, d, dtype,
                                  log2(base), stream));
}

int rr_validate_jagged(const int32_t* offsets, const int32_t* cand_start, int32_t B, int32_t T,
                       int32_t* err_flags, hipStream_t stream) {
  if (B < 0 || T < 0) return RR_EINVAL;
  if (!offsets || !err_flags) return RR_EINVAL;
  return status_of(launch_validate(offsets, cand_start, B, T, err_flags, stream));
}

}  // extern "C"
