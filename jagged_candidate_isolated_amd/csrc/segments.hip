// Segment IDs, bounds, data-contract checks and the compaction prologue.
//
// Segment rule: Candidate isolation attention mask page, section "段 ID：掩码的表达方式".
// Bounds: same section (history and candidate intervals derived from the segment IDs).
//
// Every kernel gives one workgroup to a user and loops over the user's rows, so
// no row needs a search for its user, and every row index is clamped into the
// user's own range and into [0, T).
#include "rr_internal.h"

namespace rr {
namespace {

constexpr int kThreads = 256;

struct SegParams {
  const int32_t* offsets;
  const int32_t* cand_start;
  const uint8_t* valid;
  int flag;
  int B;
  int T;
  int8_t* seg;
};

__device__ __forceinline__ void user_rows(const int32_t* offsets, int b, int T, int& lo, int& hi) {
  lo = min(max(offsets[b], 0), T);
  hi = min(max(offsets[b + 1], lo), T);
}

__global__ __launch_bounds__(kThreads) void k_segment_ids(SegParams p) {
  for (int b = blockIdx.x; b < p.B; b += gridDim.x) {
    int lo, hi;
    user_rows(p.offsets, b, p.T, lo, hi);
    const int cs = p.cand_start[b];
    for (int r = lo + threadIdx.x; r < hi; r += kThreads) {
      p.seg[r] = segment_of(r, cs, p.valid, p.flag);
    }
  }
}

struct BoundsParams {
  const int32_t* offsets;
  const int8_t* seg;
  int B;
  int T;
  int32_t* out;  // [4][B]
};

__global__ __launch_bounds__(kThreads) void k_bounds(BoundsParams p) {
  __shared__ int s_hlo, s_hhi, s_clo, s_chi;
  for (int b = blockIdx.x; b < p.B; b += gridDim.x) {
    int lo, hi;
    user_rows(p.offsets, b, p.T, lo, hi);
    if (threadIdx.x == 0) {
      s_hlo = INT32_MAX; s_hhi = INT32_MIN; s_clo = INT32_MAX; s_chi = INT32_MIN;
    }
    __syncthreads();
    int hlo = INT32_MAX, hhi = INT32_MIN, clo = INT32_MAX, chi = INT32_MIN;
    for (int r = lo + threadIdx.x; r < hi; r += kThreads) {
      const int8_t s = p.seg[r];
      if (s == 1) { hlo = min(hlo, r); hhi = max(hhi, r + 1); }
      if (s == -1) { clo = min(clo, r); chi = max(chi, r + 1); }
    }
    // min/max are order-free, so the result is deterministic
    if (hlo != INT32_MAX) { atomicMin(&s_hlo, hlo); atomicMax(&s_hhi, hhi); }
    if (clo != INT32_MAX) { atomicMin(&s_clo, clo); atomicMax(&s_chi, chi); }
    __syncthreads();
    if (threadIdx.x == 0) {
      const bool h_empty = s_hlo == INT32_MAX;
      const bool c_empty = s_clo == INT32_MAX;
      p.out[0 * p.B + b] = h_empty ? lo : s_hlo;
      p.out[1 * p.B + b] = h_empty ? lo : s_hhi;
      p.out[2 * p.B + b] = c_empty ? hi : s_clo;
      p.out[3 * p.B + b] = c_empty ? hi : s_chi;
    }
    __syncthreads();
  }
}

struct ValidateParams {
  const int32_t* offsets;
  const int32_t* cand_start;
  int B;
  int T;
  int32_t* err;
};

__global__ __launch_bounds__(kThreads) void k_validate(ValidateParams p) {
  int bits = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (p.offsets[0] != 0) bits |= 1;
    if (p.offsets[p.B] != p.T) bits |= 4;
  }
  for (int b = blockIdx.x * kThreads + threadIdx.x; b < p.B; b += gridDim.x * kThreads) {
    const int lo = p.offsets[b], hi = p.offsets[b + 1];
    if (hi < lo) bits |= 2;
    if (p.cand_start) {
      const int cs = p.cand_start[b];
      if (cs < lo || cs > hi) bits |= 8;
    }
  }
  if (bits) atomicOr(p.err, bits);
}

// Compaction prologue for batches with a padding mask.  For user b it writes the
// user's valid rows (segment != 0) in row order to idx[offsets[b] ...]; since
// every segment-1 row precedes every candidate row, the first n_kv of them are
// the keys and the rest are candidates.  The user's padding rows (segment 0)
// fill the rest of its idx range, from the end backwards; the attention kernel
// writes zeros to their output rows.
struct CompactParams {
  const int32_t* offsets;
  const int32_t* cand_start;
  const uint8_t* valid;
  int flag;
  int B;
  int T;
  UserMeta* meta;
  int32_t* idx;
};

__device__ __forceinline__ int block_exclusive_count(bool pred, int* s_wave, int& total) {
  // exclusive prefix count of `pred` over the workgroup (four waves of 64)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long m = __ballot(pred);
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[wave] = __popcll(m);
  __syncthreads();
  int before = 0;
  total = 0;
  for (int w = 0; w < kThreads / 64; ++w) {
    const int c = s_wave[w];
    if (w < wave) before += c;
    total += c;
  }
  __syncthreads();
  return before + in_wave;
}

__global__ __launch_bounds__(kThreads) void k_compact(CompactParams p) {
  __shared__ int s_wave[kThreads / 64];
  for (int b = blockIdx.x; b < p.B; b += gridDim.x) {
    int lo, hi;
    user_rows(p.offsets, b, p.T, lo, hi);
    const int cs = p.cand_start[b];
    int n_valid = 0, n_hist = 0, n_pad = 0;
    for (int base = lo; base < hi; base += kThreads) {
      const int r = base + threadIdx.x;
      const bool in = r < hi;
      const int8_t s = in ? segment_of(r, cs, p.valid, p.flag) : int8_t(0);
      int tot_v, tot_h, tot_p;
      const int pos_v = block_exclusive_count(in && s != 0, s_wave, tot_v);
      block_exclusive_count(in && s == 1, s_wave, tot_h);
      const int pos_p = block_exclusive_count(in && s == 0, s_wave, tot_p);
      if (in && s != 0) p.idx[lo + n_valid + pos_v] = r;
      if (in && s == 0) p.idx[hi - 1 - (n_pad + pos_p)] = r;
      n_valid += tot_v;
      n_hist += tot_h;
      n_pad += tot_p;
    }
    __syncthreads();   // this workgroup's idx writes are visible to its threads
    if (threadIdx.x == 0) {
      UserMeta m{};
      m.q_begin = lo;
      m.n_q = n_valid;
      m.kv_begin = lo;
      m.n_kv = n_hist;
      m.cand_rel = n_hist;
      m.n_pad = n_pad;
      // keys that form one row range (e.g. padding attended as history) load directly
      if (n_hist > 0) {
        const int first = p.idx[lo], last = p.idx[lo + n_hist - 1];
        if (last - first + 1 == n_hist) {
          m.kv_direct = 1;
          m.kv_begin = first;
        }
      }
      p.meta[b] = m;
    }
  }
}

int64_t user_grid(int B) { return B < 65535 ? B : 65535; }

}  // namespace

hipError_t launch_segment_ids(const int32_t* offsets, const int32_t* cand_start, const uint8_t* valid,
                              int flag, int B, int T, int8_t* seg, hipStream_t s) {
  return launch1(k_segment_ids, user_grid(B), kThreads, s,
                 SegParams{offsets, cand_start, valid, flag, B, T, seg});
}

hipError_t launch_bounds(const int32_t* offsets, const int8_t* seg, int B, int T, int32_t* out,
                         hipStream_t s) {
  return launch1(k_bounds, user_grid(B), kThreads, s, BoundsParams{offsets, seg, B, T, out});
}

hipError_t launch_validate(const int32_t* offsets, const int32_t* cand_start, int B, int T,
                           int32_t* err, hipStream_t s) {
  int64_t g = (B + kThreads - 1) / kThreads;
  g = g < 1 ? 1 : (g > 1024 ? 1024 : g);
  return launch1(k_validate, g, kThreads, s, ValidateParams{offsets, cand_start, B, T, err});
}

hipError_t launch_compact(const int32_t* offsets, const int32_t* cand_start, const uint8_t* valid,
                          int flag, int B, int T, UserMeta* meta, int32_t* idx, hipStream_t s) {
  return launch1(k_compact, user_grid(B), kThreads, s,
                 CompactParams{offsets, cand_start, valid, flag, B, T, meta, idx});
}

}  // namespace rr
