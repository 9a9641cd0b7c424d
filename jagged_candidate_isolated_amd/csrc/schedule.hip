// Length-sorted work list for ragged users.
//
// One workgroup builds, entirely on the device (the host never waits for the
// lengths), the list of attention work items: user b, head h, query tile qt.
// Users are ordered by the number of keys their queries read, longest first
// (longest-processing-time order), so the GPU's in-order workgroup dispatch
// starts the expensive items first and the short ones fill the tail.  The order
// is a counting sort over 128 logarithmic key-count buckets (four per octave):
// three barriers whatever the batch size, and within a bucket key counts differ
// by less than 19%, which is all the scheduling needs.  (The order of users that
// share a bucket may vary from call to call; it decides only which workgroup
// computes an item, never a result, since items write disjoint rows.)  Within a
// user the items go head by head, query tile by query tile, so neighbouring
// items read the same keys and values.
//
// Prior art: the CTI inference notes (varlen flash-attention section) build a
// block-to-sequence map on the device with a shape-derived grid upper bound and
// no host synchronisation; the grid of the attention kernels here follows the
// same idea (surplus workgroups exit at once).
#include "rr_internal.h"

namespace rr {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;
struct WorklistParams {
  int mode;              // 0: full sequence (offs_a = offsets, offs_b = cand_start)
                         // 1: candidate-only (offs_a = hist_offsets, offs_b = cand_offsets)
                         // 2: as 1 with no self-term (user-token rows: offs_b = their offsets)
                         // 3: as 1, items over key tiles (the key-major backward kernel)
  const int32_t* offs_a;
  const int32_t* offs_b;
  int meta_ready;        // meta[] already written by the compaction prologue
  int B;
  int H;
  int bm;                // query rows per tile
  int rows;              // T (full) or Tc (candidate-only), recorded in the plan header
  int kv_rows;           // rows of the key tensor (T, or Th in candidate-only mode)
  int cap;               // item capacity (= the attention grid); never exceeded, whatever the offsets
  UserMeta* meta;
  int32_t* start;        // [B + 1]
  int2* items;
  PlanHeader* header;
};

// Items of one user: H per query tile (per key tile in a key-major plan), plus one per
// tile of padding rows to zero.
__device__ __forceinline__ int user_items(const UserMeta& m, int H, int bm, int& nqt, int& nzt,
                                          bool key_major) {
  nqt = (max(key_major ? m.n_kv : m.n_q, 0) + bm - 1) / bm;
  nzt = (max(m.n_pad, 0) + bm - 1) / bm;
  return H * nqt + nzt;
}

// Row ranges are clamped into the tensors, so offsets that break the data contract
// give wrong numbers but never an access outside [0, rows).
__device__ __forceinline__ UserMeta plain_meta(const WorklistParams& p, int b) {
  UserMeta m{};
  if (p.mode == 0) {
    const int lo = min(max(p.offs_a[b], 0), p.rows);
    const int hi = min(max(p.offs_a[b + 1], lo), p.rows);
    const int cs = min(max(p.offs_b[b], lo), hi);
    m.q_begin = lo;
    m.n_q = hi - lo;
    m.kv_begin = lo;
    m.n_kv = cs - lo;
    m.cand_rel = cs - lo;
  } else {
    const int hl = min(max(p.offs_a[b], 0), p.kv_rows);
    const int hh = min(max(p.offs_a[b + 1], hl), p.kv_rows);
    const int cl = min(max(p.offs_b[b], 0), p.rows);
    const int ch = min(max(p.offs_b[b + 1], cl), p.rows);
    m.q_begin = cl;
    m.n_q = ch - cl;
    m.kv_begin = hl;
    m.n_kv = hh - hl;
    m.cand_rel = p.mode == 2 ? m.n_q : 0;   // mode 2: no query reads its own row
  }
  return m;
}

// Inclusive scan of one int per thread over the workgroup: shuffles within each
// wave, one barrier for the wave totals.
__device__ __forceinline__ int block_inclusive_scan(int x, int* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wave[w];
  __syncthreads();
  return x + before;
}

// Users up to kSortMax are planned entirely in LDS: one global read of the offsets,
// then the counting sort, the scan and the item writes without further global
// round trips.  Larger batches keep the user order and read the per-user counts
// back from `meta`.
__global__ __launch_bounds__(kThreads) void k_worklist(WorklistParams p) {
  __shared__ int s_order[kSortMax];      // users, longest key list first
  __shared__ int s_nqt[kSortMax];
  __shared__ int s_nzt[kSortMax];
  __shared__ unsigned char s_bkt[kSortMax];
  __shared__ int s_start[kSortMax + 1];
  __shared__ int s_hist[kBuckets];
  __shared__ int s_wave[kWavesPerBlock];
  const int tid = threadIdx.x;
  const bool in_lds = p.B <= kSortMax;

  for (int i = tid; i < kBuckets; i += kThreads) s_hist[i] = 0;
  __syncthreads();
  // 1. per-user counts (and the meta the attention kernel reads), bucket histogram
  for (int b = tid; b < p.B; b += kThreads) {
    const UserMeta m = p.meta_ready ? p.meta[b] : plain_meta(p, b);
    if (!p.meta_ready) p.meta[b] = m;
    if (in_lds) {
      int nqt, nzt;
      user_items(m, p.H, p.bm, nqt, nzt, p.mode == 3);
      s_nqt[b] = nqt;
      s_nzt[b] = nzt;
      const int k = cost_bucket(p.mode == 3 ? m.n_q : m.n_kv);   // the length each item loops over
      s_bkt[b] = static_cast<unsigned char>(k);
      atomicAdd(&s_hist[k], 1);
    }
  }
  __syncthreads();   // also makes the meta writes visible to the whole workgroup

  // 2. counting sort: bucket offsets (one wave scans the 128 buckets), then scatter
  if (in_lds) {
    if (tid < 64) {
      const int a = s_hist[2 * tid], c = s_hist[2 * tid + 1];
      int x = a + c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (tid >= off) x += y;
      }
      s_hist[2 * tid] = x - a - c;       // exclusive offsets
      s_hist[2 * tid + 1] = x - c;
    }
    __syncthreads();
    for (int b = tid; b < p.B; b += kThreads) s_order[atomicAdd(&s_hist[s_bkt[b]], 1)] = b;
    __syncthreads();
  }

  // 3. exclusive scan of the item counts in that order
  int carry = 0;
  for (int base = 0; base < p.B; base += kThreads) {
    const int r = base + tid;
    int cnt = 0;
    if (r < p.B) {
      if (in_lds) {
        const int b = s_order[r];
        cnt = p.H * s_nqt[b] + s_nzt[b];
      } else {
        int nqt, nzt;
        cnt = user_items(p.meta[r], p.H, p.bm, nqt, nzt, p.mode == 3);
      }
    }
    const int incl = block_inclusive_scan(cnt, s_wave);
    if (r < p.B) {
      if (in_lds) s_start[r] = carry + incl - cnt;
      else p.start[r] = carry + incl - cnt;
    }
    int block_total = 0;
    for (int w = 0; w < kWavesPerBlock; ++w) block_total += s_wave[w];
    carry += block_total;
    __syncthreads();
  }
  const int total = min(carry, p.cap);
  if (tid == 0) {
    if (in_lds) s_start[p.B] = carry;
    p.start[p.B] = carry;
    PlanHeader hd;
    hd.n_items = total;
    hd.indexed = p.meta_ready;
    hd.B = p.B;
    hd.H = p.H;
    hd.bm = p.bm;
    hd.mode = p.mode;
    hd.rows = p.rows;
    hd.magic = kPlanMagic;
    *p.header = hd;
  }
  __syncthreads();

  // 4. write the items: thread t writes one contiguous run of the item list, so no
  //    thread waits on another user's row; within a user, heads outer and query
  //    tiles inner, then the padding tiles to zero
  const int per = (total + kThreads - 1) / kThreads;
  const int i0 = tid * per, i1 = min(i0 + per, total);
  if (i0 >= i1) return;
  auto start_of = [&](int r) { return in_lds ? s_start[r] : p.start[r]; };
  int lo = 0, hi = p.B;   // last sorted user r with start_of(r) <= i0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (start_of(mid) <= i0) lo = mid; else hi = mid;
  }
  int r = lo;
  for (int i = i0; i < i1;) {
    const int s0 = start_of(r), s1 = start_of(r + 1);
    if (i >= s1) { ++r; continue; }
    int b, nqt, nzt;
    if (in_lds) {
      b = s_order[r];
      nqt = s_nqt[b];
      nzt = s_nzt[b];
    } else {
      b = r;
      user_items(p.meta[b], p.H, p.bm, nqt, nzt, p.mode == 3);
    }
    const int n_attn = p.H * nqt;
    int local = i - s0;
    int h = 0, qt = 0;
    if (local < n_attn) { h = local / nqt; qt = local - h * nqt; }
    const int end = min(i1, s1);
    for (; i < end; ++i, ++local) {
      if (local < n_attn) {
        p.items[i] = make_int2(b, (qt << 10) | h);
        if (++qt == nqt) { qt = 0; ++h; }
      } else {
        p.items[i] = make_int2(b, ((local - n_attn) << 10) | kZeroHead);
      }
    }
  }
}

}  // namespace

hipError_t launch_worklist(int mode, const int32_t* offs_a, const int32_t* offs_b, int meta_ready,
                           int B, int H, int bm, int rows, int kv_rows, int cap, UserMeta* meta,
                           int32_t* start, int2* items, PlanHeader* header, hipStream_t s) {
  return launch1(k_worklist, 1, kThreads, s,
                 WorklistParams{mode, offs_a, offs_b, meta_ready, B, H, bm, rows, kv_rows, cap, meta,
                                start, items, header});
}

}  // namespace rr
