// Length-sorted work list for ragged users.
//
// One workgroup builds, entirely on the device (the host never waits for the
// lengths), the list of attention work items: user b, head h, query tile qt.
// Users are ordered by the number of keys their queries read, longest first
// (longest-processing-time order), so the GPU's in-order workgroup dispatch
// starts the expensive items first and the short ones fill the tail.  Ties keep
// the user order.  Within a user the items go head by head, query tile by query
// tile, so neighbouring items read the same keys and values.
//
// Prior art: the CTI inference notes (varlen flash-attention section) build a
// block-to-sequence map on the device with a shape-derived grid upper bound and
// no host synchronisation; the grid of the attention kernels here follows the
// same idea (surplus workgroups exit at once).
#include "rr_internal.h"

namespace rr {
namespace {

constexpr int kThreads = 1024;

struct WorklistParams {
  int mode;              // 0: full sequence (offs_a = offsets, offs_b = cand_start)
                         // 1: candidate-only (offs_a = hist_offsets, offs_b = cand_offsets)
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

// Items of one user: H per query tile, plus one per tile of padding rows to zero.
__device__ __forceinline__ int user_items(const UserMeta& m, int H, int bm, int& nqt, int& nzt) {
  nqt = (max(m.n_q, 0) + bm - 1) / bm;
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
    m.cand_rel = 0;
  }
  return m;
}

__global__ __launch_bounds__(kThreads) void k_worklist(WorklistParams p) {
  __shared__ unsigned long long s_key[kSortMax];
  __shared__ int s_scan[kThreads];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  const bool sorted = p.B <= kSortMax;

  if (!p.meta_ready) {
    for (int b = tid; b < p.B; b += kThreads) p.meta[b] = plain_meta(p, b);
    __syncthreads();  // the meta writes are visible to the whole workgroup after the barrier
  }

  // 1. order users by key count, descending (bitonic sort of (cost, user) keys)
  int n = 1;
  if (sorted) {
    while (n < p.B) n <<= 1;
    for (int i = tid; i < n; i += kThreads) {
      unsigned long long key = ~0ull;
      if (i < p.B) {
        const int cost = max(p.meta[i].n_kv, 0);
        key = (static_cast<unsigned long long>(0x7fffffffu - static_cast<unsigned>(cost)) << 32) |
              static_cast<unsigned>(i);
      }
      s_key[i] = key;
    }
    __syncthreads();
    for (int k = 2; k <= n; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n; i += kThreads) {
          const int l = i ^ j;
          if (l > i) {
            const unsigned long long a = s_key[i], c = s_key[l];
            const bool up = (i & k) == 0;
            if ((a > c) == up) { s_key[i] = c; s_key[l] = a; }
          }
        }
        __syncthreads();
      }
    }
  }

  // 2. exclusive scan of the item counts in that order
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < p.B; base += kThreads) {
    const int r = base + tid;
    int cnt = 0;
    if (r < p.B) {
      const int b = sorted ? static_cast<int>(s_key[r] & 0xffffffffu) : r;
      int nqt, nzt;
      cnt = user_items(p.meta[b], p.H, p.bm, nqt, nzt);
    }
    s_scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int add = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    const int carry = s_carry;
    if (r < p.B) p.start[r] = carry + s_scan[tid] - cnt;
    __syncthreads();
    if (tid == kThreads - 1) s_carry = carry + s_scan[tid];
    __syncthreads();
  }
  const int total = min(s_carry, p.cap);
  if (tid == 0) {
    p.start[p.B] = total;
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

  // 3. write the items: one wave per user
  const int wave = tid >> 6, lane = tid & 63;
  for (int r = wave; r < p.B; r += kThreads / 64) {
    const int b = sorted ? static_cast<int>(s_key[r] & 0xffffffffu) : r;
    int nqt, nzt;
    const int cnt = user_items(p.meta[b], p.H, p.bm, nqt, nzt);
    const int n_attn = p.H * nqt;
    const int s0 = p.start[r];
    for (int i = lane; i < cnt && s0 + i < total; i += 64) {
      int h, qt;
      if (i < n_attn) {
        h = i / nqt;
        qt = i - h * nqt;
      } else {
        h = kZeroHead;
        qt = i - n_attn;
      }
      p.items[s0 + i] = make_int2(b, (qt << 10) | h);
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
