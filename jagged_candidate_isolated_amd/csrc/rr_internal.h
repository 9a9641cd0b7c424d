// Internal declarations shared by the librr translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rr.h"

namespace rr {

// Query-row tile heights of the attention kernels.  The work-list and the
// workspace are sized with the smallest one.
constexpr int kBmSimple = 64;      // fp32 (and bf16 d=16) VALU kernel: one wave, one row per lane
constexpr int kBmMfmaNarrow = 128; // bf16 MFMA kernel, short users: four waves of 32 query rows
constexpr int kBmMfmaWide = 256;   // bf16 MFMA kernel, long users: eight waves of 32 query rows
// Average rows per user from which the wide tile is used (compile-time tuning knob).
#ifndef RR_WIDE_MIN_ROWS
#define RR_WIDE_MIN_ROWS 2048
#endif
constexpr int kWideMinRows = RR_WIDE_MIN_ROWS;
constexpr int kBmMin = 64;
constexpr int kHeadSlots = 1024; // work items pack the head into 10 bits ...
constexpr int kZeroHead = 1023;  // ... and head 1023 marks "zero these padding rows"
constexpr int kMaxHeads = 1023;
constexpr int64_t kMaxTiles = int64_t(1) << 21;   // ... and the query tile into the 21 bits above
constexpr int kSortMax = 2048;   // users planned (and sorted) in LDS by the work-list builder
constexpr int kNormRows = 64;    // key rows per entry of the key-norm bounds (k_key_norms)

// What one user contributes to an attention call.  Query and key lists are
// either plain row ranges or, when `idx` is used, ranges of an index array that
// lists the rows (the compacted valid rows of a padded batch).
struct UserMeta {
  int32_t q_begin;   // first entry of the query list
  int32_t n_q;       // query rows
  int32_t kv_begin;  // first entry of the key list
  int32_t n_kv;      // keys every query of the user reads (segment-1 / frozen rows)
  int32_t cand_rel;  // query-list position of the first candidate (self-term from here on)
  int32_t n_pad;     // padding rows (segment 0), listed in idx right after the query list
  int32_t kv_direct; // keys are rows kv_begin + j even in an indexed plan (one contiguous range)
  int32_t spare1;
};
static_assert(sizeof(UserMeta) == 32, "UserMeta is 32 bytes");

// Work item: user b, head h, query tile qt; packed as {b, (qt << 10) | h}.
__host__ __device__ inline int item_head(int2 it) { return it.y & (kHeadSlots - 1); }
__host__ __device__ inline int item_tile(int2 it) { return it.y >> 10; }

// Written by the planning kernels at the start of the workspace; the attention
// kernels check it against their own launch so a plan made for other sizes is
// never used.
struct PlanHeader {
  int32_t n_items;
  int32_t indexed;   // query/key lists go through idx[]
  int32_t B;
  int32_t H;
  int32_t bm;
  int32_t mode;      // 0 full sequence, 1 candidate-only
  int32_t rows;      // T (full) or Tc (candidate-only)
  int32_t magic;
};
constexpr int32_t kPlanMagic = 0x52525031;  // "RRP1"

// Workspace layout (every part 256-byte aligned).
struct WsLayout {
  size_t header;     // PlanHeader
  size_t meta;       // UserMeta[B]
  size_t start;      // int32[B + 1] item starts per sorted user
  size_t idx;        // int32[T] compacted row lists
  size_t items;      // int2[item_bound]
  size_t knorm;      // float[H][knorm_tiles]: per 64 key rows, the largest squared key norm
  size_t total;
  int64_t item_bound;
  int64_t knorm_tiles;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// XCDs of an MI355X and the number of consecutive work items the MFMA kernel keeps
// together on one XCD (for L2 reuse of a user's keys and values).
constexpr int kXcds = 8;
#ifndef RR_XCD_CHUNK
#define RR_XCD_CHUNK 8
#endif
constexpr int kXcdChunk = RR_XCD_CHUNK;
// The forward attention kernel keeps longer runs together: 32 consecutive items (query
// tiles of one user and head) share an XCD, so a long user's keys and values enter
// fewer L2s.
#ifndef RR_ATTN_XCD_CHUNK
#define RR_ATTN_XCD_CHUNK 32
#endif
constexpr int kAttnXcdChunk = RR_ATTN_XCD_CHUNK;
static_assert(kAttnXcdChunk % kXcdChunk == 0, "attention chunks are whole backward chunks");

// Workgroups of an attention launch for tile height bm: one per possible work item,
// rounded up to whole XCD chunks of the forward kernel (whole chunks of the backward too).
inline int64_t attn_grid(int64_t B, int64_t rows, int64_t H, int bm) {
  const int64_t n = (H + 1) * ((rows + bm - 1) / bm + B);
  const int64_t q = int64_t(kXcds) * kAttnXcdChunk;
  return (n + q - 1) / q * q;
}

inline int64_t item_upper_bound(int64_t B, int64_t rows, int64_t H) {
  // sum_b ceil(n_b / BM) <= rows / BM + B for any split of `rows` over B users;
  // H attention items per query tile plus at most one zeroing item per padding tile
  // (>= attn_grid for every tile height, so the items array holds any capped list)
  return attn_grid(B, rows, H, kBmMin);
}

inline WsLayout ws_layout(int64_t B, int64_t T_idx, int64_t q_rows, int64_t H) {
  WsLayout w{};
  size_t off = 0;
  w.header = off; off += 256;
  w.meta = off; off = align256(off + sizeof(UserMeta) * size_t(B));
  w.start = off; off = align256(off + sizeof(int32_t) * size_t(B + 1));
  w.idx = off; off = align256(off + sizeof(int32_t) * size_t(T_idx));
  w.item_bound = item_upper_bound(B, q_rows, H);
  w.items = off; off = align256(off + sizeof(int2) * size_t(w.item_bound));
  w.knorm_tiles = (T_idx + kNormRows - 1) / kNormRows;
  w.knorm = off; off = align256(off + sizeof(float) * size_t(H) * size_t(w.knorm_tiles));
  w.total = off;
  return w;
}

// Arguments of the attention kernels (what every workgroup reads first comes first,
// so that it arrives in one kernel-argument load).
struct AttnArgs {
  const PlanHeader* plan;
  const int2* items;
  const UserMeta* meta;
  int32_t B;
  int32_t H;
  int32_t mode;
  int32_t rows;
  const void* q;       // query rows
  const void* k;       // key rows read by every query of the user
  const void* v;
  const void* k_self;  // own key/value of a candidate, at the query's row
  const void* v_self;
  void* o;
  const int32_t* idx;  // row lists (used when plan->indexed)
  float scale_log2;    // softmax scale * log2(e)
  float* lse;          // [rows][H] natural-log sum of exp(scale q.k) over each row's keys, or NULL
  const int32_t* offsets;     // self-planned launches only: the batch's offsets and cand_start
  const int32_t* cand_start;
  double rope_log2_base;      // != 0: rotate each query row in registers first (log2 of the base);
                              // full sequence without padding: position min(row - start, n_kv),
                              // candidate-only: position n_kv (the frozen history's length)
  const float* knorm;         // full-sequence plans: k_key_norms' bounds for this k,
                              // [H][knorm_tiles]; NULL = none (every key tile forms its maximum)
  int32_t knorm_tiles;
};

// The work item of workgroup slot `item` and its user: false when the plan in the
// workspace does not match this launch or the item is past the list.  The header
// is read as one 32-byte load and the item next to it, and the user's meta as soon
// as the item arrives, all before the test, so that a workgroup waits for two
// memory round trips here rather than one per field.  Both reads stay in bounds
// whatever the workspace holds: item < gridDim.x <= the items array's length for any
// launch the host makes for these sizes, and the user index is clamped into [0, B)
// (B >= 1 whenever a kernel is launched); the values are used only if the test passes.
__device__ __forceinline__ bool fetch_item(const AttnArgs& a, int bm, int item, int2& it,
                                           UserMeta& um, bool& indexed) {
  const PlanHeader p = *a.plan;
  it = a.items[item];
  const int b = min(max(it.x, 0), a.B - 1);
  um = a.meta[b];
  indexed = p.indexed != 0;
  return (p.magic == kPlanMagic) & (p.B == a.B) & (p.H == a.H) & (p.bm == bm) &
         (p.mode == a.mode) & (p.rows == a.rows) & (item < p.n_items) & (b == it.x) &
         (um.n_q >= 0);   // always true for a listed user; keeps the meta load ahead of the test
}

// Segment-ID rule of one row (candidate isolation mask page, segment-ID section).
__device__ __forceinline__ int8_t segment_of(int row, int cand_start, const uint8_t* valid,
                                             int attend_padded_history) {
  const bool is_candidate = row >= cand_start;
  bool ok = valid ? (valid[row] != 0) : true;
  if (attend_padded_history) ok = ok || !is_candidate;
  return ok ? (is_candidate ? int8_t(-1) : int8_t(1)) : int8_t(0);
}

// Rotary encoding (candidate isolation mask page, section on positions shared by
// candidates; the standard pairwise rotation).  The rotary pass and the attention
// kernels that rotate their queries in registers share these, so a query rotated either
// way has the same bits.
// Inverse frequency of feature pair i of d: base^(-2i/d), in double.
__device__ __forceinline__ double rotary_inv_freq(int i, int d, double log2_base) {
  return exp2(-(2.0 * i / d) * log2_base);
}
// Sine and cosine of p * inv_freq.  The angle is formed and reduced in double (positions
// reach 10^4 radians for the low frequencies, where a float angle would be off by about
// 1e-3): a multiple k of pi/2 is taken off, leaving y in [-pi/4, pi/4]; sin y and cos y
// are then the Taylor polynomials through y^9 and y^10 in float (their truncation error
// at pi/4 is below 2e-9, under float precision), and the quadrant k mod 4 picks signs
// and roles.  Short and branch-free, so a kernel that rotates its queries in registers
// keeps its occupancy.
__device__ __forceinline__ void rotary_sincos(int p, double inv_freq, float& c, float& s) {
  const double x = static_cast<double>(p) * inv_freq;
  const double half_pi = 1.5707963267948966192313216916398;
  const double k = rint(x * (1.0 / half_pi));
  const float y = static_cast<float>(fma(-k, half_pi, x));
  const float y2 = y * y;
  // sin y = y (1 - y^2/3! (1 - y^2/(4*5) (1 - y^2/(6*7) (1 - y^2/(8*9)))))
  float ps = fmaf(-y2, 1.0f / 72.0f, 1.0f);
  ps = fmaf(-y2 * (1.0f / 42.0f), ps, 1.0f);
  ps = fmaf(-y2 * (1.0f / 20.0f), ps, 1.0f);
  ps = fmaf(-y2 * (1.0f / 6.0f), ps, 1.0f);
  const float sy = y * ps;
  // cos y = 1 - y^2/2! (1 - y^2/(3*4) (1 - y^2/(5*6) (1 - y^2/(7*8) (1 - y^2/(9*10)))))
  float pc = fmaf(-y2, 1.0f / 90.0f, 1.0f);
  pc = fmaf(-y2 * (1.0f / 56.0f), pc, 1.0f);
  pc = fmaf(-y2 * (1.0f / 30.0f), pc, 1.0f);
  pc = fmaf(-y2 * (1.0f / 12.0f), pc, 1.0f);
  const float cy = fmaf(-y2 * 0.5f, pc, 1.0f);
  const int q = static_cast<int>(static_cast<long long>(k) & 3);
  const float ss = (q & 1) ? cy : sy, cc = (q & 1) ? sy : cy;
  s = (q & 2) ? -ss : ss;
  c = ((q + 1) & 2) ? -cc : cc;
}
// one feature pair (x0, x1) turned by the angle whose cosine and sine are c, s
__device__ __forceinline__ void rotate_pair(float x0, float x1, float c, float s, float& y0, float& y1) {
  y0 = fmaf(x0, c, -x1 * s);
  y1 = fmaf(x0, s, x1 * c);
}

constexpr int kBuckets = 128;      // logarithmic key-count buckets of the work list's sort

// Bucket of a key count, longest first: bucket 0 holds the largest counts and the
// last bucket the users without keys.  Four buckets per octave.
__device__ __forceinline__ int cost_bucket(int cost) {
  if (cost <= 0) return kBuckets - 1;
  const int lg = 31 - __clz(cost);                                   // 0..30
  const int frac = lg >= 2 ? (cost >> (lg - 2)) & 3 : (cost << (2 - lg)) & 3;
  return kBuckets - 2 - min(lg * 4 + frac, kBuckets - 2);            // 0..126
}

// Self-planned launches.  A small unpadded full-sequence batch (at most kSelfPlanUsers
// users and a grid of at most kSelfPlanGrid workgroups) skips the separate planning
// kernel: every workgroup rebuilds the work list in LDS from offsets and cand_start
// and takes its own item.  The list is the planning kernel's (users by descending
// key-count bucket, heads outer and query tiles inner within a user) with ties broken
// by user index, so every workgroup builds the same one.  Worth it only when there are
// about as many items as workgroup slots: then the planning launch is a large part of
// the batch's latency, while each workgroup's own planning costs a few microseconds
// once rather than once per round of items.
constexpr int kSelfPlanUsers = 256;
constexpr int kSelfPlanGrid = 1024;

struct SelfPlanLds {
  int32_t lo[kSelfPlanUsers];
  int32_t nq[kSelfPlanUsers];
  int32_t nkv[kSelfPlanUsers];
  int32_t order[kSelfPlanUsers];
  int32_t start[kSelfPlanUsers + 1];
  int32_t hist[kBuckets];
  int32_t wave[16];
  uint32_t bkt[kSelfPlanUsers / 4];   // one byte per user
};

// A self-planned launch on the narrow tile is about one or two rounds of items with two or
// more workgroups resident per CU.  The first 256 workgroups take the 256 CUs one each (the
// dispatcher places workgroups in index order, breadth first, as the timing below bears
// out), so the next ones are the CUs' second.  Items 256 onward (up to 512) go in reverse:
// the CU with the k-th longest item gets one of the shortest as its second, the classic
// pairing for two jobs a machine on top of longest-first order (short-history batch:
// kernel 21.5 -> 20.9 us).  A bijection on the items, so every item is still computed once
// and no output depends on which workgroup does it.  The wide tile (one workgroup per CU,
// the second round handed out as CUs free up) keeps plain longest-first order.
constexpr int kCUs = 256;
__device__ __forceinline__ int second_pass_reversed(int item, int total, int bm) {
  const int end = min(total, 2 * kCUs);
  return (bm == kBmMfmaNarrow && item >= kCUs && item < end) ? kCUs + (end - 1 - item) : item;
}

// Item `item` of the batch (offsets, cand_start: B users over `rows` rows, H heads,
// bm-row query tiles) into it / um; false past the last item.  blockDim.x >= B.
__device__ __forceinline__ bool self_plan_item(const int32_t* offsets, const int32_t* cand_start, int B, int H,
                                               int bm, int rows, int item, SelfPlanLds& s, int2& it,
                                               UserMeta& um) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  for (int i = tid; i < kBuckets; i += blockDim.x) s.hist[i] = 0;
  for (int i = tid; i < kSelfPlanUsers / 4; i += blockDim.x) s.bkt[i] = 0;
  __syncthreads();
  int bkt = kBuckets - 1;
  if (tid < B) {   // row ranges clamped into [0, rows), as the planning kernel does
    const int lo = min(max(offsets[tid], 0), rows);
    const int hi = min(max(offsets[tid + 1], lo), rows);
    const int cs = min(max(cand_start[tid], lo), hi);
    s.lo[tid] = lo;
    s.nq[tid] = hi - lo;
    s.nkv[tid] = cs - lo;
    bkt = cost_bucket(cs - lo);
    atomicOr(&s.bkt[tid >> 2], static_cast<uint32_t>(bkt) << (8 * (tid & 3)));
    atomicAdd(&s.hist[bkt], 1);
  }
  __syncthreads();
  if (tid < 64) {   // exclusive offsets of the 128 buckets
    const int a = s.hist[2 * tid], c = s.hist[2 * tid + 1];
    int x = a + c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (tid >= off) x += y;
    }
    s.hist[2 * tid] = x - a - c;
    s.hist[2 * tid + 1] = x - c;
  }
  __syncthreads();
  if (tid < B) {   // stable rank: users before this one in its bucket, four bytes a read
    int rank = s.hist[bkt];
    const uint32_t pat = 0x01010101u * static_cast<uint32_t>(bkt);
    for (int w = 0; w < (tid >> 2); ++w) {
      const uint32_t x = s.bkt[w] ^ pat;   // zero bytes = same bucket
      rank += __popc(~(((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x | 0x7f7f7f7fu));
    }
    for (int j = tid & ~3; j < tid; ++j) rank += ((s.bkt[j >> 2] >> (8 * (j & 3))) & 0xff) == static_cast<uint32_t>(bkt);
    s.order[rank] = tid;
  }
  __syncthreads();
  // exclusive scan of the item counts in that order (B <= blockDim.x: one pass)
  int c = 0;
  if (tid < B) {
    const int u = s.order[tid];
    c = H * ((s.nq[u] + bm - 1) / bm);
  }
  int x = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s.wave[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s.wave[w];
  if (tid < B) s.start[tid] = before + x - c;
  if (tid == 0) {
    int total = 0;
    for (int w = 0; w < nw; ++w) total += s.wave[w];
    s.start[B] = total;
  }
  __syncthreads();
  if (item >= s.start[B]) return false;
  item = second_pass_reversed(item, s.start[B], bm);
  int lo = 0, hi = B;   // last r with start[r] <= item
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s.start[mid] <= item) lo = mid; else hi = mid;
  }
  const int u = s.order[lo];
  const int nqt = (s.nq[u] + bm - 1) / bm, local = item - s.start[lo];
  it = make_int2(u, ((local % nqt) << 10) | (local / nqt));
  um = UserMeta{};
  um.q_begin = s.lo[u];
  um.n_q = s.nq[u];
  um.kv_begin = s.lo[u];
  um.n_kv = s.nkv[u];
  um.cand_rel = s.nkv[u];
  um.kv_direct = 1;
  return true;
}

// self_plan_item for a batch of at most 64 users, by every wave on its own (no LDS, no
// barrier): lane u holds user u's counts; a user's place in the list (descending
// key-count bucket, ties by user index: self_plan_item's order) and its first item, the
// item count of the users before it, come from one pass over the 64 lanes.
__device__ __forceinline__ bool self_plan_item_wave(const int32_t* offsets, const int32_t* cand_start, int B, int H,
                                                    int bm, int rows, int item, int2& it, UserMeta& um) {
  const int lane = threadIdx.x & 63;
  int lo = 0, nq = 0, nkv = 0, key = (kBuckets << 6) | lane;   // past every user of the batch
  if (lane < B) {   // row ranges clamped into [0, rows), as the planning kernel does
    lo = min(max(offsets[lane], 0), rows);
    const int hi = min(max(offsets[lane + 1], lo), rows);
    const int cs = min(max(cand_start[lane], lo), hi);
    nq = hi - lo;
    nkv = cs - lo;
    key = (cost_bucket(nkv) << 6) | lane;
  }
  const int cnt = H * ((nq + bm - 1) / bm);
  int first = 0, total = 0;
#pragma unroll 8
  for (int v = 0; v < 64; ++v) {
    const int kv = __builtin_amdgcn_readlane(key, v), cv = __builtin_amdgcn_readlane(cnt, v);
    first += kv < key ? cv : 0;
    total += cv;
  }
  if (item >= total) return false;
  item = second_pass_reversed(item, total, bm);
  const uint64_t own = __ballot(cnt > 0 && first <= item && item < first + cnt);   // one lane
  const int u = __ffsll(static_cast<long long>(own)) - 1;
  const int nq_u = __builtin_amdgcn_readlane(nq, u), nkv_u = __builtin_amdgcn_readlane(nkv, u);
  const int nqt = (nq_u + bm - 1) / bm, local = item - __builtin_amdgcn_readlane(first, u);
  it = make_int2(u, ((local % nqt) << 10) | (local / nqt));
  um = UserMeta{};
  um.q_begin = __builtin_amdgcn_readlane(lo, u);
  um.n_q = nq_u;
  um.kv_begin = um.q_begin;
  um.n_kv = nkv_u;
  um.cand_rel = nkv_u;
  um.kv_direct = 1;
  return true;
}

// Launch a kernel that takes one parameter struct; returns the launch status
// (hipLaunchKernel reports it directly, so no sticky last-error is read or cleared).
template <typename P>
inline hipError_t launch1(void (*k)(P), int64_t grid, int block, hipStream_t s, P params) {
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {&params};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), dim3(static_cast<unsigned>(grid)),
                         dim3(block), args, 0, s);
}

// Launchers (each returns hipSuccess or the launch error).
hipError_t launch_segment_ids(const int32_t* offsets, const int32_t* cand_start, const uint8_t* valid,
                              int flag, int B, int T, int8_t* seg, hipStream_t s);
hipError_t launch_bounds(const int32_t* offsets, const int8_t* seg, int B, int T, int32_t* out,
                         hipStream_t s);
hipError_t launch_validate(const int32_t* offsets, const int32_t* cand_start, int B, int T,
                           int32_t* err, hipStream_t s);
hipError_t launch_compact(const int32_t* offsets, const int32_t* cand_start, const uint8_t* valid,
                          int flag, int B, int T, UserMeta* meta, int32_t* idx, hipStream_t s);
// mode 0: full sequence from offsets/cand_start (meta_ready: meta already written by compact)
// mode 1: candidate-only from hist_offsets/cand_offsets
hipError_t launch_worklist(int mode, const int32_t* offs_a, const int32_t* offs_b, int meta_ready,
                           int B, int H, int bm, int rows, int kv_rows, int cap, UserMeta* meta,
                           int32_t* start, int2* items, PlanHeader* header, hipStream_t s);
hipError_t launch_attn_simple(const AttnArgs& a, int d, int dtype, int64_t grid, hipStream_t s);
// a.knorm[h][t] = the largest squared norm, in head h, of the rows among rows [64 t, 64 t + 64)
// of a.k that lie in some user's key span (from its first to its last key row), for a
// full-sequence plan (other rows count 0); `rows` = the K rows, d = head width
hipError_t launch_key_norms(const AttnArgs& a, int rows, int d, hipStream_t s);
hipError_t launch_attn_mfma(const AttnArgs& a, int d, int bm, int64_t grid, hipStream_t s);
hipError_t launch_attn_mfma_self_planned(const AttnArgs& a, int d, int bm, int64_t grid, hipStream_t s);
// the backward: k_bwd_dq over plan aq (tiles of bm_q query rows), k_bwd_dkdv over plan ak
// (its items read as key tiles; the same plan in full mode, a key-major one in a
// candidate-only layer)
hipError_t launch_attn_bwd(const AttnArgs& aq, int bm_q, int64_t grid_q, const AttnArgs& ak, int bm_k,
                           int64_t grid_k, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           void* dk_self, void* dv_self, float* delta, float scale, int d, hipStream_t s);
hipError_t launch_rope_positions(const int32_t* offsets, const int32_t* cand_start,
                                 const int32_t* pos_base, int B, int T, int32_t* pos, hipStream_t s);
hipError_t launch_rope_qk(const void* q, const void* k, void* qo, void* ko, const int32_t* offsets,
                          const int32_t* cand_start, const int32_t* pos_base, int B, int T, int H,
                          int d, int dtype, double log2_base, hipStream_t s);
// launch_rope_qk that also writes the rows before each user's candidate start into the
// compact history blocks kc (rotated k) and vc (a copy of v), row hoff[b] + r - offsets[b]
hipError_t launch_rope_qk_cache(const void* q, const void* k, void* qo, void* ko, const int32_t* offsets,
                                const int32_t* cand_start, const int32_t* pos_base, int B, int T, int H, int d,
                                int dtype, double log2_base, void* kc, const void* v, void* vc,
                                const int32_t* hoff, int Th, hipStream_t s);

// Zero the output rows of a padding tile: rows idx[q_begin + n_q + qt*bm ...], every head
// (and set their log-sum-exp to -inf when the forward writes it).
// `nthreads` threads of the workgroup cooperate; rows are `row_bytes` long (a multiple of 16).
__device__ __forceinline__ void zero_padding_tile(const AttnArgs& a, const UserMeta& um, int qt,
                                                  int bm, int row_bytes, int tid, int nthreads) {
  const int first = qt * bm;
  const int nrows = min(bm, um.n_pad - first);   // padding rows follow the query list in idx
  const int chunks = row_bytes / 16;
  uint4* o = static_cast<uint4*>(a.o);
  for (int e = tid; e < nrows * chunks; e += nthreads) {
    const int r = a.idx[um.q_begin + um.n_q + first + e / chunks];
    o[static_cast<int64_t>(r) * chunks + (e % chunks)] = make_uint4(0, 0, 0, 0);
  }
  if (a.lse)   // a padding row admits no key: its log-sum-exp is -inf in every head
    for (int e = tid; e < nrows * a.H; e += nthreads) {
      const int r = a.idx[um.q_begin + um.n_q + first + e / a.H];
      a.lse[static_cast<int64_t>(r) * a.H + (e % a.H)] = -INFINITY;
    }
}

}  // namespace rr
