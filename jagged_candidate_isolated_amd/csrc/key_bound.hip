// Key-norm bounds for the attention kernel's softmax.
//
// The bf16 attention kernel keeps a per-row reference for its exponentials and, for every
// key tile, forms the tile's row maximum to decide whether the reference must move up
// (it moves only when the maximum exceeds it by more than 2^8, in log2 units).  By the
// Cauchy-Schwarz inequality a score q.k never exceeds |q| |k|, so once a row's
// reference is within 2^8 of |q| times the largest norm among its user's keys, no later
// tile can move it, and the kernel can skip forming the maximum: the same decision, hence
// the same bits, without the maximum's instructions in the chain between the score
// product and the exponentials.
//
// This pass supplies the key side of that bound: for every 64 rows of k and every head,
// the largest squared norm among the rows in some user's key span.  A user's rows start at
// its query-list start in either kind of full-sequence plan, so the last user whose list
// starts at or before a row owns it; the row counts when it lies between that user's first
// and last key rows (its key range, or for a padded batch the first and last rows of its
// listed keys: any padding between them only loosens the bound).  Candidate rows are
// skipped (no query reads them through the key loop), so the pass reads about the key
// rows' bytes once.
#include "rr_internal.h"

namespace rr {
namespace {

constexpr int kNormThreads = 256;
constexpr int kNormUnroll = 8;   // 16-byte loads in flight per thread
constexpr int kNormGrid = 2048;  // workgroups of a launch (about one round on the chip)

struct KeyNormArgs {
  AttnArgs a;   // the plan (header, meta), k, B, H, rows
  float* out;   // [H][a.knorm_tiles]
};

template <int D>
__global__ __launch_bounds__(kNormThreads) void k_key_norms(KeyNormArgs ka) {
  const AttnArgs& a = ka.a;
  constexpr int CH = D / 8;   // 16-byte chunks per row and head
  __shared__ unsigned s_max[kMaxHeads];
  __shared__ unsigned long long s_keys;
  const int tid = threadIdx.x, lane = tid & 63;
  const PlanHeader p = *a.plan;
  // only a full-sequence plan for this launch has the bounds used
  if (!((p.magic == kPlanMagic) & (p.B == a.B) & (p.H == a.H) & (p.mode == 0) & (p.rows == a.rows))) return;
  const bool listed = p.indexed != 0;
  const int n_tiles = (a.rows + kNormRows - 1) / kNormRows;
  const int per_row = a.H * CH;
  const int n = kNormRows * per_row;   // chunks per tile
  // grid-stride over the tiles of 64 rows: a launch of about one round of workgroups
  for (int rt = blockIdx.x; rt < n_tiles; rt += gridDim.x) {
    const int r0 = rt * kNormRows;
    for (int h = tid; h < a.H; h += kNormThreads) s_max[h] = 0u;
    if (tid < 64) {
      const int r = r0 + lane;
      bool key = false;
      if (r < a.rows) {
        int lo = 0, hi = a.B - 1;   // the last user whose rows start at or before r
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (a.meta[mid].q_begin <= r) lo = mid;
          else hi = mid - 1;
        }
        const UserMeta m = a.meta[lo];
        if (m.n_kv > 0) {
          const bool direct = !listed || m.kv_direct;
          const int first = direct ? m.kv_begin : a.idx[m.kv_begin];
          const int last = direct ? m.kv_begin + m.n_kv - 1 : a.idx[m.kv_begin + m.n_kv - 1];
          key = r >= first && r <= last;
        }
      }
      const unsigned long long keys = __ballot(key);
      if (lane == 0) s_keys = keys;
    }
    __syncthreads();
    const unsigned long long keys = s_keys;
    if (keys != 0) {
      // chunk c of the tile: row c / (H * CH), head (c / CH) % H, 8 features from (c % CH) * 8;
      // consecutive threads read consecutive 16 bytes
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + int64_t(r0) * a.H * D);
      for (int c0 = 0; c0 < n; c0 += kNormThreads * kNormUnroll) {
        uint4 w[kNormUnroll];
        bool live[kNormUnroll];
#pragma unroll
        for (int u = 0; u < kNormUnroll; ++u) {
          const int c = c0 + u * kNormThreads + tid;
          const int row = min(c / per_row, kNormRows - 1);
          live[u] = c < n && ((keys >> row) & 1ull);
          w[u] = live[u] ? src[c] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kNormUnroll; ++u) {
          const unsigned x[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
          float ss = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float lo = __uint_as_float(x[j] << 16), hi = __uint_as_float(x[j] & 0xffff0000u);
            ss = fmaf(lo, lo, ss);
            ss = fmaf(hi, hi, ss);
          }
          // the CH threads of one (row, head) are consecutive lanes starting at a multiple of CH
#pragma unroll
          for (int off = CH / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
          const int c = c0 + u * kNormThreads + tid;
          if (live[u] && (c % CH) == 0) atomicMax(&s_max[(c / CH) % a.H], __float_as_uint(ss));
        }
      }
    }
    __syncthreads();
    // squared norms are >= 0, so their bit patterns order as the values do (NaN above +inf)
    for (int h = tid; h < a.H; h += kNormThreads)
      ka.out[int64_t(h) * a.knorm_tiles + rt] = __uint_as_float(s_max[h]);
    __syncthreads();   // s_max and s_keys are reused by the next tile
  }
}

}  // namespace

hipError_t launch_key_norms(const AttnArgs& a, int rows, int d, hipStream_t s) {
  const int64_t tiles = (int64_t(rows) + kNormRows - 1) / kNormRows;
  if (a.B <= 0 || a.H <= 0 || !a.knorm || tiles > a.knorm_tiles || rows != a.rows) return hipErrorInvalidValue;
  const int64_t grid = tiles < kNormGrid ? tiles : kNormGrid;
  // the bounds area is the caller's workspace, written here and read by the attention launch
  const KeyNormArgs ka{a, const_cast<float*>(a.knorm)};
  switch (d) {
    case 32: return launch1(k_key_norms<32>, grid, kNormThreads, s, ka);
    case 64: return launch1(k_key_norms<64>, grid, kNormThreads, s, ka);
    case 128: return launch1(k_key_norms<128>, grid, kNormThreads, s, ka);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rr
