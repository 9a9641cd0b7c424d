// Right-anchored rotary positions and the rotary encoding of q and k, in one pass.
//
// Candidate isolation attention mask page, section "位置编码：候选共用一个位置": the
// newest history row of every user sits at history_end - 1 and every candidate at
// history_end, so the encoding cannot tell candidates apart.  Rows are numbered within
// the user's row and history_end is the candidate start (plus an optional per-user
// base, which places the candidate rows of a candidate-only layer after their frozen
// history).  The rotation is the standard pairwise one: features (2i, 2i+1) turn by
// pos * base^(-2i/d).
//
// One thread per (row, group of four feature pairs): it finds the row's user by
// binary search over the offsets and takes each pair's angle in double precision
// (positions reach 10^4 radians for the low frequencies, where a float angle would be
// off by about 1e-3), reduces it modulo 2 pi in double, then takes the sine and cosine
// of the reduced angle in float.  It then rotates those four pairs in every head of q
// and of k with 16-byte loads and stores (32-byte for fp32), all heads' loads issued
// before their rotations.  Consecutive threads take consecutive groups of one row, so
// each head's row segment moves as one contiguous run.  HBM-bound: q and k are read
// once and written once.  Head dimensions not a multiple of 8 take one pair per thread.
#include "rr_internal.h"

namespace rr {
namespace {

struct RopeArgs {
  const void* q;
  const void* k;
  void* qo;
  void* ko;
  const int32_t* offsets;
  const int32_t* cand_start;
  const int32_t* pos_base;
  int32_t B;
  int32_t T;
  int32_t H;
  int32_t d;
  double log2_base;
  // optional: rows before their user's candidate start also go, k rotated, to the
  // compact history blocks kc / vc (row hoff[b] + r - offsets[b] < Th); v is copied
  void* kc;
  const void* v;
  void* vc;
  const int32_t* hoff;
  int32_t Th;
};

// The user owning row r: the last b in [0, B) with offsets[b] <= r (0 if none).
__device__ __forceinline__ int user_of(const int32_t* offsets, int B, int r) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int position_of(const RopeArgs& a, int r) {
  const int b = user_of(a.offsets, a.B, r);
  const int off = a.offsets[b];
  return (a.pos_base ? a.pos_base[b] : 0) + min(r - off, a.cand_start[b] - off);
}

__global__ __launch_bounds__(256) void k_rope_positions(RopeArgs a, int32_t* pos) {
  for (int64_t r = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; r < a.T;
       r += int64_t(gridDim.x) * blockDim.x)
    pos[r] = position_of(a, static_cast<int>(r));
}

// 8 consecutive elements (4 pairs) as float
__device__ __forceinline__ void load8(const float* p, float* x) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void store8(float* p, const float* y) {
  reinterpret_cast<float4*>(p)[0] = make_float4(y[0], y[1], y[2], y[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(y[4], y[5], y[6], y[7]);
}
__device__ __forceinline__ void load8(const __bf16* p, float* x) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  const unsigned u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(u[j] << 16);
    x[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ void store8(__bf16* p, const float* y) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  unsigned u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x2 v = {static_cast<__bf16>(y[2 * j]), static_cast<__bf16>(y[2 * j + 1])};   // RNE
    u[j] = __builtin_bit_cast(unsigned, v);
  }
  *reinterpret_cast<uint4*>(p) = make_uint4(u[0], u[1], u[2], u[3]);
}
__device__ __forceinline__ void load2(const float* p, float* x) {
  const float2 a = *reinterpret_cast<const float2*>(p);
  x[0] = a.x; x[1] = a.y;
}
__device__ __forceinline__ void store2(float* p, const float* y) {
  *reinterpret_cast<float2*>(p) = make_float2(y[0], y[1]);
}
__device__ __forceinline__ void load2(const __bf16* p, float* x) {
  const unsigned w = *reinterpret_cast<const unsigned*>(p);
  x[0] = __uint_as_float(w << 16); x[1] = __uint_as_float(w & 0xffff0000u);
}
__device__ __forceinline__ void store2(__bf16* p, const float* y) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {static_cast<__bf16>(y[0]), static_cast<__bf16>(y[1])};
  *reinterpret_cast<unsigned*>(p) = __builtin_bit_cast(unsigned, v);
}

// rotate NP pairs (2 NP elements at `first`) of every head of x into y (and into y2 at
// `first2` when y2 is given)
template <int NP, typename T>
__device__ __forceinline__ void rotate_heads(const T* x, T* y, int64_t first, int H, int d,
                                             const float* c, const float* s, T* y2 = nullptr,
                                             int64_t first2 = 0) {
  constexpr int HU = 4;   // heads in flight
  for (int h0 = 0; h0 < H; h0 += HU) {
    float v[HU][2 * NP];
#pragma unroll
    for (int u = 0; u < HU; ++u)
      if (h0 + u < H) {
        if constexpr (NP == 4) load8(x + first + static_cast<int64_t>(h0 + u) * d, v[u]);
        else load2(x + first + static_cast<int64_t>(h0 + u) * d, v[u]);
      }
#pragma unroll
    for (int u = 0; u < HU; ++u)
      if (h0 + u < H) {
        float w[2 * NP];
#pragma unroll
        for (int j = 0; j < NP; ++j) rotate_pair(v[u][2 * j], v[u][2 * j + 1], c[j], s[j], w[2 * j], w[2 * j + 1]);
        if constexpr (NP == 4) store8(y + first + static_cast<int64_t>(h0 + u) * d, w);
        else store2(y + first + static_cast<int64_t>(h0 + u) * d, w);
        if (y2) {
          if constexpr (NP == 4) store8(y2 + first2 + static_cast<int64_t>(h0 + u) * d, w);
          else store2(y2 + first2 + static_cast<int64_t>(h0 + u) * d, w);
        }
      }
  }
}

// copy NP pairs of every head of row `first` of x to y at `first2`
template <int NP, typename T>
__device__ __forceinline__ void copy_heads(const T* x, T* y, int64_t first, int64_t first2, int H, int d) {
  for (int h = 0; h < H; ++h) {
    const int64_t o = static_cast<int64_t>(h) * d;
    if constexpr (NP == 4 && sizeof(T) == 2) {
      *reinterpret_cast<uint4*>(y + first2 + o) = *reinterpret_cast<const uint4*>(x + first + o);
    } else {
#pragma unroll
      for (int j = 0; j < 2 * NP; ++j) y[first2 + o + j] = x[first + o + j];
    }
  }
}

// NP = 4: one thread per 4 consecutive pairs (d % 8 == 0); NP = 1 otherwise.  CACHE: also
// fill the compact history blocks (a.kc, a.vc).
constexpr int kRopeLdsUsers = 1024;   // batches up to this many users search their offsets in LDS
constexpr int kRopeMaxD = 256;        // the largest head width the rotary pass takes

template <typename T, int NP, bool CACHE>
__global__ __launch_bounds__(256) void k_rope_qk(RopeArgs a) {
  // the batch's offsets, candidate starts and position bases in LDS (one read per workgroup)
  // so that each row's user is found without a chain of dependent global reads
  __shared__ int32_t s_off[kRopeLdsUsers + 1], s_cs[kRopeLdsUsers], s_pb[kRopeLdsUsers];
  __shared__ double s_inv[kRopeMaxD / 2];   // the pairs' inverse frequencies, once per workgroup
  const bool in_lds = a.B <= kRopeLdsUsers;
  if (in_lds) {
    for (int i = threadIdx.x; i <= a.B; i += blockDim.x) {
      s_off[i] = a.offsets[i];
      if (i < a.B) {
        s_cs[i] = a.cand_start[i];
        s_pb[i] = a.pos_base ? a.pos_base[i] : 0;
      }
    }
  }
  for (int i = threadIdx.x; i < a.d / 2; i += blockDim.x) s_inv[i] = rotary_inv_freq(i, a.d, a.log2_base);
  __syncthreads();
  const int groups = a.d / (2 * NP);
  const int64_t n = static_cast<int64_t>(a.T) * groups;
  for (int64_t g = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; g < n;
       g += int64_t(gridDim.x) * blockDim.x) {
    const int r = static_cast<int>(g / groups), i0 = static_cast<int>(g % groups) * NP;
    int b, off, cs, pb;
    if (in_lds) {
      int lo = 0, hi = a.B;   // the last b with offsets[b] <= r
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= r) lo = mid;
        else hi = mid;
      }
      b = lo; off = s_off[b]; cs = s_cs[b]; pb = s_pb[b];
    } else {
      b = user_of(a.offsets, a.B, r);
      off = a.offsets[b]; cs = a.cand_start[b]; pb = a.pos_base ? a.pos_base[b] : 0;
    }
    const int p = pb + min(r - off, cs - off);
    float c[NP], s[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j)
      rotary_sincos(p, s_inv[i0 + j], c[j], s[j]);
    const int64_t first = static_cast<int64_t>(r) * a.H * a.d + 2 * i0;
    if (a.q) rotate_heads<NP>(static_cast<const T*>(a.q), static_cast<T*>(a.qo), first, a.H, a.d, c, s);
    if constexpr (CACHE) {
      // a history row's place in the compact history blocks
      int64_t hrow = -1;
      if (r < cs) {
        hrow = static_cast<int64_t>(a.hoff[b]) + r - off;
        if (hrow >= a.Th) hrow = -1;
      }
      const int64_t first2 = hrow * a.H * a.d + 2 * i0;
      if (a.k)
        rotate_heads<NP>(static_cast<const T*>(a.k), static_cast<T*>(a.ko), first, a.H, a.d, c, s,
                         hrow >= 0 && a.kc ? static_cast<T*>(a.kc) : nullptr, first2);
      if (a.vc && hrow >= 0)
        copy_heads<NP>(static_cast<const T*>(a.v), static_cast<T*>(a.vc), first, first2, a.H, a.d);
    } else if (a.k) {
      rotate_heads<NP>(static_cast<const T*>(a.k), static_cast<T*>(a.ko), first, a.H, a.d, c, s);
    }
  }
}

int64_t grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return g < 1 ? 1 : (g > (int64_t(1) << 20) ? (int64_t(1) << 20) : g);
}

RopeArgs rope_args(const int32_t* offsets, const int32_t* cand_start, const int32_t* pos_base, int B,
                   int T) {
  RopeArgs a{};
  a.offsets = offsets;
  a.cand_start = cand_start;
  a.pos_base = pos_base;
  a.B = B;
  a.T = T;
  return a;
}

}  // namespace

hipError_t launch_rope_positions(const int32_t* offsets, const int32_t* cand_start,
                                 const int32_t* pos_base, int B, int T, int32_t* pos, hipStream_t s) {
  const RopeArgs a = rope_args(offsets, cand_start, pos_base, B, T);
  const int64_t grid = grid_for(T);
  void* args[] = {const_cast<RopeArgs*>(&a), &pos};
  return hipLaunchKernel(reinterpret_cast<const void*>(k_rope_positions), dim3(static_cast<unsigned>(grid)),
                         dim3(256), args, 0, s);
}

hipError_t launch_rope_qk(const void* q, const void* k, void* qo, void* ko, const int32_t* offsets,
                          const int32_t* cand_start, const int32_t* pos_base, int B, int T, int H,
                          int d, int dtype, double log2_base, hipStream_t s) {
  return launch_rope_qk_cache(q, k, qo, ko, offsets, cand_start, pos_base, B, T, H, d, dtype, log2_base, nullptr,
                              nullptr, nullptr, nullptr, 0, s);
}

hipError_t launch_rope_qk_cache(const void* q, const void* k, void* qo, void* ko, const int32_t* offsets,
                                const int32_t* cand_start, const int32_t* pos_base, int B, int T, int H, int d,
                                int dtype, double log2_base, void* kc, const void* v, void* vc,
                                const int32_t* hoff, int Th, hipStream_t s) {
  RopeArgs a = rope_args(offsets, cand_start, pos_base, B, T);
  a.q = q; a.k = k; a.qo = qo; a.ko = ko;
  a.H = H; a.d = d; a.log2_base = log2_base;
  a.kc = kc; a.v = v; a.vc = vc; a.hoff = hoff; a.Th = Th;
  const bool cache = (kc || vc) && hoff;
  if (d % 8 == 0) {
    const int64_t grid = grid_for(static_cast<int64_t>(T) * (d / 8));
    if (cache)
      return dtype == RR_BF16 ? launch1(k_rope_qk<__bf16, 4, true>, grid, 256, s, a)
                              : launch1(k_rope_qk<float, 4, true>, grid, 256, s, a);
    return dtype == RR_BF16 ? launch1(k_rope_qk<__bf16, 4, false>, grid, 256, s, a)
                            : launch1(k_rope_qk<float, 4, false>, grid, 256, s, a);
  }
  const int64_t grid = grid_for(static_cast<int64_t>(T) * (d / 2));
  if (cache)
    return dtype == RR_BF16 ? launch1(k_rope_qk<__bf16, 1, true>, grid, 256, s, a)
                            : launch1(k_rope_qk<float, 1, true>, grid, 256, s, a);
  return dtype == RR_BF16 ? launch1(k_rope_qk<__bf16, 1, false>, grid, 256, s, a)
                          : launch1(k_rope_qk<float, 1, false>, grid, 256, s, a);
}

}  // namespace rr
