// VALU attention kernel: fp32 inputs (any supported d) and bf16 inputs with d = 16.
//
// One wave per work item (user, head, 64-query tile); lane i owns query row i of
// the tile.  Every query of a user reads the same key list (the user's segment-1
// rows, or the frozen history in a candidate-only layer), so each tile of keys
// and values is staged once in LDS and read by all 64 lanes as broadcasts.
// Online softmax in fp32 with exp2 (scale * log2 e folded into the score).
// A candidate adds its own key after the key list: the candidate self-term of
// the mask rule (Candidate isolation attention mask page, section "段 ID：掩码的表达方式").
#include "rr_internal.h"

namespace rr {
namespace {

constexpr int kLanes = kBmSimple;   // 64 query rows per item, one per lane

template <int D>
constexpr int keys_per_tile() { return D == 128 ? 32 : 64; }   // LDS tiles stay within 32 KB each

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const __bf16* p) { return static_cast<float>(*p); }
__device__ __forceinline__ void st(float* p, float x) { *p = x; }
__device__ __forceinline__ void st(__bf16* p, float x) { *p = static_cast<__bf16>(x); }

template <typename T, int D, bool KEY_IDX>
__device__ __forceinline__ void attn_item(const AttnArgs& a, const int2 it, const UserMeta& um,
                                          bool indexed, float (*__restrict__ s_k)[D],
                                          float (*__restrict__ s_v)[D]) {
  constexpr int kKeys = keys_per_tile<D>();
  const int h = item_head(it), qt = item_tile(it);
  const int lane = threadIdx.x;
  const int64_t rs = static_cast<int64_t>(a.H) * D;
  const T* __restrict__ Q = static_cast<const T*>(a.q);
  const T* __restrict__ K = static_cast<const T*>(a.k);
  const T* __restrict__ V = static_cast<const T*>(a.v);
  const T* __restrict__ KS = static_cast<const T*>(a.k_self);
  const T* __restrict__ VS = static_cast<const T*>(a.v_self);
  T* __restrict__ O = static_cast<T*>(a.o);

  const int qpos = qt * kLanes + lane;
  const bool qvalid = qpos < um.n_q;
  const int qe = um.q_begin + min(qpos, um.n_q - 1);
  const int qrow = indexed ? a.idx[qe] : qe;
  const float sl2 = a.scale_log2;

  float q[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = ld(Q + qrow * rs + h * D + e);
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int n_kv = um.n_kv;
  for (int j0 = 0; j0 < n_kv; j0 += kKeys) {
    __syncthreads();
    if (lane < kKeys) {
      const int j = min(j0 + lane, n_kv - 1);
      const int ke = um.kv_begin + j;
      const int krow = KEY_IDX ? a.idx[ke] : ke;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        s_k[lane][e] = ld(K + krow * rs + h * D + e);
        s_v[lane][e] = ld(V + krow * rs + h * D + e);
      }
    }
    __syncthreads();
    const int nj = min(kKeys, n_kv - j0);
    float s[kKeys];
    float tmax = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kKeys; ++jj) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(q[e], s_k[jj][e], dot);
      s[jj] = jj < nj ? dot * sl2 : -INFINITY;
      tmax = fmaxf(tmax, s[jj]);
    }
    const float m_new = fmaxf(m, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] *= alpha;
#pragma unroll
    for (int jj = 0; jj < kKeys; ++jj) {
      const float p = __builtin_amdgcn_exp2f(s[jj] - m_new);
      l += p;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(p, s_v[jj][e], acc[e]);
    }
    m = m_new;
  }
  if (qpos >= um.cand_rel) {
    // candidate self-term: its own key and value, after the key list
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) dot = fmaf(q[e], ld(KS + qrow * rs + h * D + e), dot);
    const float t = dot * sl2;
    const float m_new = fmaxf(m, t);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    const float beta = __builtin_amdgcn_exp2f(t - m_new);
    l = l * alpha + beta;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] = acc[e] * alpha + beta * ld(VS + qrow * rs + h * D + e);
    m = m_new;
  }
  if (qvalid) {
    if (a.lse)
      a.lse[static_cast<int64_t>(qrow) * a.H + h] =
          l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) st(O + qrow * rs + h * D + e, acc[e] * inv);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kLanes) void k_attn_simple(AttnArgs a) {
  constexpr int kKeys = keys_per_tile<D>();
  __shared__ float s_k[kKeys][D];
  __shared__ float s_v[kKeys][D];
  int2 it;
  UserMeta um;
  bool indexed;
  if (!fetch_item(a, kLanes, blockIdx.x, it, um, indexed)) return;
  if (item_head(it) == kZeroHead) {
    zero_padding_tile(a, um, item_tile(it), kLanes, a.H * D * int(sizeof(T)), threadIdx.x, kLanes);
    return;
  }
  // key rows go through idx[] only for a padded user whose key rows are not one range
  if (indexed && !um.kv_direct)
    attn_item<T, D, true>(a, it, um, indexed, s_k, s_v);
  else
    attn_item<T, D, false>(a, it, um, indexed, s_k, s_v);
}

template <typename T, int D>
hipError_t go(const AttnArgs& a, int64_t grid, hipStream_t s) {
  return launch1(k_attn_simple<T, D>, grid, kLanes, s, a);
}

}  // namespace

hipError_t launch_attn_simple(const AttnArgs& a, int d, int dtype, int64_t grid, hipStream_t s) {
  if (dtype == RR_BF16) {
    if (d == 16) return go<__bf16, 16>(a, grid, s);
    return hipErrorInvalidValue;
  }
  switch (d) {
    case 16: return go<float, 16>(a, grid, s);
    case 32: return go<float, 32>(a, grid, s);
    case 64: return go<float, 64>(a, grid, s);
    case 128: return go<float, 128>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rr
