// bf16 attention kernel on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Work item = (user, head, 128-query tile); a workgroup of four waves, 32 query
// rows per wave.  Under the candidate-isolation mask (Candidate isolation
// attention mask page, section "段 ID：掩码的表达方式") every valid query of a user
// reads the same key list -- the user's segment-1 rows, or in a candidate-only
// layer the frozen history (section "只更新候选的末尾层") -- so the main loop is a
// dense, unmasked rectangle: each K/V tile is staged once in LDS and shared by
// all 128 queries of the tile, history rows and candidates alike.  Only the last
// key tile is masked (its tail past the key count).  A candidate's extra key,
// itself, is added after the loop as a dot product across the wave's two lane
// halves rather than as a masked tile.
//
// Matrix orientation.  The kernel computes S^T = K Q^T so that each lane owns one
// query column of the 32x32 accumulator: the softmax row statistics (max, sum)
// are then in-lane reductions plus one exchange between the lane halves.  The
// output is accumulated transposed too, O^T = V^T P^T, with P^T taken straight
// from the S^T accumulators as the B operand.  Lane layouts of the 32x32x16 bf16
// instruction (lane l, i = l % 32, half = l / 32):
//   A operand (32 x 16): row i, k = 8*half + j      (j = 0..7, one 16-byte load)
//   B operand (16 x 32): column i, k = 8*half + j
//   C/D (32 x 32, 16 fp32): column i, row 8*(r/4) + 4*half + r%4   (r = 0..15)
// P^T's k index therefore comes out of the accumulator in a permuted key order
// (bits 2 and 3 of the key index within each group of 16 swapped); V^T is written
// to LDS in that same permuted order so the A and B operands agree.
//
// Numerics: bf16 operands, fp32 accumulation, online softmax in fp32 with exp2
// (scale * log2 e folded into one FMA), P rounded to bf16 for the PV product,
// output rounded to bf16 (round to nearest even).
#include "rr_internal.h"

namespace rr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;

constexpr int kWaves = 4;
constexpr int kQw = 32;                  // query rows per wave
constexpr int kBm = kWaves * kQw;        // query rows per work item
static_assert(kBm == kBmMfma, "tile height");
constexpr int kThreads = kWaves * 64;

__device__ __forceinline__ int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(unsigned, v);
}

template <int D, int BN, bool INDEXED>
__device__ __forceinline__ void attn_item(const AttnArgs& a, const int2 it, u16* __restrict__ s_k,
                                          u16* __restrict__ s_v) {
  constexpr int KSTR = D + 8;             // K tile row stride (elements); +16 B staggers LDS banks
  constexpr int VSTR = BN + 8;            // V^T tile row stride
  constexpr int KK = D / 16;              // k-steps of S^T
  constexpr int KB = BN / 32;             // 32-key blocks per tile
  constexpr int DB = D / 32;              // 32-wide blocks of O^T
  constexpr int KCH = BN * D / 8;         // 16-byte chunks of a K tile
  constexpr int KCH_T = (KCH + kThreads - 1) / kThreads;
  constexpr int VBLK = (BN / 4) * (D / 8);  // 4-key x 8-element blocks of a V tile
  constexpr int VBLK_T = (VBLK + kThreads - 1) / kThreads;
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");

  const int b = it.x, h = item_head(it), qt = item_tile(it);
  const UserMeta um = a.meta[b];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, ql = lane & 31;
  const int64_t rs = static_cast<int64_t>(a.H) * D;
  const u16* __restrict__ Qp = static_cast<const u16*>(a.q) + h * D;
  const u16* __restrict__ Kp = static_cast<const u16*>(a.k) + h * D;
  const u16* __restrict__ Vp = static_cast<const u16*>(a.v) + h * D;
  const u16* __restrict__ KSp = static_cast<const u16*>(a.k_self) + h * D;
  const u16* __restrict__ VSp = static_cast<const u16*>(a.v_self) + h * D;
  u16* __restrict__ Op = static_cast<u16*>(a.o) + h * D;
  const float sl2 = a.scale_log2;

  // this lane's query row
  const int qpos = qt * kBm + wave * kQw + ql;
  const bool qvalid = qpos < um.n_q;
  const int qe = um.q_begin + min(qpos, um.n_q - 1);
  const int qrow = INDEXED ? a.idx[qe] : qe;

  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(Qp + qrow * rs + 16 * kk + 8 * half);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_i = -INFINITY, l_i = 0.f;

  const int n_kv = um.n_kv;
  const int ntiles = (n_kv + BN - 1) / BN;

  uint4 kst[KCH_T];
  uint4 vst[VBLK_T][4];

  auto key_row = [&](int j) {
    const int e = um.kv_begin + min(j, n_kv - 1);   // clamp the tail into the key list
    return INDEXED ? a.idx[e] : e;
  };
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < KCH_T; ++i) {
      const int c = tid + kThreads * i;
      if (KCH % kThreads == 0 || c < KCH) {
        const int r = c / (D / 8), c8 = c % (D / 8);
        kst[i] = *reinterpret_cast<const uint4*>(Kp + key_row(t * BN + r) * rs + c8 * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < VBLK_T; ++i) {
      const int vb = tid + kThreads * i;
      if (VBLK % kThreads == 0 || vb < VBLK) {
        const int g = vb % (BN / 4), c8 = vb / (BN / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vst[i][r] = *reinterpret_cast<const uint4*>(Vp + key_row(t * BN + 4 * g + r) * rs + c8 * 8);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KCH_T; ++i) {
      const int c = tid + kThreads * i;
      if (KCH % kThreads == 0 || c < KCH) {
        const int r = c / (D / 8), c8 = c % (D / 8);
        *reinterpret_cast<uint4*>(&s_k[r * KSTR + c8 * 8]) = kst[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VBLK_T; ++i) {
      const int vb = tid + kThreads * i;
      if (VBLK % kThreads == 0 || vb < VBLK) {
        const int g = vb % (BN / 4), c8 = vb / (BN / 4);
        const int kv0 = 4 * g;
        const int col = (kv0 & ~15) | swap23(kv0 & 15);   // 4 keys stay contiguous
        const unsigned w0[4] = {vst[i][0].x, vst[i][0].y, vst[i][0].z, vst[i][0].w};
        const unsigned w1[4] = {vst[i][1].x, vst[i][1].y, vst[i][1].z, vst[i][1].w};
        const unsigned w2[4] = {vst[i][2].x, vst[i][2].y, vst[i][2].z, vst[i][2].w};
        const unsigned w3[4] = {vst[i][3].x, vst[i][3].y, vst[i][3].z, vst[i][3].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int wi = e >> 1;
          unsigned lo, hi;
          if (e & 1) {
            lo = (w0[wi] >> 16) | (w1[wi] & 0xffff0000u);
            hi = (w2[wi] >> 16) | (w3[wi] & 0xffff0000u);
          } else {
            lo = (w0[wi] & 0xffffu) | (w1[wi] << 16);
            hi = (w2[wi] & 0xffffu) | (w3[wi] << 16);
          }
          *reinterpret_cast<uint2*>(&s_v[(c8 * 8 + e) * VSTR + col]) = make_uint2(lo, hi);
        }
      }
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile();
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) load_tile(t + 1);   // next tile's global loads overlap this tile's math

    // S^T = K Q^T for this wave's 32 queries
    f32x16 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(&s_k[(kb * 32 + ql) * KSTR + 16 * kk + 8 * half]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc[kb], 0, 0, 0);
      }
    }
    if (t == ntiles - 1 && (n_kv % BN) != 0) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = t * BN + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (j >= n_kv) sacc[kb][r] = -INFINITY;
        }
    }
    // online softmax, one query per lane (key halves split across the lane halves)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_i, mx * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m_i - m_new);
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], sl2, -m_new));
        sacc[kb][r] = p;
        ls += p;
      }
    l_i = l_i * alpha + ls;
    m_i = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
      const int kb = ks >> 1, s8 = (ks & 1) * 8;
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = static_cast<__bf16>(sacc[kb][s8 + j]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 vf =
            *reinterpret_cast<const bf16x8*>(&s_v[(db * 32 + ql) * VSTR + 16 * ks + 8 * half]);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[db], 0, 0, 0);
      }
    }
    __syncthreads();
    if (more) {
      store_tile();
      __syncthreads();
    }
  }

  // both lane halves hold partial sums of the same query
  float l_tot = l_i + __shfl_xor(l_i, 32);

  // candidate self-term: <q, own k> as a dot product split across the two halves
  float sd = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const uint4 kw = *reinterpret_cast<const uint4*>(KSp + qrow * rs + 16 * kk + 8 * half);
    const unsigned kwv[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sd = fmaf(static_cast<float>(qf[kk][2 * j]), bf16_lo(kwv[j]), sd);
      sd = fmaf(static_cast<float>(qf[kk][2 * j + 1]), bf16_hi(kwv[j]), sd);
    }
  }
  sd += __shfl_xor(sd, 32);
  if (qpos >= um.cand_rel) {
    const float ts = sd * sl2;
    const float mn = fmaxf(m_i, ts);
    const float al = __builtin_amdgcn_exp2f(m_i - mn);
    const float be = __builtin_amdgcn_exp2f(ts - mn);
    l_tot = l_tot * al + be;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint2 vw =
            *reinterpret_cast<const uint2*>(VSp + qrow * rs + db * 32 + 8 * g + 4 * half);
        oacc[db][4 * g + 0] = oacc[db][4 * g + 0] * al + be * bf16_lo(vw.x);
        oacc[db][4 * g + 1] = oacc[db][4 * g + 1] * al + be * bf16_hi(vw.x);
        oacc[db][4 * g + 2] = oacc[db][4 * g + 2] * al + be * bf16_lo(vw.y);
        oacc[db][4 * g + 3] = oacc[db][4 * g + 3] * al + be * bf16_hi(vw.y);
      }
  }

  if (qvalid) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint2 w = make_uint2(pack_bf16(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                                   pack_bf16(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv));
        *reinterpret_cast<uint2*>(Op + qrow * rs + db * 32 + 8 * g + 4 * half) = w;
      }
  }
}

template <int D, int BN>
__global__ __launch_bounds__(kThreads, 2) void k_attn_mfma(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) u16 s_k[BN * (D + 8)];
  __shared__ __attribute__((aligned(16))) u16 s_v[D * (BN + 8)];
  if (!plan_matches(a, kBm)) return;
  const int item = blockIdx.x;
  if (item >= a.plan->n_items) return;
  const int2 it = a.items[item];
  if (item_head(it) == kZeroHead) {
    zero_padding_tile(a, a.meta[it.x], item_tile(it), kBm, a.H * D * 2, threadIdx.x, kThreads);
    return;
  }
  if (a.plan->indexed)
    attn_item<D, BN, true>(a, it, s_k, s_v);
  else
    attn_item<D, BN, false>(a, it, s_k, s_v);
}

template <int D, int BN>
hipError_t go(const AttnArgs& a, int64_t grid, hipStream_t s) {
  return launch1(k_attn_mfma<D, BN>, grid, kThreads, s, a);
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, int d, int64_t grid, hipStream_t s) {
  switch (d) {
    case 32: return go<32, 128>(a, grid, s);
    case 64: return go<64, 128>(a, grid, s);
    case 128: return go<128, 64>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rr
