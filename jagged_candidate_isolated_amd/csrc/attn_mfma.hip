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

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(unsigned, v);
}

// LDS tile layout.  A K or V tile is BN rows of D bf16 (row-major), stored in
// 16-byte chunks; chunk c of row r sits at position c ^ swz(r) of that row.  The
// swizzle keeps both kinds of reads free of bank conflicts: the K reads (16
// consecutive rows, one chunk each) and the transposed V reads (4 consecutive rows,
// 4 chunks each) touch distinct banks.  Tiles arrive by direct-to-LDS loads: lane l
// of a load writes LDS slot l, so the swizzle is applied by choosing which global
// chunk each lane fetches.
template <int CH>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CH == 16) return 4 * (row & 3) + ((row >> 2) & 3);
  else if constexpr (CH == 8) return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
  else return (row >> 2) & 3;   // CH == 4: 64-byte rows
}

#define LDS_AS __attribute__((address_space(3)))
typedef short v4i16 __attribute__((ext_vector_type(4)));

// V^T operand of the PV product for k-step ks and output block db: eight keys of one
// V column per lane, read with two transposed LDS loads.  Within each 16-lane group
// the transposed load returns, in lane j, element j%4 of the 8-byte pieces addressed
// by lanes 4k + j/4 (k = 0..3); each lane therefore addresses row (key) 4*half + s/4
// at columns 4*(s%4)..+3 of its group's 16 columns, and gets one column, four keys.
template <int D>
__device__ __forceinline__ bf16x8 read_vt(const u16* __restrict__ sv, int ks, int db, int lane) {
  constexpr int CH = D / 8;
  const int s = lane & 15, grp = (lane >> 4) & 1, half = lane >> 5;
  const int col = db * 32 + 16 * grp + 4 * (s & 3);      // first of 4 columns (elements)
  const int c = col >> 3, sub = (col & 7) * 2;           // 16-byte chunk, byte offset in it
  v4i16 r[2];
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    const int row = ks * 16 + 8 * part + 4 * half + (s >> 2);
    const int p = c ^ swz<CH>(row);
    LDS_AS char* addr = (LDS_AS char*)(sv) + (row * CH + p) * 16 + sub;   // generic -> LDS address space
    r[part] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)addr);
  }
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 w = {r[0][0], r[0][1], r[0][2], r[0][3], r[1][0], r[1][1], r[1][2], r[1][3]};
  return __builtin_bit_cast(bf16x8, w);
}

template <int D, int BN, bool INDEXED>
__device__ __forceinline__ void attn_item(const AttnArgs& a, const int2 it, u16* __restrict__ s_k,
                                          u16* __restrict__ s_v) {
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int TILE = BN * D;               // elements per K (or V) tile
  constexpr int LOADS = TILE * 2 / (kThreads * 16);   // direct-to-LDS loads per thread per tile
  constexpr int KK = D / 16;                 // k-steps of S^T
  constexpr int KB = BN / 32;                // 32-key blocks per tile
  constexpr int DB = D / 32;                 // 32-wide blocks of O^T
  static_assert(D % 32 == 0 && BN % 32 == 0 && LOADS >= 1 && TILE * 2 % (kThreads * 16) == 0,
                "tile shape");

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

  const int n_kv = um.n_kv;
  const int ntiles = (n_kv + BN - 1) / BN;

  // Issue the direct-to-LDS loads of key/value tile t into buffer t & 1.  Load i of
  // wave w fills LDS slots (w*LOADS + i)*64 + lane; slot -> (row, chunk position).
  auto issue_tile = [&](int t) {
    u16* dk = s_k + (t & 1) * TILE;
    u16* dv = s_v + (t & 1) * TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int slot = (wave * LOADS + i) * 64 + lane;
      const int row = slot / CH, p = slot % CH;
      const int c = p ^ swz<CH>(row);
      const int e = um.kv_begin + min(t * BN + row, n_kv - 1);   // clamp the tail into the list
      const int64_t g = static_cast<int64_t>(INDEXED ? a.idx[e] : e) * rs + c * 8;
      const int lds_off = (wave * LOADS + i) * 64 * 8;           // elements; one load = 1 KiB
      __builtin_amdgcn_global_load_lds(Kp + g, (LDS_AS void*)(dk + lds_off), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(Vp + g, (LDS_AS void*)(dv + lds_off), 16, 0, 0);
    }
  };

  if (ntiles > 0) issue_tile(0);

  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(Qp + qrow * rs + 16 * kk + 8 * half);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_i = -INFINITY, l_i = 0.f;

  // per-lane parts of the K operand addresses (rows kb*32 + ql)
  int k_row_off[KB], k_mask[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int row = kb * 32 + ql;
    k_row_off[kb] = row * CH;
    k_mask[kb] = swz<CH>(row) ^ half;
  }

  for (int t = 0; t < ntiles; ++t) {
    // tile t has landed (this wave's loads) and is visible (every wave's, after the
    // barrier); the barrier also tells that every wave is done with buffer (t+1)&1
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntiles) issue_tile(t + 1);   // overlaps this tile's math
    const u16* sk = s_k + (t & 1) * TILE;
    const u16* sv = s_v + (t & 1) * TILE;

    // S^T = K Q^T for this wave's 32 queries
    f32x16 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int p = (2 * kk) ^ k_mask[kb];
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sk + (k_row_off[kb] + p) * 8);
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
    // online softmax, one query per lane (key halves split across the lane halves);
    // max and sum as trees to keep the dependency chains short
    float mx[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float m4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        m4[g] = fmaxf(fmaxf(sacc[kb][4 * g], sacc[kb][4 * g + 1]),
                      fmaxf(sacc[kb][4 * g + 2], sacc[kb][4 * g + 3]));
      mx[kb] = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    }
#pragma unroll
    for (int w = 1; w < KB; w <<= 1)
#pragma unroll
      for (int kb = 0; kb + w < KB; kb += 2 * w) mx[kb] = fmaxf(mx[kb], mx[kb + w]);
    float tmax = fmaxf(mx[0], __shfl_xor(mx[0], 32));
    const float m_new = fmaxf(m_i, tmax * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m_i - m_new);
    float ls[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float s4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int r = 4 * g; r < 4 * g + 4; ++r)
          sacc[kb][r] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], sl2, -m_new));
        s4[g] = (sacc[kb][4 * g] + sacc[kb][4 * g + 1]) + (sacc[kb][4 * g + 2] + sacc[kb][4 * g + 3]);
      }
      ls[kb] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
#pragma unroll
    for (int w = 1; w < KB; w <<= 1)
#pragma unroll
      for (int kb = 0; kb + w < KB; kb += 2 * w) ls[kb] += ls[kb + w];
    l_i = l_i * alpha + ls[0];
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
      for (int db = 0; db < DB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_vt<D>(sv, ks, db, lane), pf, oacc[db],
                                                           0, 0, 0);
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
  // no wave may leave while others still read LDS tiles it helped load (the loads
  // are complete once every wave passed the last in-loop barrier), nothing to wait for
}

template <int D, int BN>
__global__ __launch_bounds__(kThreads, 2) void k_attn_mfma(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) u16 s_k[2 * BN * D];   // double-buffered K tiles
  __shared__ __attribute__((aligned(16))) u16 s_v[2 * BN * D];   // double-buffered V tiles
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
