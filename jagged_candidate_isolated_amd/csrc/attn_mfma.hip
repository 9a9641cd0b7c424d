// bf16 attention kernel on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Work item = (user, head, query tile of NW*32 rows); a workgroup of NW waves, 32
// query rows per wave.  Under the candidate-isolation mask (Candidate isolation
// attention mask page, section "段 ID：掩码的表达方式") every valid query of a user
// reads the same key list -- the user's segment-1 rows, or in a candidate-only
// layer the frozen history (section "只更新候选的末尾层") -- so the main loop is a
// dense, unmasked rectangle: each K/V tile is staged once in LDS and shared by all
// queries of the tile, history rows and candidates alike.  Only the last key tile
// is masked (its tail past the key count).  A candidate's extra key, itself, is
// added after the loop as a dot product across the wave's two lane halves rather
// than as a masked tile.
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
// (bits 2 and 3 of the key index within each group of 16 swapped); the V^T
// operand is read in that same permuted order so the A and B operands agree.
//
// Pipeline.  K and V tiles go to LDS by direct-to-LDS loads (no register staging)
// into NS rotating buffers, NS-1 tiles ahead of the tile being computed; one
// barrier per tile.  Two tile shapes: narrow (four waves, 128 query rows, two stages,
// two to four workgroups per CU) and wide (eight waves, 256 query rows, four stages, one
// workgroup per CU) for batches of long users.  A small unpadded batch can skip the
// planning kernel: each workgroup then builds the work list itself (self_plan_item).
//
// Numerics: bf16 operands, fp32 accumulation, online softmax in fp32 with exp2
// (scale * log2 e folded into one FMA), P rounded to bf16 for the PV product,
// output rounded to bf16 (round to nearest even).
#include "mfma_tile.h"

namespace rr {
namespace {

template <int D, int BN, int NW, int NS, bool KEY_IDX>
__device__ __forceinline__ void attn_item(const AttnArgs& a, const int2 it, const UserMeta& um,
                                          bool indexed, const Stages& st) {
  constexpr int kThreads = NW * 64;
  constexpr int kBm = NW * kQw;
  using Loader = KvLoader<D, BN, kThreads, KEY_IDX>;
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int LPT = Loader::LPT;           // vector-memory operations per thread per tile
  constexpr int KK = D / 16;                 // k-steps of S^T
  constexpr int KB = BN / 32;                // 32-key blocks per tile
  constexpr int DB = D / 32;                 // 32-wide blocks of O^T
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");
  static_assert(NS >= 2 && NS <= 4, "pipeline stages");

  const int h = item_head(it), qt = item_tile(it);

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

  // this lane's query row, and its Q operand (loaded before any tile, so the tile
  // loads are the only vector-memory operations the loop waits on)
  const int qpos = qt * kBm + wave * kQw + ql;
  const bool qvalid = qpos < um.n_q;
  const int qe = um.q_begin + min(qpos, um.n_q - 1);
  const int qrow = indexed ? a.idx[qe] : qe;
  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(Qp + qrow * rs + 16 * kk + 8 * half);

  const int n_kv = um.n_kv;
  const int ntiles = (n_kv + BN - 1) / BN;

  constexpr int AHEAD = NS - 1;   // tiles loaded ahead of the tile being computed
  static_assert((AHEAD - 1) * Loader::LPT < 64, "pipeline depth");

  // direct-to-LDS loads of key/value tile t into stage t % NS
  const Loader ld(Kp, Vp, a.idx, rs, um.kv_begin, n_kv, tid);
  auto issue_tile = [&](int t, auto stage_tag) {
    constexpr int STAGE = decltype(stage_tag)::value;
    ld.issue(t, st.k[STAGE], st.v[STAGE]);
  };

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1 % NS>;
  using C2 = std::integral_constant<int, 2 % NS>;
  using C3 = std::integral_constant<int, 3 % NS>;
  // prologue: the first AHEAD tiles in flight
  if (0 < ntiles) issue_tile(0, C0{});
  if constexpr (AHEAD > 1) {
    if (1 < ntiles) issue_tile(1, C1{});
  }
  if constexpr (AHEAD > 2) {
    if (2 < ntiles) issue_tile(2, C2{});
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_i = -INFINITY, l_i = 0.f;
  f32x16 sacc[KB];   // S^T of the tile between its S and PV steps (P after the softmax)

  // per-lane byte offsets of the LDS operand reads (k-step / block add constants)
  uint32_t k_off[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) k_off[kk] = (ql * CH + ((2 * kk + half) ^ swz<CH>(ql))) * 16;
  uint32_t v_off[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    v_off[db][0] = vt_offset<D>(db, 0, lane);
    v_off[db][1] = vt_offset<D>(db, 1, lane);
  }

  // S^T = K Q^T for this wave's 32 queries; the KB accumulator chains interleave
  auto s_step = [&](auto stage_tag) {
    const char* sk = reinterpret_cast<const char*>(st.k[decltype(stage_tag)::value]);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sk + k_off[kk] + kb * 32 * CH * 16);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc[kb], 0, 0, 0);
      }
  };
  // online softmax of tile t, one query per lane (key halves split across the lane halves)
  auto softmax_step = [&](int t) {
    if ((t + 1) * BN > n_kv) {
      // The partial last tile: keys past the list get -inf.  Element (kb, r) of this
      // lane is key t*BN + c + 4*half with c = 32 kb + 8 (r/4) + r%4; it is masked
      // when c >= lim.  Adding 0 or -inf built from the sign of c - lim keeps the
      // per-element tests in vector registers (compares would each take a scalar
      // lane mask).
      const int lim = n_kv - t * BN - 4 * half;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
          sacc[kb][r] += __int_as_float(~((c - lim) >> 31) & static_cast<int>(0xff800000u));
        }
    }
    float mx[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float m = max3f(sacc[kb][0], sacc[kb][1], sacc[kb][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) m = max3f(m, sacc[kb][r], sacc[kb][r + 1]);
      mx[kb] = fmaxf(m, sacc[kb][15]);
    }
#pragma unroll
    for (int w = 1; w < KB; w <<= 1)
#pragma unroll
      for (int kb = 0; kb + w < KB; kb += 2 * w) mx[kb] = fmaxf(mx[kb], mx[kb + w]);
    const float tmax = halves_max(mx[0]) * sl2;
    const bool move = tmax > m_i + kLazyRescale;   // per row: move the reference up
    if (__any(move)) {
      const float alpha = move ? __builtin_amdgcn_exp2f(m_i - tmax) : 1.f;
      l_i *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_i = move ? tmax : m_i;
    }
    float ls[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float s4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int r = 4 * g; r < 4 * g + 4; ++r)
          sacc[kb][r] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], sl2, -m_i));
        s4[g] = (sacc[kb][4 * g] + sacc[kb][4 * g + 1]) + (sacc[kb][4 * g + 2] + sacc[kb][4 * g + 3]);
      }
      ls[kb] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
#pragma unroll
    for (int w = 1; w < KB; w <<= 1)
#pragma unroll
      for (int kb = 0; kb + w < KB; kb += 2 * w) ls[kb] += ls[kb + w];
    l_i += ls[0];
  };
  // O^T += V^T P^T
  auto pv_step = [&](auto stage_tag) {
    const char* sv = reinterpret_cast<const char*>(st.v[decltype(stage_tag)::value]);
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
      const int kb = ks >> 1, s8 = (ks & 1) * 8;
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = static_cast<__bf16>(sacc[kb][s8 + j]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char* base = sv + ks * 16 * CH * 16;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_vt(base, v_off[db][0], v_off[db][1]),
                                                           pf, oacc[db], 0, 0, 0);
      }
    }
  };

  auto tile = [&](int t, auto cur_tag) {
    constexpr int CUR = decltype(cur_tag)::value;
    // Tile t has landed once no more than the loads of the tiles issued after it are
    // outstanding (this wave's loads, retiring in order); the barrier makes every
    // wave's loads visible and tells that every wave is done with the stage of tile
    // t+AHEAD, refilled next to overlap the following tiles' math.
    wait_tiles<LPT>(min(AHEAD - 1, ntiles - 1 - t));
    tile_barrier();
    if (t + AHEAD < ntiles) issue_tile(t + AHEAD, std::integral_constant<int, (CUR + AHEAD) % NS>{});
    s_step(cur_tag);
    softmax_step(t);
    pv_step(cur_tag);
  };
  // One loop, NS tiles per trip, so that tile t always uses stage t % NS as a
  // compile-time constant; the tiles past the end of the list are skipped.
  for (int t = 0; t < ntiles; t += NS) {
    tile(t, C0{});
    if (t + 1 < ntiles) tile(t + 1, C1{});
    if constexpr (NS > 2) {
      if (t + 2 < ntiles) tile(t + 2, C2{});
    }
    if constexpr (NS > 3) {
      if (t + 3 < ntiles) tile(t + 3, C3{});
    }
  }
  // both lane halves hold partial sums of the same query
  float l_tot = halves_sum(l_i);

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
  sd = halves_sum(sd);
  float mref = m_i;   // the reference the row's sum l_tot is taken against (log2 units)
  if (qpos >= um.cand_rel) {
    const float ts = sd * sl2;
    const float mn = fmaxf(m_i, ts);
    mref = mn;
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
    if (a.lse && half == 0)
      a.lse[static_cast<int64_t>(qrow) * a.H + h] =
          l_tot > 0.f ? (mref + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
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

template <int D, int BN, int NW, int NS, bool SELF>
__global__ __launch_bounds__(NW * 64, 2) void k_attn_mfma(AttnArgs a) {
  // pipeline stages (stages past NS are never referenced and take no LDS)
  __shared__ __attribute__((aligned(16))) u16 k0[BN * D], k1[BN * D], k2[BN * D], k3[BN * D];
  __shared__ __attribute__((aligned(16))) u16 v0[BN * D], v1[BN * D], v2[BN * D], v3[BN * D];
  const Stages st{{k0, k1, k2, k3}, {v0, v1, v2, v3}};
  int2 it;
  UserMeta um;
  bool indexed = false;
  if constexpr (SELF) {   // an unpadded batch planned in this workgroup
    __shared__ SelfPlanLds sp;
    if (!self_plan_item(a.offsets, a.cand_start, a.B, a.H, NW * kQw, a.rows, xcd_item(blockIdx.x), sp, it, um))
      return;
    attn_item<D, BN, NW, NS, false>(a, it, um, false, st);
    return;
  }
  if (!fetch_item(a, NW * kQw, xcd_item(blockIdx.x), it, um, indexed)) return;
  if (item_head(it) == kZeroHead) {
    zero_padding_tile(a, um, item_tile(it), NW * kQw, a.H * D * 2, threadIdx.x, NW * 64);
    return;
  }
  // key rows go through idx[] only for a padded user whose key rows are not one range
  if (indexed && !um.kv_direct)
    attn_item<D, BN, NW, NS, true>(a, it, um, indexed, st);
  else
    attn_item<D, BN, NW, NS, false>(a, it, um, indexed, st);
}

template <int D, int BN, int NW, int NS, bool SELF = false>
hipError_t go(const AttnArgs& a, int64_t grid, hipStream_t s) {
  return launch1(k_attn_mfma<D, BN, NW, NS, SELF>, grid, NW * 64, s, a);
}

}  // namespace

// Tile shapes (compile-time tuning knobs).  Narrow: four waves, 128 query rows, four
// workgroups per CU at d = 32 and 64, two at d = 128 (registers).  Wide: eight waves,
// 256 query rows, one workgroup per CU.
#ifndef RR_NARROW_STAGES
#define RR_NARROW_STAGES 2
#endif
#ifndef RR_NARROW_BN64
#define RR_NARROW_BN64 64
#endif
#ifndef RR_NARROW_BN128
#define RR_NARROW_BN128 64
#endif
#ifndef RR_WIDE_STAGES
#define RR_WIDE_STAGES 4
#endif
#ifndef RR_WIDE_BN64
#define RR_WIDE_BN64 64
#endif
#ifndef RR_WIDE_BN128
#define RR_WIDE_BN128 64
#endif

namespace {

template <bool SELF>
hipError_t launch_mfma(const AttnArgs& a, int d, int bm, int64_t grid, hipStream_t s) {
  if (bm == kBmMfmaWide) {
    constexpr int NW = kBmMfmaWide / kQw, NS = RR_WIDE_STAGES;
    switch (d) {
      case 32: return go<32, 128, NW, NS, SELF>(a, grid, s);
      case 64: return go<64, RR_WIDE_BN64, NW, NS, SELF>(a, grid, s);
      case 128: return go<128, RR_WIDE_BN128, NW, NS, SELF>(a, grid, s);
      default: return hipErrorInvalidValue;
    }
  }
  constexpr int NW = kBmMfmaNarrow / kQw, NS = RR_NARROW_STAGES;
  switch (d) {
    case 32: return go<32, 128, NW, NS, SELF>(a, grid, s);
    case 64: return go<64, RR_NARROW_BN64, NW, NS, SELF>(a, grid, s);
    case 128: return go<128, RR_NARROW_BN128, NW, NS, SELF>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, int d, int bm, int64_t grid, hipStream_t s) {
  return launch_mfma<false>(a, d, bm, grid, s);
}

// The batch's offsets and cand_start in a.offsets / a.cand_start, no plan: a.B <=
// kSelfPlanUsers (and <= the workgroup size, 2 bm) and grid <= kSelfPlanGrid.
hipError_t launch_attn_mfma_self_planned(const AttnArgs& a, int d, int bm, int64_t grid, hipStream_t s) {
  if (a.B > kSelfPlanUsers || a.B > 2 * bm || grid > kSelfPlanGrid) return hipErrorInvalidValue;
  return launch_mfma<true>(a, d, bm, grid, s);
}

}  // namespace rr
