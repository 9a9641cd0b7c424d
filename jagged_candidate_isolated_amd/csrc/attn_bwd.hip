// Backward pass of the candidate-isolated attention on gfx950 matrix cores.
//
// Gradients of O = softmax(scale q k^T over the admitted keys) v, with the softmax
// recomputed from the forward's per-row log-sum-exp (lse):
//   P = exp(scale s - lse),  dV = P^T dO,  dP = dO v^T,  dS = P (dP - delta),
//   dq = scale dS k,  dk = scale dS^T q,  delta = rowsum(dO * O).
// Under the isolation mask (Candidate isolation attention mask page, section
// "段 ID：掩码的表达方式") every valid query of a user reads the same key list (its
// segment-1 rows) and a candidate also reads itself, so
//   * a history key's dk, dv sum over all valid queries of its user: a dense
//     rectangle, computed key-major (k_bwd_dkdv);
//   * a query's dq sums over its user's key list plus, for a candidate, its own key:
//     the forward's loop shape, computed query-major (k_bwd_dq);
//   * a candidate's own key and value are read by that candidate alone, so their
//     gradients come straight out of k_bwd_dq's self-term.
// Every output row is written by exactly one workgroup (no atomics), so the result
// is deterministic.  A candidate-only layer (Candidate isolation attention mask page,
// section "只更新候选的末尾层") runs the same two kernels: the query-major one over its
// candidates (own key and value gradients from the self-term), the key-major one over
// the frozen history keys with a plan whose items are key tiles.  Both kernels take the forward's plan as it is (tiles of 128 or 256
// query rows) and give each 128-row sub-tile of an item its own workgroup: query rows
// in the query-major kernel; in the key-major kernel item (user, head, t) stands for
// key tile t of the same height, which always exists because a user's keys are a
// subset of its queries.
//
// Orientations follow the forward kernel (attn_mfma.hip): k_bwd_dq computes S^T and
// dP^T with one query column per lane and accumulates dq^T = k^T dS^T with the
// transposed LDS reads the forward uses for V; k_bwd_dkdv computes S and dP with one
// key column per lane and accumulates dv^T = dO^T P and dk^T = q^T dS the same way.
#include "mfma_tile.h"

// Tuning knobs: k_bwd_dq's key tile per head dimension (at d = 64, 64 keys for launches
// of at most RR_BWD_SMALL_GRID workgroups, whose longest items set the time, and
// RR_BWD_DQ_BN64 otherwise), k_bwd_dkdv's query tile at d = 64, and the smallest head
// dimension whose k_bwd_dkdv reads V operands from LDS rather than registers.  The
// tiles change no result: every gradient accumulates the same 16-row MFMA steps in
// the same order whatever the tile.
#ifndef RR_BWD_DQ_BN64
#define RR_BWD_DQ_BN64 32
#endif
#ifndef RR_BWD_SMALL_GRID
#define RR_BWD_SMALL_GRID 2048
#endif
#ifndef RR_BWD_DQ_BN128
#define RR_BWD_DQ_BN128 32
#endif
#ifndef RR_BWD_VLDS_MIN_D
#define RR_BWD_VLDS_MIN_D 128
#endif
#ifndef RR_BWD_DKDV_BQ64
#define RR_BWD_DKDV_BQ64 64
#endif

namespace rr {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdRows = kBwdWaves * kQw;   // 128: query rows (dq) or keys (dk, dv) per sub-tile
static_assert(kBmMfmaNarrow % kBwdRows == 0 && kBmMfmaWide % kBwdRows == 0, "plan tiles");
constexpr float kLog2e = 1.4426950408889634f;

struct BwdArgs {
  AttnArgs a;            // q, k, v, o = the forward output; the plan; scale_log2
  const void* dout;      // dO [rows][H][d]
  const float* lse;      // [rows][H], natural log, from the forward
  void* dq;
  void* dk;
  void* dv;
  float* delta;          // [rows][H] rowsum(dO * O): written by k_bwd_dq, read by k_bwd_dkdv
  void* dk_self;         // a candidate's own key and value gradients (dk, dv in full mode;
  void* dv_self;         // the candidate tensors' gradients in a candidate-only layer)
  float scale;
  int bm;                // the plan's tile height (a multiple of kBwdRows)
};

__device__ __forceinline__ bf16x8 load8(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ float dot8(const bf16x8 a, const bf16x8 b, float acc) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = fmaf(static_cast<float>(a[j]), static_cast<float>(b[j]), acc);
  return acc;
}

__device__ __forceinline__ void store8(u16* p, const bf16x8 x, float f) {
  bf16x8 y;
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = static_cast<__bf16>(static_cast<float>(x[j]) * f);
  *reinterpret_cast<bf16x8*>(p) = y;
}

// One O^T-layout accumulator row set of a lane (d = db*32 + 8g + 4*half + t) -> bf16 row.
template <int DB>
__device__ __forceinline__ void store_acc_row(u16* row, const f32x16 (&acc)[DB], float f, int half) {
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint2 w = make_uint2(pack_bf16(acc[db][4 * g + 0] * f, acc[db][4 * g + 1] * f),
                                 pack_bf16(acc[db][4 * g + 2] * f, acc[db][4 * g + 3] * f));
      *reinterpret_cast<uint2*>(row + db * 32 + 8 * g + 4 * half) = w;
    }
}

// --------------------------------------------------------------------------- dq

template <int D, int BN, bool KEY_IDX>
__device__ __forceinline__ void dq_item(const BwdArgs& g, int h, int qt, const UserMeta& um,
                                        bool indexed, const Stages& st) {
  constexpr int NS = 2, kThreads = kBwdWaves * 64;
  using Loader = KvLoader<D, BN, kThreads, KEY_IDX>;
  constexpr int CH = D / 8, KK = D / 16, KB = BN / 32, DB = D / 32;
  const AttnArgs& a = g.a;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, ql = lane & 31;
  const int64_t rs = static_cast<int64_t>(a.H) * D;
  const u16* Qp = static_cast<const u16*>(a.q) + h * D;
  const u16* Kp = static_cast<const u16*>(a.k) + h * D;
  const u16* Vp = static_cast<const u16*>(a.v) + h * D;
  const u16* Op = static_cast<const u16*>(a.o) + h * D;
  const u16* DOp = static_cast<const u16*>(g.dout) + h * D;
  const float sl2 = a.scale_log2;

  const int qpos = qt * kBwdRows + wave * kQw + ql;
  const bool qvalid = qpos < um.n_q;
  const int qe = um.q_begin + min(qpos, um.n_q - 1);
  const int qrow = indexed ? a.idx[qe] : qe;
  const int64_t rbase = static_cast<int64_t>(qrow) * rs;
  bf16x8 qf[KK], df[KK];
  float dsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qf[kk] = load8(Qp + rbase + 16 * kk + 8 * half);
    df[kk] = load8(DOp + rbase + 16 * kk + 8 * half);
    dsum = dot8(df[kk], load8(Op + rbase + 16 * kk + 8 * half), dsum);
  }
  const float drow = halves_sum(dsum);                          // delta of this query row
  const float lse2 = g.lse[static_cast<int64_t>(qrow) * a.H + h] * kLog2e;
  if (qvalid && half == 0) g.delta[static_cast<int64_t>(qrow) * a.H + h] = drow;

  const int n_kv = um.n_kv, ntiles = (n_kv + BN - 1) / BN;
  const Loader ld(Kp, Vp, a.idx, rs, um.kv_begin, n_kv, tid);
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  if (ntiles > 0) ld.issue(0, st.k[0], st.v[0]);

  uint32_t k_off[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) k_off[kk] = (ql * CH + ((2 * kk + half) ^ swz<CH>(ql))) * 16;
  uint32_t v_off[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    v_off[db][0] = vt_offset<D>(db, 0, lane);
    v_off[db][1] = vt_offset<D>(db, 1, lane);
  }
  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

  auto tile = [&](int t, auto cur_tag) {
    constexpr int CUR = decltype(cur_tag)::value;
    wait_vmem<0>();
    tile_barrier();
    if (t + 1 < ntiles) ld.issue(t + 1, st.k[(CUR + 1) % NS], st.v[(CUR + 1) % NS]);
    const char* sk = reinterpret_cast<const char*>(st.k[CUR]);
    const char* sv = reinterpret_cast<const char*>(st.v[CUR]);
    // S^T = K Q^T and dP^T = V dO^T
    f32x16 sacc[KB], pacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) { sacc[kb] = f32x16{}; pacc[kb] = f32x16{}; }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint32_t o = k_off[kk] + kb * 32 * CH * 16;
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(sk + o), qf[kk], sacc[kb], 0, 0, 0);
        pacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(sv + o), df[kk], pacc[kb], 0, 0, 0);
      }
    if ((t + 1) * BN > n_kv) {   // keys past the list: P = 0
      const int lim = n_kv - t * BN - 4 * half;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
          sacc[kb][r] += __int_as_float(~((c - lim) >> 31) & static_cast<int>(0xff800000u));
        }
    }
    // dS^T = P^T (dP^T - delta), into sacc
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], sl2, -lse2));
        sacc[kb][r] = p * (pacc[kb][r] - drow);
      }
    // dq^T += K^T dS^T (K^T read transposed from LDS, in dS^T's key order)
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
      const int kb = ks >> 1, s8 = (ks & 1) * 8;
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = static_cast<__bf16>(sacc[kb][s8 + j]);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            read_vt(sk + ks * 16 * CH * 16, v_off[db][0], v_off[db][1]), pf, dqacc[db], 0, 0, 0);
    }
  };
  for (int t = 0; t < ntiles; t += NS) {
    tile(t, C0{});
    if (t + 1 < ntiles) tile(t + 1, C1{});
  }

  // The row's addresses again from an opaque copy of its index: otherwise the compiler
  // forms them before the key loop and keeps them (in scratch, at d = 128) until here.
  int qrow_e = qrow;
  asm volatile("" : "+v"(qrow_e));
  const int64_t ebase = static_cast<int64_t>(qrow_e) * rs;
  // a candidate reads its own key too: its term of dq, and the only gradient its own
  // key and value receive
  u16* dqp = static_cast<u16*>(g.dq) + h * D;
  if (qpos >= um.cand_rel) {
    const u16* KSp = static_cast<const u16*>(a.k_self) + h * D;
    const u16* VSp = static_cast<const u16*>(a.v_self) + h * D;
    // q and dO as opaque copies too, so that their float forms from before the loop (the
    // delta dot product) are not kept for these products
    bf16x8 qe[KK], de[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      v4i32 wq = __builtin_bit_cast(v4i32, qf[kk]), wd = __builtin_bit_cast(v4i32, df[kk]);
      asm volatile("" : "+v"(wq), "+v"(wd));
      qe[kk] = __builtin_bit_cast(bf16x8, wq);
      de[kk] = __builtin_bit_cast(bf16x8, wd);
    }
    float sraw = 0.f, dp = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      sraw = dot8(qe[kk], load8(KSp + ebase + 16 * kk + 8 * half), sraw);
      dp = dot8(de[kk], load8(VSp + ebase + 16 * kk + 8 * half), dp);
    }
    const float p = __builtin_amdgcn_exp2f(fmaf(halves_sum(sraw), sl2, -lse2));
    const float ds = p * (halves_sum(dp) - drow);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const uint2 kw = *reinterpret_cast<const uint2*>(KSp + ebase + db * 32 + 8 * gg + 4 * half);
        dqacc[db][4 * gg + 0] = fmaf(ds, bf16_lo(kw.x), dqacc[db][4 * gg + 0]);
        dqacc[db][4 * gg + 1] = fmaf(ds, bf16_hi(kw.x), dqacc[db][4 * gg + 1]);
        dqacc[db][4 * gg + 2] = fmaf(ds, bf16_lo(kw.y), dqacc[db][4 * gg + 2]);
        dqacc[db][4 * gg + 3] = fmaf(ds, bf16_hi(kw.y), dqacc[db][4 * gg + 3]);
      }
    if (qvalid) {
      u16* dkp = static_cast<u16*>(g.dk_self) + h * D + ebase;
      u16* dvp = static_cast<u16*>(g.dv_self) + h * D + ebase;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        store8(dkp + 16 * kk + 8 * half, qe[kk], g.scale * ds);   // dk_c = scale ds q_c
        store8(dvp + 16 * kk + 8 * half, de[kk], p);              // dv_c = p dO_c
      }
    }
  }
  if (qvalid) store_acc_row<DB>(dqp + ebase, dqacc, g.scale, half);
}

template <int D, int BN>
__global__ __launch_bounds__(kBwdWaves * 64, 2) void k_bwd_dq(BwdArgs g) {
  __shared__ __attribute__((aligned(16))) u16 k0[BN * D], k1[BN * D], v0[BN * D], v1[BN * D];
  const Stages st{{k0, k1, k0, k1}, {v0, v1, v0, v1}};
  int2 it;
  UserMeta um;
  bool indexed;
  const int subs = g.bm / kBwdRows, w = xcd_item(blockIdx.x);
  if (!fetch_item(g.a, g.bm, w / subs, it, um, indexed)) return;
  if (item_head(it) == kZeroHead) {   // padding rows: no gradient
    if (w % subs) return;
    AttnArgs z = g.a;
    z.o = g.dq;
    zero_padding_tile(z, um, item_tile(it), g.bm, g.a.H * D * 2, threadIdx.x, kBwdWaves * 64);
    z.o = g.dk;
    zero_padding_tile(z, um, item_tile(it), g.bm, g.a.H * D * 2, threadIdx.x, kBwdWaves * 64);
    z.o = g.dv;
    zero_padding_tile(z, um, item_tile(it), g.bm, g.a.H * D * 2, threadIdx.x, kBwdWaves * 64);
    return;
  }
  const int qt = item_tile(it) * subs + w % subs;
  if (qt * kBwdRows >= um.n_q) return;   // the item's last sub-tile may hold no rows
  if (indexed && !um.kv_direct) dq_item<D, BN, true>(g, item_head(it), qt, um, indexed, st);
  else dq_item<D, BN, false>(g, item_head(it), qt, um, indexed, st);
}

// --------------------------------------------------------------------------- dk, dv

// KEY_IDX: the key list goes through idx; QRY_IDX: the query list does (an indexed plan)
template <int D, int BQ, bool KEY_IDX, bool QRY_IDX, bool VLDS>
__device__ __forceinline__ void dkdv_item(const BwdArgs& g, int h, int kt, const UserMeta& um,
                                          const Stages& st, float* const (&ls)[2], u16* vblock) {
  constexpr int NS = 2, QB = BQ / kQw, kThreads = kBwdWaves * 64;
  static_assert(BQ % kQw == 0, "query tile");
  constexpr bool indexed = QRY_IDX;
  using Loader = KvLoader<D, BQ, kThreads, QRY_IDX>;     // query rows (Q and dO) of one tile
  constexpr int CH = D / 8, KK = D / 16, DB = D / 32;
  const AttnArgs& a = g.a;
  const int n_kv = um.n_kv, n_q = um.n_q;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, ql = lane & 31;
  const int64_t rs = static_cast<int64_t>(a.H) * D;
  const u16* Qp = static_cast<const u16*>(a.q) + h * D;
  const u16* Kp = static_cast<const u16*>(a.k) + h * D;
  const u16* Vp = static_cast<const u16*>(a.v) + h * D;
  const u16* DOp = static_cast<const u16*>(g.dout) + h * D;
  const float sl2 = a.scale_log2;

  // this lane's key (one key column per lane) and its K, V operands
  const int kpos = kt * kBwdRows + wave * kQw + ql;
  const bool kvalid = kpos < n_kv;
  const int ke = um.kv_begin + min(kpos, n_kv - 1);
  const int krow = KEY_IDX ? a.idx[ke] : ke;
  const int64_t kbase = static_cast<int64_t>(krow) * rs;
  // V operands: in registers, or (VLDS, to leave registers to the two accumulators)
  // read per use from the item's V rows staged in LDS once
  bf16x8 kf[KK], vf[VLDS ? 1 : KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    kf[kk] = load8(Kp + kbase + 16 * kk + 8 * half);
    if constexpr (!VLDS) vf[kk] = load8(Vp + kbase + 16 * kk + 8 * half);
  }
  if constexpr (VLDS) {
    const KvLoader<D, kBwdRows, kThreads, KEY_IDX> vl(Kp, Vp, a.idx, rs, um.kv_begin, n_kv, tid);
    vl.issue_v(kt, vblock);
  }

  // query tiles of BQ rows: Q and dO rows, and the rows' lse and delta (per 32-row block,
  // lanes 0-31 and 32-63 of one 4-byte load per wave; every wave loads the same bytes)
  const Loader ld(Qp, DOp, a.idx, rs, um.q_begin, n_q, tid);
  const int nqt = (n_q + BQ - 1) / BQ;
  auto issue = [&](int t, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    ld.issue(t, st.k[S], st.v[S]);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int e = um.q_begin + min(t * BQ + qb * kQw + ql, n_q - 1);
      const int64_t r = indexed ? a.idx[e] : e;
      const float* src = (half ? static_cast<const float*>(g.delta) : g.lse) + r * a.H + h;
      lds_dma_global4(src, __builtin_amdgcn_readfirstlane(lds_address(ls[S] + 64 * qb)));
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  if (nqt > 0) issue(0, C0{});   // a candidate-only user may have keys but no queries

  uint32_t q_off[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) q_off[kk] = (ql * CH + ((2 * kk + half) ^ swz<CH>(ql))) * 16;
  uint32_t t_off[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    t_off[db][0] = vt_offset<D>(db, 0, lane);
    t_off[db][1] = vt_offset<D>(db, 1, lane);
  }
  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) { dkacc[db] = f32x16{}; dvacc[db] = f32x16{}; }

  auto tile = [&](int t, auto cur_tag) {
    constexpr int CUR = decltype(cur_tag)::value;
    wait_vmem<0>();
    tile_barrier();
    if (t + 1 < nqt) issue(t + 1, std::integral_constant<int, (CUR + 1) % NS>{});
    const char* sq = reinterpret_cast<const char*>(st.k[CUR]);
    const char* sd = reinterpret_cast<const char*>(st.v[CUR]);
    const LDS_AS float* sl = (const LDS_AS float*)ls[CUR];
    // S = Q K^T and dP = dO V^T (rows: queries of this tile, column: this lane's key)
    f32x16 sacc[QB], pacc[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) { sacc[qb] = f32x16{}; pacc[qb] = f32x16{}; }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8 vop;
      if constexpr (VLDS)
        vop = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(vblock) + q_off[kk] +
                                               wave * kQw * CH * 16);
      else
        vop = vf[kk];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const uint32_t o = q_off[kk] + qb * kQw * CH * 16;
        sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(sq + o), kf[kk],
                                                           sacc[qb], 0, 0, 0);
        pacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(sd + o), vop,
                                                           pacc[qb], 0, 0, 0);
      }
    }
    if ((t + 1) * BQ > n_q) {   // query rows past the list: P = 0
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int lim = n_q - t * BQ - qb * kQw - 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 8 * (r >> 2) + (r & 3);
          sacc[qb][r] += __int_as_float(~((c - lim) >> 31) & static_cast<int>(0xff800000u));
        }
      }
    }
    // P = exp(scale s - lse) and dS = P (dP - delta), per query row 8(r/4) + 4 half + r%4
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 lv = *(const LDS_AS f32x4*)(sl + 64 * qb + 8 * gq + 4 * half);
        const f32x4 dv4 = *(const LDS_AS f32x4*)(sl + 64 * qb + 32 + 8 * gq + 4 * half);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * gq + u;
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[qb][r], sl2, -lv[u] * kLog2e));
          sacc[qb][r] = p;
          pacc[qb][r] = p * (pacc[qb][r] - dv4[u]);
        }
      }
    // dv^T += dO^T P and dk^T += Q^T dS (dO^T, Q^T read transposed, in P's row order)
#pragma unroll
    for (int ks = 0; ks < BQ / 16; ++ks) {
      const int qb = ks >> 1, s8 = (ks & 1) * 8;
      bf16x8 pf, sf;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pf[j] = static_cast<__bf16>(sacc[qb][s8 + j]);
        sf[j] = static_cast<__bf16>(pacc[qb][s8 + j]);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            read_vt(sd + ks * 16 * CH * 16, t_off[db][0], t_off[db][1]), pf, dvacc[db], 0, 0, 0);
        dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            read_vt(sq + ks * 16 * CH * 16, t_off[db][0], t_off[db][1]), sf, dkacc[db], 0, 0, 0);
      }
    }
  };
  for (int t = 0; t < nqt; t += NS) {
    tile(t, C0{});
    if (t + 1 < nqt) tile(t + 1, C1{});
  }
  if (kvalid) {
    // the row's address again from an opaque copy of its index (not kept through the loop)
    int krow_e = krow;
    asm volatile("" : "+v"(krow_e));
    const int64_t ebase = static_cast<int64_t>(krow_e) * rs;
    store_acc_row<DB>(static_cast<u16*>(g.dk) + h * D + ebase, dkacc, g.scale, half);
    store_acc_row<DB>(static_cast<u16*>(g.dv) + h * D + ebase, dvacc, 1.f, half);
  }
}

template <int D>
__global__ __launch_bounds__(kBwdWaves * 64, 2) void k_bwd_dkdv(BwdArgs g) {
  constexpr bool VLDS = D >= RR_BWD_VLDS_MIN_D;   // the V operands of the item's 128 keys from LDS
  constexpr int BQ = D == 64 ? RR_BWD_DKDV_BQ64 : kQw;   // query rows per tile
  __shared__ __attribute__((aligned(16))) u16 q0[BQ * D], q1[BQ * D], d0[BQ * D], d1[BQ * D];
  __shared__ __attribute__((aligned(16))) u16 vb[VLDS ? kBwdRows * D : 8];
  __shared__ __attribute__((aligned(16))) float l0[2 * BQ], l1[2 * BQ];
  const Stages st{{q0, q1, q0, q1}, {d0, d1, d0, d1}};
  float* const ls[2] = {l0, l1};
  int2 it;
  UserMeta um;
  bool indexed;
  const int subs = g.bm / kBwdRows, w = xcd_item(blockIdx.x);
  if (!fetch_item(g.a, g.bm, w / subs, it, um, indexed)) return;
  if (item_head(it) == kZeroHead) return;
  const int kt = item_tile(it) * subs + w % subs;
  if (kt * kBwdRows >= um.n_kv) return;   // no keys in this tile
  if (!indexed) dkdv_item<D, BQ, false, false, VLDS>(g, item_head(it), kt, um, st, ls, vb);
  else if (um.kv_direct) dkdv_item<D, BQ, false, true, VLDS>(g, item_head(it), kt, um, st, ls, vb);
  else dkdv_item<D, BQ, true, true, VLDS>(g, item_head(it), kt, um, st, ls, vb);
}

template <int D>
hipError_t go(const BwdArgs& gq, int64_t grid_q, const BwdArgs& gk, int64_t grid_k, hipStream_t s) {
  constexpr int BN = D == 128 ? RR_BWD_DQ_BN128 : RR_BWD_DQ_BN64;   // key tile of k_bwd_dq (register budget)
  hipError_t e;
  if constexpr (D == 64)
    e = grid_q <= RR_BWD_SMALL_GRID ? launch1(k_bwd_dq<D, 64>, grid_q, kBwdWaves * 64, s, gq)
                                    : launch1(k_bwd_dq<D, BN>, grid_q, kBwdWaves * 64, s, gq);
  else
    e = launch1(k_bwd_dq<D, BN>, grid_q, kBwdWaves * 64, s, gq);
  if (e != hipSuccess) return e;
  return launch1(k_bwd_dkdv<D>, grid_k, kBwdWaves * 64, s, gk);
}

}  // namespace

hipError_t launch_attn_bwd(const AttnArgs& aq, int bm_q, int64_t grid_q, const AttnArgs& ak, int bm_k,
                           int64_t grid_k, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           void* dk_self, void* dv_self, float* delta, float scale, int d, hipStream_t s) {
  if (bm_q % kBwdRows != 0 || bm_k % kBwdRows != 0) return hipErrorInvalidValue;
  BwdArgs gq{};
  gq.dout = dout; gq.lse = lse; gq.dq = dq; gq.dk = dk; gq.dv = dv; gq.delta = delta;
  gq.dk_self = dk_self; gq.dv_self = dv_self; gq.scale = scale;
  BwdArgs gk = gq;
  gq.a = aq; gq.bm = bm_q;
  gk.a = ak; gk.bm = bm_k;
  // one workgroup per 128-row sub-tile of every item
  grid_q *= bm_q / kBwdRows;
  grid_k *= bm_k / kBwdRows;
  switch (d) {
    case 64: return go<64>(gq, grid_q, gk, grid_k, s);
    case 128: return go<128>(gq, grid_q, gk, grid_k, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rr
