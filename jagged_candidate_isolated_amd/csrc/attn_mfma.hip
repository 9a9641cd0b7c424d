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
#include <type_traits>

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

// V^T operand of the PV product: eight keys of one V column per lane, read with two
// transposed LDS loads.  Within each 16-lane group the transposed load returns, in
// lane j, element j%4 of the 8-byte pieces addressed by lanes 4k + j/4 (k = 0..3); so
// lane s of a group addresses row (key) 4*half + s/4 at columns 4*(s%4)..+3 of the
// group's 16 columns, and receives one column, four keys.  vt_offset() gives the
// byte offset of that piece for k-step 0; k-step ks adds ks * 16 rows.
template <int D>
__device__ __forceinline__ uint32_t vt_offset(int db, int part, int lane) {
  constexpr int CH = D / 8;
  const int s = lane & 15, grp = (lane >> 4) & 1, half = lane >> 5;
  const int col = db * 32 + 16 * grp + 4 * (s & 3);      // first of 4 columns (elements)
  const int c = col >> 3, sub = (col & 7) * 2;           // 16-byte chunk, byte offset in it
  const int row = 8 * part + 4 * half + (s >> 2);        // swz() ignores multiples of 16 rows
  return static_cast<uint32_t>((row * CH + (c ^ swz<CH>(row))) * 16 + sub);
}

__device__ __forceinline__ bf16x8 read_vt(const char* sv, uint32_t off0, uint32_t off1) {
  const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(sv + off0));
  const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(sv + off1));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 w = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  return __builtin_bit_cast(bf16x8, w);
}

// Max of three.  This file is compiled without NaN support (no value here is ever
// NaN: scores are finite or -inf, and no expression subtracts two infinities), so
// the compiler emits v_max3_f32 directly instead of first canonicalising each MFMA
// result for IEEE maxNum semantics.
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Buffer resource of a raw byte range (gfx9 dword 3: 32-bit data, no swizzle); loads
// past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// Rows keep their running maximum as the softmax reference until a tile's maximum
// exceeds it by more than 2^kLazyRescale (log2 units); only then are the row's
// accumulator and sum rescaled.  Probabilities stay below 2^kLazyRescale, far from
// any overflow, and each row decides for itself, so a row's result never depends
// on the other rows of its wave.
#ifndef RR_LAZY_RESCALE
#define RR_LAZY_RESCALE 8.f
#endif
constexpr float kLazyRescale = RR_LAZY_RESCALE;

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

  // Direct-to-LDS loads of key/value tile t into buffer t & 1.  Load i of wave w fills
  // LDS slots (w*LOADS + i)*64 + lane; slot -> (row, chunk position) -> global chunk.
  // A full tile of a plain row list is one byte range: a buffer resource whose per-lane
  // offsets never change between tiles.  The partial last tile, and row lists through
  // idx[], load per row with the row index clamped into the key list (the last tile
  // masks the repeated rows), so every byte that reaches LDS is a real key or value.
  int ld_row[LOADS];
  uint32_t ld_off[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int slot = (wave * LOADS + i) * 64 + lane;
    const int row = slot / CH, p = slot % CH;
    ld_row[i] = row;
    ld_off[i] = static_cast<uint32_t>(row * rs * 2 + (p ^ swz<CH>(row)) * 16);
  }
  const int64_t user_bytes = n_kv > 0 ? (static_cast<int64_t>(n_kv - 1) * rs + D) * 2 : 0;
#ifdef RR_NO_RANGED_LOADS
  const bool ranged = false;
#else
  const bool ranged = !INDEXED && user_bytes + static_cast<int64_t>(BN) * rs * 2 < (int64_t(1) << 31);
#endif
  const char* k_user = reinterpret_cast<const char*>(Kp) + static_cast<int64_t>(um.kv_begin) * rs * 2;
  const char* v_user = reinterpret_cast<const char*>(Vp) + static_cast<int64_t>(um.kv_begin) * rs * 2;
  auto issue_tile = [&](int t) {
    u16* dk = s_k + (t & 1) * TILE;
    u16* dv = s_v + (t & 1) * TILE;
    if (ranged && (t + 1) * BN <= n_kv) {
      // a full tile: the descriptor starts at the tile and ends at the user's last key
      // byte, so the range check also keeps every load inside the user's keys
      const int64_t tile_off = static_cast<int64_t>(t) * BN * rs * 2;
      const uint32_t left = static_cast<uint32_t>(user_bytes - tile_off);
      const __amdgpu_buffer_rsrc_t k_rsrc = byte_range(k_user + tile_off, left);
      const __amdgpu_buffer_rsrc_t v_rsrc = byte_range(v_user + tile_off, left);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int lds_off = (wave * LOADS + i) * 64 * 8;         // elements; one load = 1 KiB
        __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (LDS_AS void*)(dk + lds_off), 16,
                                                 static_cast<int>(ld_off[i]), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(v_rsrc, (LDS_AS void*)(dv + lds_off), 16,
                                                 static_cast<int>(ld_off[i]), 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int lds_off = (wave * LOADS + i) * 64 * 8;
        const int row = ld_row[i];
        const int e = um.kv_begin + min(t * BN + row, n_kv - 1);   // clamp the tail into the list
        const int64_t g = static_cast<int64_t>(INDEXED ? a.idx[e] : e) * rs * 2 +
                          (ld_off[i] - static_cast<uint32_t>(row * rs * 2));
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(Kp) + g,
                                         (LDS_AS void*)(dk + lds_off), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(Vp) + g,
                                         (LDS_AS void*)(dv + lds_off), 16, 0, 0);
      }
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

  auto tile = [&](int t, auto buf_tag, auto tail_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr bool TAIL = decltype(tail_tag)::value;
    // tile t has landed (this wave's loads) and is visible (every wave's, after the
    // barrier); the barrier also tells that every wave is done with the other buffer
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntiles) issue_tile(t + 1);   // overlaps this tile's math
    const char* sk = reinterpret_cast<const char*>(s_k + BUF * TILE);
    const char* sv = reinterpret_cast<const char*>(s_v + BUF * TILE);

    // S^T = K Q^T for this wave's 32 queries; the KB accumulator chains interleave
    f32x16 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sk + k_off[kk] + kb * 32 * CH * 16);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc[kb], 0, 0, 0);
      }
    if constexpr (TAIL) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = t * BN + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (j >= n_kv) sacc[kb][r] = -INFINITY;
        }
    }
    // online softmax, one query per lane (key halves split across the lane halves)
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
    const float tmax = fmaxf(mx[0], __shfl_xor(mx[0], 32)) * sl2;
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
    // O^T += V^T P^T
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
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  const int full_tiles = (n_kv % BN) ? ntiles - 1 : ntiles;
  int t = 0;
  for (; t + 1 < full_tiles; t += 2) {
    tile(t, B0{}, std::false_type{});
    tile(t + 1, B1{}, std::false_type{});
  }
  if (t < full_tiles) {          // an odd number of full tiles: the last one is even
    tile(t, B0{}, std::false_type{});
    ++t;
  }
  if (t < ntiles) {              // the partial tail tile
    if (t & 1) tile(t, B1{}, std::true_type{});
    else tile(t, B0{}, std::true_type{});
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

// XCD-aware item order.  Workgroup i runs on XCD i % kXcds (the dispatcher deals
// workgroups out round-robin), each XCD with its own L2.  Chunks of kXcdChunk
// consecutive items -- query tiles of one user and head, which read the same keys
// and values -- go to one XCD together, chunk c to XCD c % kXcds, so a K/V tile
// comes into that L2 once and serves the whole chunk; chunks still start in the
// work list's longest-first order.  The grid is a multiple of kXcds * kXcdChunk,
// which makes the map a permutation.
__device__ __forceinline__ int xcd_item(int wg) {
  const int x = wg % kXcds, slot = wg / kXcds;
  return ((slot / kXcdChunk) * kXcds + x) * kXcdChunk + slot % kXcdChunk;
}

template <int D, int BN>
__global__ __launch_bounds__(kThreads, 2) void k_attn_mfma(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) u16 s_k[2 * BN * D];   // double-buffered K tiles
  __shared__ __attribute__((aligned(16))) u16 s_v[2 * BN * D];   // double-buffered V tiles
  if (!plan_matches(a, kBm)) return;
  const int item = xcd_item(blockIdx.x);
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
