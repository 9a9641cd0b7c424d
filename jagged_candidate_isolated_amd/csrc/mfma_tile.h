// Device helpers shared by the bf16 MFMA attention kernels (gfx950,
// v_mfma_f32_32x32x16_bf16): operand layouts, the swizzled LDS tile layout,
// direct-to-LDS K/V tile loads, counted waits and the tile barrier.
#pragma once

#include <type_traits>

#include "rr_internal.h"

namespace rr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef short v4i16 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kQw = 32;   // query rows of one 32x32 MFMA block

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

// the same read at two LDS byte addresses
__device__ __forceinline__ bf16x8 read_vt_lds(uint32_t a0, uint32_t a1) {
  const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(uintptr_t)a0);
  const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(uintptr_t)a1);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 w = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  return __builtin_bit_cast(bf16x8, w);
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

// Max / sum of a value and its copy in the other half of the wave (lanes l and
// l ^ 32): v_permlane32_swap exchanges the halves of its two operands, so with both
// operands x the two results hold x[l] and x[l ^ 32] in some order in every lane.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource of a raw byte range (gfx9 layout: base address, stride 0, size in
// bytes, dword 3 = 32-bit data, no swizzle); loads past `bytes` return zero.
typedef int v4i32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i32 byte_range(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const v4i32 r = {static_cast<int>(p), static_cast<int>((p >> 32) & 0xffff), static_cast<int>(bytes),
                   0x00020000};
  return r;
}

// Direct-to-LDS 16-byte loads: lane l writes its 16 bytes to LDS address
// lds_addr + 16 l; no register receives data.  They are written as assembly so the
// compiler's wait-count pass does not track them: that pass, unable to tell the
// stage being filled from the stage being read, would wait for every load in
// flight before LDS reads and so empty the tile pipeline.  The kernels order these
// loads themselves, with counted waits (wait_vmem) before each tile's barrier.
// `lds_addr` is wave-uniform; m0 carries it to the load.  m0 is a register the
// compiler reserves, so each block saves it, sets it (one wait state before the
// load reads it) and restores it once the load has issued (the load takes m0 at
// issue).
__device__ __forceinline__ void lds_dma_buffer16(v4i32 rsrc, uint32_t voffset, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voffset), "s"(rsrc)
      : "memory");
}
__device__ __forceinline__ void lds_dma_global16(const void* gptr, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(gptr)
      : "memory");
}

// 4-byte variant: lane l writes its 4 bytes to lds_addr + 4 l.
__device__ __forceinline__ void lds_dma_global4(const void* gptr, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(gptr)
      : "memory");
}

// LDS address (byte offset in the workgroup's LDS) of a __shared__ location.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS const void*)p));
}

// Wait until at most N vector-memory operations of this wave are outstanding (they
// retire in issue order); LDS and scalar counters are not waited on.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence.  The tile pipeline needs no fence: each
// wave waits for its own direct-to-LDS loads (wait_vmem) before the barrier, and
// every LDS read of the previous tile has been consumed by an MFMA before its wave
// reaches the barrier.  (__syncthreads() would also wait for every load in flight,
// i.e. for the tiles being prefetched.)  The signal fences only keep the compiler
// from moving memory operations across the barrier.
__device__ __forceinline__ void tile_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// LDS stages of the K/V pipeline, one object per stage so the compiler can tell
// which stage a direct-to-LDS load writes and which stage an operand read uses.
struct Stages {
  u16* k[4];
  u16* v[4];
  double* inv_freq;   // the rotary inverse frequencies of the D/2 feature pairs (when rotating)
};

// Rows keep their running maximum as the softmax reference until a tile's maximum
// exceeds it by more than 2^kLazyRescale (log2 units); only then are the row's
// accumulator and sum rescaled.  Probabilities stay below 2^kLazyRescale, far from
// any overflow, and each row decides for itself, so a row's result never depends
// on the other rows of its wave.
constexpr float kLazyRescale = 8.f;

// Slack on the Cauchy-Schwarz bound of a row's scores (q.k <= |q| |k|) against the
// rounding of the computed quantities: the fp32 score of a d <= 128 product of bf16
// features exceeds the exact one by at most a relative d * 2^-24 of |q| |k|, and the
// squared norms, square root and products of the bound lose a few times that; 2^-7
// covers both with room to spare.
constexpr float kBoundSlack = 1.0078125f;

// Direct-to-LDS loads of K/V tiles (BN keys of D bf16) by NT threads.  Load i of
// wave w fills LDS slots (w*LOADS + i)*64 + lane; slot -> (row, chunk position) ->
// global chunk.  A full tile of a contiguous key list is one byte range: a buffer
// resource whose per-lane offsets never change between tiles.  The partial last
// tile, and key lists through idx[], load per row with the row index clamped into
// the list (the last tile masks the repeated rows), so every byte reaching LDS is a
// real key.
template <int D, int BN, int NT, bool KEY_IDX>
struct KvLoader {
  static constexpr int CH = D / 8;
  static constexpr int LOADS = BN * D * 2 / (NT * 16);   // loads per thread per K (or V) tile
  static constexpr int LPT = 2 * LOADS;                   // vector-memory operations per tile
  static_assert(LOADS >= 1 && BN * D * 2 % (NT * 16) == 0, "tile shape");

  int ld_row[LOADS];
  uint32_t ld_off[LOADS];
  const u16* kp;
  const u16* vp;
  const char* k_user;
  const char* v_user;
  const int32_t* idx;
  int64_t user_bytes;
  int64_t rs2;      // bytes per row
  int kv_begin, n_kv, lds_base;
  bool ranged;

  __device__ __forceinline__ KvLoader(const u16* K, const u16* V, const int32_t* idx_, int64_t rs,
                                      int kv_begin_, int n_kv_, int tid)
      : kp(K), vp(V), idx(idx_), rs2(rs * 2), kv_begin(kv_begin_), n_kv(n_kv_) {
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int slot = (wave * LOADS + i) * 64 + lane;
      const int row = slot / CH, p = slot % CH;
      ld_row[i] = row;
      ld_off[i] = static_cast<uint32_t>(row * rs2 + (p ^ swz<CH>(row)) * 16);
    }
    lds_base = wave * LOADS * 64 * 8;   // elements; one load fills 1 KiB
    user_bytes = n_kv > 0 ? static_cast<int64_t>(n_kv - 1) * rs2 + D * 2 : 0;
    ranged = !KEY_IDX && user_bytes + static_cast<int64_t>(BN) * rs2 < (int64_t(1) << 31);
    k_user = reinterpret_cast<const char*>(K) + static_cast<int64_t>(kv_begin) * rs2;
    v_user = reinterpret_cast<const char*>(V) + static_cast<int64_t>(kv_begin) * rs2;
  }

  // tile t into the LDS buffers dk / dv
  __device__ __forceinline__ void issue(int t, u16* dk, u16* dv) const {
    const uint32_t lk = __builtin_amdgcn_readfirstlane(lds_address(dk + lds_base));
    const uint32_t lv = __builtin_amdgcn_readfirstlane(lds_address(dv + lds_base));
    if (ranged && (t + 1) * BN <= n_kv) {
      // a full tile: the descriptor starts at the tile and ends at the user's last key
      // byte, so the range check also keeps every load inside the user's keys
      const int64_t tile_off = static_cast<int64_t>(t) * BN * rs2;
      const uint32_t left = static_cast<uint32_t>(user_bytes - tile_off);
      const v4i32 k_rsrc = byte_range(k_user + tile_off, left);
      const v4i32 v_rsrc = byte_range(v_user + tile_off, left);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        lds_dma_buffer16(k_rsrc, ld_off[i], lk + i * 1024);
        lds_dma_buffer16(v_rsrc, ld_off[i], lv + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int row = ld_row[i];
        const int e = kv_begin + min(t * BN + row, n_kv - 1);   // clamp the tail into the list
        const int64_t g = static_cast<int64_t>(KEY_IDX ? idx[e] : e) * rs2 +
                          (ld_off[i] - static_cast<uint32_t>(row * rs2));
        lds_dma_global16(reinterpret_cast<const char*>(kp) + g, lk + i * 1024);
        lds_dma_global16(reinterpret_cast<const char*>(vp) + g, lv + i * 1024);
      }
    }
  }

  // the value rows of tile t only, into dv
  __device__ __forceinline__ void issue_v(int t, u16* dv) const {
    const uint32_t lv = __builtin_amdgcn_readfirstlane(lds_address(dv + lds_base));
    if (ranged && (t + 1) * BN <= n_kv) {
      const int64_t tile_off = static_cast<int64_t>(t) * BN * rs2;
      const v4i32 v_rsrc = byte_range(v_user + tile_off, static_cast<uint32_t>(user_bytes - tile_off));
#pragma unroll
      for (int i = 0; i < LOADS; ++i) lds_dma_buffer16(v_rsrc, ld_off[i], lv + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int row = ld_row[i];
        const int e = kv_begin + min(t * BN + row, n_kv - 1);
        const int64_t g = static_cast<int64_t>(KEY_IDX ? idx[e] : e) * rs2 +
                          (ld_off[i] - static_cast<uint32_t>(row * rs2));
        lds_dma_global16(reinterpret_cast<const char*>(vp) + g, lv + i * 1024);
      }
    }
  }
};

// Wait until this wave's loads of the tiles issued before the last `later` ones
// have landed (later = 0, 1 or 2 tiles of LPT operations each).
template <int LPT>
__device__ __forceinline__ void wait_tiles(int later) {
  if (later >= 2) wait_vmem<2 * LPT>();
  else if (later == 1) wait_vmem<LPT>();
  else wait_vmem<0>();
}

// XCD-aware item order.  Workgroup i runs on XCD i % kXcds (the dispatcher deals
// workgroups out round-robin), each XCD with its own L2.  Chunks of C
// consecutive items -- query tiles of one user and head, which read the same keys
// and values -- go to one XCD together, chunk c to XCD c % kXcds, so a K/V tile
// comes into that L2 once and serves the whole chunk; chunks still start in the
// work list's longest-first order.  The grid is a multiple of kXcds * C,
// which makes the map a permutation.
template <int C = kXcdChunk>
__device__ __forceinline__ int xcd_item(int wg) {
  const int x = wg % kXcds, slot = wg / kXcds;
  return ((slot / C) * kXcds + x) * C + slot % C;
}

}  // namespace
}  // namespace rr
