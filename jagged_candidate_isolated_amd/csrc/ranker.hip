// The ranker's layer stack on the GPU: row norm, the projections (a bf16 MFMA GEMM
// with fused epilogues), the split of the hidden states into frozen history and
// candidates, and the host-side driver that runs full layers, the split and the
// candidate-only layers (Candidate isolation attention mask page, section
// "只更新候选的末尾层"), or a later request's candidates against the cached history
// keys and values of every layer.
//
// Each layer is a pre-norm attention block (the pages do not print the layer's
// inside; this is the reading taken):
//   h = rms_norm(x) * gain;  [q | k | v] = h W_qkv^T;  q, k rotated (right-anchored);
//   x += attention(q, k, v) W_o^T.
// x is float32, the projections' inputs and outputs bf16 with fp32 accumulation.
// Every kernel here computes each row from that row alone, in a fixed order, so a
// candidate's result does not depend on which other rows share the launch: a cached
// request reproduces the full request's candidate states bit for bit.
#include <cmath>

#include "mfma_tile.h"

namespace rr {
namespace {

// ------------------------------------------------------------------ row norm

// out[r] = bf16(x[r] / sqrt(mean(x[r]^2) + eps) * gain): one wave per row.
__global__ __launch_bounds__(256) void k_rms_norm(const float* x, const float* gain, u16* out, int M,
                                                  int D, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* xr = x + row * D;
  float ss = 0.f;
  for (int c = 4 * lane; c < D; c += 256) {
    const float4 v = *reinterpret_cast<const float4*>(xr + c);
    ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  u16* orow = out + row * D;
  for (int c = 4 * lane; c < D; c += 256) {
    const float4 v = *reinterpret_cast<const float4*>(xr + c);
    const float4 g = *reinterpret_cast<const float4*>(gain + c);
    *reinterpret_cast<uint2*>(orow + c) =
        make_uint2(pack_bf16(v.x * inv * g.x, v.y * inv * g.y), pack_bf16(v.z * inv * g.z, v.w * inv * g.w));
  }
}

// ------------------------------------------------------------------ GEMM

// C[m][n] = sum_k A[m][k] W[n][k]: A bf16 [M][K] (activations), W bf16 [N][K] (a
// projection, out x in).  One workgroup of WM x WN waves per (WM TM 32) x (WN TN 32)
// tile of C, each wave TM x TN blocks of 32 x 32; K in steps of 64 through two LDS
// stages filled by direct-to-LDS loads (the swizzled layout of the attention kernels,
// 8 chunks per row).  The MFMA takes W rows as its A operand and A rows as its B
// operand, so each lane ends up owning one row m of C with 16 of its columns per
// block: the epilogue writes 8-byte (bf16) or 16-byte (fp32) pieces of one row.  Rows
// past M are read as zero by the buffer range check and never written.  N must be a
// multiple of the tile's width and K of 64.
constexpr int kGk = 64, kGch = kGk / 8, kGn = 128;   // kGn: the N granularity every tile shape divides

struct GemmArgs {
  const u16* a;
  const u16* w;
  int M, N, K;
  int m_tiles, n_tiles;
  // epilogue 0: bf16 C split by columns into out[n / out_cols] ([M][out_cols] each,
  // NULL = not written); epilogue 1: res[m][n] += C[m][n] (float32 [M][N])
  u16* out[3];
  int out_cols;
  float* res;
};

template <int EPI, int WM, int WN, int TM, int TN, int NS>
__global__ __launch_bounds__(WM * WN * 64, (WM * WN >= 8 || (WM * WN == 4 && TM * TN == 4 && NS == 2)) ? 2 : 1)
    void k_gemm_bt(
    GemmArgs g) {
  constexpr int kThr = WM * WN * 64, BMt = WM * TM * 32, BNt = WN * TN * 32;
  constexpr int LA = BMt * kGch / kThr, LW = BNt * kGch / kThr;   // 16-byte loads per thread and K step
  static_assert(LA >= 1 && LW >= 1 && BMt * kGch % kThr == 0 && BNt * kGch % kThr == 0, "tile shape");
  static_assert(NS >= 2 && NS <= 4, "pipeline stages");
  // stages past NS are never referenced and take no LDS
  __shared__ __attribute__((aligned(16))) u16 a0[BMt * kGk], a1[BMt * kGk], a2[BMt * kGk], a3[BMt * kGk];
  __shared__ __attribute__((aligned(16))) u16 w0[BNt * kGk], w1[BNt * kGk], w2[BNt * kGk], w3[BNt * kGk];
  u16* const sa_[4] = {a0, a1, a2, a3};
  u16* const sw_[4] = {w0, w1, w2, w3};
  const int logical = xcd_item(blockIdx.x);
  const int mt = logical / g.n_tiles, nt = logical % g.n_tiles;
  if (mt >= g.m_tiles) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5;
  const int wm = wave % WM, wn = wave / WM;
  const int64_t m0 = static_cast<int64_t>(mt) * BMt, n0 = static_cast<int64_t>(nt) * BNt;
  const int rows = static_cast<int>(min<int64_t>(BMt, g.M - m0));
  const uint32_t rb = static_cast<uint32_t>(g.K) * 2;   // bytes per row of A and W

  // per-thread load slots: global byte offset of its 16-byte chunk (swizzled on the global side)
  uint32_t la_off[LA], lw_off[LW];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int slot = (wave * LA + i) * 64 + lane, row = slot / kGch, p = slot % kGch;
    la_off[i] = row * rb + (p ^ swz<kGch>(row)) * 16;
  }
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const int slot = (wave * LW + i) * 64 + lane, row = slot / kGch, p = slot % kGch;
    lw_off[i] = row * rb + (p ^ swz<kGch>(row)) * 16;
  }
  const char* a_base = reinterpret_cast<const char*>(g.a) + m0 * rb;
  const char* w_base = reinterpret_cast<const char*>(g.w) + n0 * rb;
  const uint32_t a_bytes = static_cast<uint32_t>(rows) * rb, w_bytes = BNt * rb;
  auto issue = [&](int t, u16* sa, u16* sw) {
    const uint32_t la = __builtin_amdgcn_readfirstlane(lds_address(sa) + wave * LA * 1024);
    const uint32_t lw = __builtin_amdgcn_readfirstlane(lds_address(sw) + wave * LW * 1024);
    const uint32_t k_off = static_cast<uint32_t>(t) * kGk * 2;
    const v4i32 ra = byte_range(a_base + k_off, a_bytes - k_off);
    const v4i32 rw = byte_range(w_base + k_off, w_bytes - k_off);
#pragma unroll
    for (int i = 0; i < LA; ++i) lds_dma_buffer16(ra, la_off[i], la + i * 1024);
#pragma unroll
    for (int i = 0; i < LW; ++i) lds_dma_buffer16(rw, lw_off[i], lw + i * 1024);
  };

  // operand reads: row r of a 32-row block, chunk 2 kk + half
  constexpr int TB = TM > TN ? TM : TN;
  uint32_t op_off[TB][kGk / 16];
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int kk = 0; kk < kGk / 16; ++kk) {
      const int r = b * 32 + (lane & 31);
      op_off[b][kk] = (r * kGch + ((2 * kk + half) ^ swz<kGch>(r))) * 16;
    }
  f32x16 acc[TN][TM];   // [n block][m block]
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x16{};

  const int nk = g.K / kGk;
  // steps 0 .. NS-2 in flight before the loop; step t + NS - 1 is issued after step t's
  // barrier into the stage step t - 1 used
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < nk) issue(t, sa_[t], sw_[t]);
  auto step = [&](int t, auto cur_tag) {
    constexpr int CUR = decltype(cur_tag)::value;
    // wait for step t's loads: the later steps already issued may stay in flight
    wait_tiles<LA + LW>(min(NS - 2, nk - 1 - t));
    tile_barrier();
    if (t + NS - 1 < nk) issue(t + NS - 1, sa_[(CUR + NS - 1) % NS], sw_[(CUR + NS - 1) % NS]);
    const char* ca = reinterpret_cast<const char*>(sa_[CUR]) + wm * TM * 32 * kGch * 16;
    const char* cw = reinterpret_cast<const char*>(sw_[CUR]) + wn * TN * 32 * kGch * 16;
#pragma unroll
    for (int kk = 0; kk < kGk / 16; ++kk) {
      bf16x8 wf[TN], af[TM];
#pragma unroll
      for (int b = 0; b < TN; ++b) wf[b] = *reinterpret_cast<const bf16x8*>(cw + op_off[b][kk]);
#pragma unroll
      for (int b = 0; b < TM; ++b) af[b] = *reinterpret_cast<const bf16x8*>(ca + op_off[b][kk]);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
    }
  };
  for (int t = 0; t < nk; t += NS) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nk) step(t + 1, std::integral_constant<int, 1 % NS>{});
    if constexpr (NS > 2)
      if (t + 2 < nk) step(t + 2, std::integral_constant<int, 2 % NS>{});
    if constexpr (NS > 3)
      if (t + 3 < nk) step(t + 3, std::integral_constant<int, 3 % NS>{});
  }

  // epilogue: lane owns row m of each m block, columns 8 gq + 4 half + (0..3) of each n block
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int64_t m = m0 + wm * TM * 32 + j * 32 + (lane & 31);
    if (m >= g.M) continue;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int64_t n = n0 + wn * TN * 32 + i * 32 + 8 * gq + 4 * half;
        const f32x16& c = acc[i][j];
        if constexpr (EPI == 0) {
          u16* dst = g.out[n / g.out_cols];
          if (dst)
            *reinterpret_cast<uint2*>(dst + m * g.out_cols + n % g.out_cols) =
                make_uint2(pack_bf16(c[4 * gq], c[4 * gq + 1]), pack_bf16(c[4 * gq + 2], c[4 * gq + 3]));
        } else {
          float4* p = reinterpret_cast<float4*>(g.res + m * g.N + n);
          float4 r = *p;
          r.x += c[4 * gq]; r.y += c[4 * gq + 1]; r.z += c[4 * gq + 2]; r.w += c[4 * gq + 3];
          *p = r;
        }
      }
  }
}

template <int WM, int WN, int TM, int TN, int NS>
hipError_t gemm_go(GemmArgs g, hipStream_t s) {
  constexpr int BMt = WM * TM * 32, BNt = WN * TN * 32;
  g.m_tiles = (g.M + BMt - 1) / BMt;
  g.n_tiles = g.N / BNt;
  const int64_t q = int64_t(kXcds) * kXcdChunk;
  const int64_t grid = (int64_t(g.m_tiles) * g.n_tiles + q - 1) / q * q;
  return g.res ? launch1(k_gemm_bt<1, WM, WN, TM, TN, NS>, grid, WM * WN * 64, s, g)
               : launch1(k_gemm_bt<0, WM, WN, TM, TN, NS>, grid, WM * WN * 64, s, g);
}

// ------------------------------------------------------------------ split

// Per-user history and candidate counts and their exclusive sums (one workgroup):
// hoff[b] = sum of (cand_start - offsets) before b, coff[b] = sum of
// (offsets[b+1] - cand_start) before b, hlen[b] = user b's history rows.
__global__ __launch_bounds__(256) void k_split_offsets(const int32_t* offsets, const int32_t* cand_start,
                                                       int B, int32_t* hoff, int32_t* coff, int32_t* hlen) {
  __shared__ int32_t sh[256], sc[256];
  const int tid = threadIdx.x;
  int32_t carry_h = 0, carry_c = 0;
  if (tid == 0) { hoff[0] = 0; coff[0] = 0; }
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    int32_t h = 0, c = 0;
    if (b < B) {   // the candidate start clamped into the user's rows
      const int32_t lo = offsets[b], hi = max(offsets[b + 1], lo), cs = min(max(cand_start[b], lo), hi);
      h = cs - lo;
      c = hi - cs;
    }
    sh[tid] = h; sc[tid] = c;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {   // inclusive scan
      const int32_t xh = tid >= o ? sh[tid - o] : 0, xc = tid >= o ? sc[tid - o] : 0;
      __syncthreads();
      sh[tid] += xh; sc[tid] += xc;
      __syncthreads();
    }
    if (b < B) {
      hoff[b + 1] = carry_h + sh[tid];
      coff[b + 1] = carry_c + sc[tid];
      hlen[b] = h;
    }
    carry_h += sh[255]; carry_c += sc[255];
    __syncthreads();
  }
}

__device__ __forceinline__ int owner_of(const int32_t* offsets, int B, int r) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Row r of src (row_bytes, a multiple of 16) goes to hist[hoff[b] + r - offsets[b]] if it
// precedes its user's candidate start, else to cand[coff[b] + r - cand_start[b]]; a NULL
// destination is skipped, and so is a destination row outside [0, Th) or [0, Tc) (data
// that breaks the layout contract).  One thread per 16-byte chunk.
__global__ __launch_bounds__(256) void k_split_rows(const char* src, int64_t row_bytes, const int32_t* offsets,
                                                    const int32_t* cand_start, const int32_t* hoff,
                                                    const int32_t* coff, int B, int T, char* hist, int Th,
                                                    char* cand, int Tc) {
  const int64_t chunks = row_bytes / 16, n = static_cast<int64_t>(T) * chunks;
  for (int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; e < n; e += int64_t(gridDim.x) * blockDim.x) {
    const int r = static_cast<int>(e / chunks);
    const int64_t c = e % chunks;
    const int b = owner_of(offsets, B, r);
    const int cs = min(max(cand_start[b], offsets[b]), offsets[b + 1]);
    const int64_t j = r < cs ? static_cast<int64_t>(hoff[b]) + r - offsets[b] : static_cast<int64_t>(coff[b]) + r - cs;
    char* const base = r < cs ? hist : cand;
    char* dst = (base && j >= 0 && j < (r < cs ? Th : Tc)) ? base + j * row_bytes : nullptr;
    if (dst)
      reinterpret_cast<uint4*>(dst)[c] = reinterpret_cast<const uint4*>(src + static_cast<int64_t>(r) * row_bytes)[c];
  }
}

// User-token rows: p[b] = min(max(user_tokens[b], 0), rows of user b's history block),
// poff = their exclusive sums (one workgroup).
__global__ __launch_bounds__(256) void k_prefix_offsets(const int32_t* user_tokens, const int32_t* hoff, int B,
                                                        int32_t* poff) {
  __shared__ int32_t sp[256];
  const int tid = threadIdx.x;
  int32_t carry = 0;
  if (tid == 0) poff[0] = 0;
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    const int32_t x = b < B ? min(max(user_tokens[b], 0), max(hoff[b + 1] - hoff[b], 0)) : 0;
    sp[tid] = x;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int32_t y = tid >= o ? sp[tid - o] : 0;
      __syncthreads();
      sp[tid] += y;
      __syncthreads();
    }
    if (b < B) poff[b + 1] = carry + sp[tid];
    carry += sp[255];
    __syncthreads();
  }
}

// Between the compact user-token rows (row j of user b: j in [poff[b], poff[b+1])) and
// the first rows of each user's block in a blocked tensor (row block[b] + j - poff[b]):
// gather (to_compact) or scatter.  Rows outside [0, n_compact) or [0, n_blocked) are
// skipped.  One thread per 16-byte chunk.
__global__ __launch_bounds__(256) void k_prefix_rows(char* compact, char* blocked, int64_t row_bytes,
                                                     const int32_t* block, const int32_t* poff, int B,
                                                     int n_compact, int n_blocked, int to_compact) {
  const int64_t chunks = row_bytes / 16, n = static_cast<int64_t>(n_compact) * chunks;
  for (int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; e < n; e += int64_t(gridDim.x) * blockDim.x) {
    const int j = static_cast<int>(e / chunks);
    const int64_t c = e % chunks;
    const int b = owner_of(poff, B, j);
    const int64_t r = static_cast<int64_t>(block[b]) + j - poff[b];
    if (j >= poff[b + 1] || r < 0 || r >= n_blocked) continue;
    uint4* cp = reinterpret_cast<uint4*>(compact + static_cast<int64_t>(j) * row_bytes) + c;
    uint4* bp = reinterpret_cast<uint4*>(blocked + r * row_bytes) + c;
    if (to_compact) *cp = *bp;
    else *bp = *cp;
  }
}

int64_t grid_of(int64_t n, int64_t per) {
  const int64_t g = (n + per - 1) / per;
  return g < 1 ? 1 : (g > (int64_t(1) << 20) ? (int64_t(1) << 20) : g);
}

}  // namespace

hipError_t launch_rms_norm(const float* x, const float* gain, void* out, int M, int D, float eps, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  void* args[] = {&x, &gain, &out, &M, &D, &eps};
  return hipLaunchKernel(reinterpret_cast<const void*>(k_rms_norm), dim3(static_cast<unsigned>((M + 3) / 4)),
                         dim3(256), args, 0, s);
}

// bf16 C = A W^T into out[0..2] by column blocks of out_cols, or (res != NULL) res += C.
#ifndef RR_GEMM_STAGES
#define RR_GEMM_STAGES 2
#endif
hipError_t launch_gemm_bt(const void* a, const void* w, int M, int N, int K, void* const out[3], int out_cols,
                          float* res, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (N % kGn || K % kGk || K <= 0) return hipErrorInvalidValue;
  if (!res && (out_cols <= 0 || out_cols % kGn || N > 3 * int64_t(out_cols))) return hipErrorInvalidValue;
  GemmArgs g{};
  g.a = static_cast<const u16*>(a);
  g.w = static_cast<const u16*>(w);
  g.M = M; g.N = N; g.K = K;
  for (int i = 0; i < 3; ++i) g.out[i] = out ? static_cast<u16*>(out[i]) : nullptr;
  g.out_cols = out_cols;
  g.res = res;
  // Large products: 256 x 256 tiles of 8 waves, 128 x 64 each (two waves per SIMD, one
  // workgroup per CU; each LDS operand read feeds 1.33 MFMAs instead of 1), used when
  // they fill the chip at least twice over.  Smaller ones: 128 x 128 tiles of 4 waves,
  // 64 x 64 each.  Every element's sum runs through the same MFMA sequence at the same
  // position of a 32 x 32 block in both shapes, so a row's result never depends on the
  // shape chosen, i.e. on the other rows of the launch.
  constexpr int64_t kFill = 512;
  if (N % 256 == 0 && int64_t((M + 255) / 256) * (N / 256) >= kFill)
    return gemm_go<2, 4, 4, 2, RR_GEMM_STAGES>(g, s);
  return gemm_go<2, 2, 2, 2, RR_GEMM_STAGES>(g, s);
}

hipError_t launch_prefix_offsets(const int32_t* user_tokens, const int32_t* hoff, int B, int32_t* poff,
                                 hipStream_t s) {
  void* args[] = {&user_tokens, &hoff, &B, &poff};
  return hipLaunchKernel(reinterpret_cast<const void*>(k_prefix_offsets), dim3(1), dim3(256), args, 0, s);
}

hipError_t launch_prefix_rows(void* compact, void* blocked, int64_t row_bytes, const int32_t* block,
                              const int32_t* poff, int B, int n_compact, int n_blocked, int to_compact,
                              hipStream_t s) {
  if (n_compact <= 0) return hipSuccess;
  char* cp = static_cast<char*>(compact);
  char* bp = static_cast<char*>(blocked);
  void* args[] = {&cp, &bp, &row_bytes, &block, &poff, &B, &n_compact, &n_blocked, &to_compact};
  const int64_t grid = grid_of(static_cast<int64_t>(n_compact) * (row_bytes / 16), 256);
  return hipLaunchKernel(reinterpret_cast<const void*>(k_prefix_rows), dim3(static_cast<unsigned>(grid)), dim3(256),
                         args, 0, s);
}

hipError_t launch_split_offsets(const int32_t* offsets, const int32_t* cand_start, int B, int32_t* hoff,
                                int32_t* coff, int32_t* hlen, hipStream_t s) {
  void* args[] = {&offsets, &cand_start, &B, &hoff, &coff, &hlen};
  return hipLaunchKernel(reinterpret_cast<const void*>(k_split_offsets), dim3(1), dim3(256), args, 0, s);
}

hipError_t launch_split_rows(const void* src, int64_t row_bytes, const int32_t* offsets, const int32_t* cand_start,
                             const int32_t* hoff, const int32_t* coff, int B, int T, void* hist, int Th, void* cand,
                             int Tc, hipStream_t s) {
  if (T <= 0 || (!hist && !cand)) return hipSuccess;
  const char* sp = static_cast<const char*>(src);
  char* hp = static_cast<char*>(hist);
  char* cp = static_cast<char*>(cand);
  void* args[] = {&sp, &row_bytes, &offsets, &cand_start, &hoff, &coff, &B, &T, &hp, &Th, &cp, &Tc};
  const int64_t grid = grid_of(static_cast<int64_t>(T) * (row_bytes / 16), 256);
  return hipLaunchKernel(reinterpret_cast<const void*>(k_split_rows), dim3(static_cast<unsigned>(grid)), dim3(256),
                         args, 0, s);
}

namespace {

constexpr float kRmsEps = 1e-6f;

struct RankerWs {
  size_t h, q, k, v, o, kh, vh, xh, xp, hoff, coff, hlen, poff, attn, cand, utok, total;
};

// Workspace of a layer-stack call: normed rows h, q, k, v, o (bf16, `rows` rows), the
// history keys and values when no cache is given and the frozen history states when
// the caller does not take them (`th_buf` rows each), the split offsets, and the two
// attention plans (full layers over T rows; candidate-only over Th history and Tc
// candidate rows).
RankerWs ranker_layout(int64_t B, int64_t rows, int64_t th_buf, int64_t T, int64_t Th, int64_t Tc, int64_t Tp,
                       int64_t H, int64_t d) {
  const int64_t D = H * d;
  RankerWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off = align256(off + bytes); return at; };
  w.h = take(2 * rows * D);
  w.q = take(2 * rows * D);
  w.k = take(2 * rows * D);
  w.v = take(2 * rows * D);
  w.o = take(2 * rows * D);
  w.kh = take(2 * th_buf * D);
  w.vh = take(2 * th_buf * D);
  w.xh = take(4 * th_buf * D);
  w.xp = take(4 * Tp * D);
  w.hoff = take(4 * (B + 1));
  w.coff = take(4 * (B + 1));
  w.hlen = take(4 * (B + 1));
  w.poff = take(4 * (B + 1));
  w.attn = take(T > 0 ? rr_attn_workspace_bytes(static_cast<int32_t>(B), static_cast<int32_t>(T),
                                                 static_cast<int32_t>(H), static_cast<int32_t>(d))
                      : 0);
  w.cand = take(rr_cand_only_workspace_bytes(static_cast<int32_t>(B), static_cast<int32_t>(Th),
                                             static_cast<int32_t>(Tc), static_cast<int32_t>(H),
                                             static_cast<int32_t>(d)));
  w.utok = take(Tp > 0 ? rr_user_token_attn_workspace_bytes(static_cast<int32_t>(B), static_cast<int32_t>(Th),
                                                            static_cast<int32_t>(Tp), static_cast<int32_t>(H),
                                                            static_cast<int32_t>(d))
                       : 0);
  w.total = off;
  return w;
}

// the full request: T rows, Tc of them candidates
RankerWs full_layout(int64_t B, int64_t T, int64_t Tc, int64_t Tp, int64_t H, int64_t d) {
  return ranker_layout(B, T, T - Tc, T, T - Tc, Tc, Tp, H, d);
}

// a cached request: Tc candidate rows against Th cached history rows
RankerWs cached_layout(int64_t B, int64_t Th, int64_t Tc, int64_t H, int64_t d) {
  return ranker_layout(B, Tc, 0, 0, Th, Tc, 0, H, d);
}

int ranker_sizes(int32_t B, int32_t T, int32_t Tc, int32_t H, int32_t d, int32_t Tp = 0) {
  if (B < 0 || T < 0 || Tc < 0 || Tc > T || Tp < 0 || Tp > T - Tc || H <= 0 || d <= 0) return RR_EINVAL;
  if (!(d == 32 || d == 64 || d == 128)) return RR_EUNSUPPORTED;   // the bf16 MFMA attention
  const int64_t D = int64_t(H) * d;
  if (D % kGn != 0 || D > 16384) return RR_EUNSUPPORTED;           // projection tiles
  if (rr_attn_workspace_bytes(B, T, H, d) == 0 || rr_cand_only_workspace_bytes(B, T - Tc, Tc, H, d) == 0)
    return RR_EUNSUPPORTED;
  return RR_OK;
}

int layers_ok(const rr_layer* layers, int32_t n) {
  if (!layers || n <= 0) return 0;
  for (int i = 0; i < n; ++i)
    if (!layers[i].norm_gain || !layers[i].w_qkv || !layers[i].w_o) return 0;
  return 1;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

int st(hipError_t e) { return e == hipSuccess ? RR_OK : RR_EHIP; }

#define RR_TRY(x)                  \
  do {                             \
    const int rr_s_ = (x);         \
    if (rr_s_ != RR_OK) return rr_s_; \
  } while (0)

double log2_theta(float theta_base) {
  return std::log2(theta_base > 0.f ? static_cast<double>(theta_base) : 10000.0);
}

// One candidate-only layer over Tc candidate rows x_cand, whose users' history keys
// (already rotated) and values are kh, vh [Th][H][d]; the plan is in wc.
int cand_layer(float* x_cand, const rr_layer& L, const void* kh, const void* vh, const int32_t* cand_offsets,
               const int32_t* hlen, int32_t B, int32_t Th, int32_t Tc, int32_t H, int32_t d, double lb,
               void* ws, const RankerWs& w, void* wc, size_t wc_bytes, hipStream_t s) {
  const int D = H * d;
  void* q = at<void>(ws, w.q);
  void* k = at<void>(ws, w.k);
  void* v = at<void>(ws, w.v);
  void* o = at<void>(ws, w.o);
  void* h = at<void>(ws, w.h);
  void* qkv[3] = {q, k, v};
  RR_TRY(st(launch_rms_norm(x_cand, L.norm_gain, h, Tc, D, kRmsEps, s)));
  RR_TRY(st(launch_gemm_bt(h, L.w_qkv, Tc, 3 * D, D, qkv, D, nullptr, s)));
  // every candidate at its user's history end: cand_start = the user's first candidate row
  RR_TRY(st(launch_rope_qk(q, k, q, k, cand_offsets, cand_offsets, hlen, B, Tc, H, d, RR_BF16, lb, s)));
  RR_TRY(rr_cand_only_run(q, kh, vh, k, v, o, B, Th, Tc, H, d, RR_BF16, 0.f, wc, wc_bytes, s));
  return st(launch_gemm_bt(o, L.w_o, Tc, D, D, nullptr, 0, x_cand, s));
}

}  // namespace
}  // namespace rr

using namespace rr;

extern "C" {

size_t rr_ranker_workspace_bytes(int32_t B, int32_t T, int32_t Tc, int32_t Tp, int32_t H, int32_t d) {
  if (ranker_sizes(B, T, Tc, H, d, Tp) != RR_OK) return 0;
  return full_layout(B, T, Tc, Tp, H, d).total;
}

int rr_rms_norm(const float* x, const float* gain, void* out, int32_t M, int32_t D, float eps,
                hipStream_t stream) {
  if (M < 0 || D <= 0 || D % 4 != 0) return RR_EINVAL;
  if (M == 0) return RR_OK;
  if (!x || !gain || !out) return RR_EINVAL;
  return st(launch_rms_norm(x, gain, out, M, D, eps > 0.f ? eps : kRmsEps, stream));
}

int rr_linear(const void* a, const void* w, void* out, float* residual, int32_t M, int32_t N, int32_t K,
              hipStream_t stream) {
  if (M < 0 || N <= 0 || K <= 0) return RR_EINVAL;
  if (N % kGn != 0 || K % kGk != 0) return RR_EUNSUPPORTED;
  if (M == 0) return RR_OK;
  if (!a || !w || (!out && !residual) || (out && residual)) return RR_EINVAL;
  void* outs[3] = {out, nullptr, nullptr};
  return st(launch_gemm_bt(a, w, M, N, K, outs, N, residual, stream));
}

int rr_ranker_fwd(float* x, const rr_layer* layers, int32_t n_layers, int32_t n_cand_only,
                  const int32_t* offsets, const int32_t* cand_start, const int32_t* user_tokens, int32_t B,
                  int32_t T, int32_t Tc, int32_t Tp, int32_t H, int32_t d, float theta_base, float* x_cand_out,
                  float* x_hist_out, void* kv_cache, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  if (!user_tokens) Tp = 0;
  RR_TRY(ranker_sizes(B, T, Tc, H, d, Tp));
  if (!layers_ok(layers, n_layers) || n_cand_only < 0 || n_cand_only > n_layers) return RR_EINVAL;
  if (B == 0 || T == 0) return RR_OK;
  if (!x || !offsets || !cand_start || (Tc > 0 && !x_cand_out)) return RR_EINVAL;
  const RankerWs w = full_layout(B, T, Tc, Tp, H, d);
  if (!workspace || workspace_bytes < w.total) return RR_EWORKSPACE;
  const int32_t Th = T - Tc, D = H * d, n_full = n_layers - n_cand_only;
  const double lb = log2_theta(theta_base);
  void* ws = workspace;
  int32_t* hoff = at<int32_t>(ws, w.hoff);
  int32_t* coff = at<int32_t>(ws, w.coff);
  int32_t* hlen = at<int32_t>(ws, w.hlen);
  void* wa = at<void>(ws, w.attn);
  void* wc = at<void>(ws, w.cand);
  const size_t wa_bytes = w.cand - w.attn, wc_bytes = w.total - w.cand;
  u16* cache = static_cast<u16*>(kv_cache);
  const int64_t layer_elems = int64_t(Th) * D;
  RR_TRY(st(launch_split_offsets(offsets, cand_start, B, hoff, coff, hlen, stream)));

  void* q = at<void>(ws, w.q);
  void* k = at<void>(ws, w.k);
  void* v = at<void>(ws, w.v);
  void* o = at<void>(ws, w.o);
  void* h = at<void>(ws, w.h);
  void* qkv[3] = {q, k, v};
  if (n_full > 0)
    RR_TRY(rr_attn_plan(offsets, cand_start, nullptr, 0, B, T, H, d, RR_BF16, wa, wa_bytes, stream));
  for (int l = 0; l < n_full; ++l) {
    const rr_layer& L = layers[l];
    RR_TRY(st(launch_rms_norm(x, L.norm_gain, h, T, D, kRmsEps, stream)));
    RR_TRY(st(launch_gemm_bt(h, L.w_qkv, T, 3 * D, D, qkv, D, nullptr, stream)));
    // the rotary pass also writes this layer's history keys (rotated) and values, compacted,
    // into the cache
    RR_TRY(st(launch_rope_qk_cache(q, k, q, k, offsets, cand_start, nullptr, B, T, H, d, RR_BF16, lb,
                                   cache ? cache + (2 * l) * layer_elems : nullptr, v,
                                   cache ? cache + (2 * l + 1) * layer_elems : nullptr, hoff, Th, stream)));
    RR_TRY(rr_attn_run(q, k, v, o, B, T, H, d, RR_BF16, 0.f, wa, wa_bytes, stream));
    RR_TRY(st(launch_gemm_bt(o, L.w_o, T, D, D, nullptr, 0, x, stream)));
  }

  // the split: history states freeze, candidates go on
  float* xh = x_hist_out ? x_hist_out : at<float>(ws, w.xh);
  RR_TRY(st(launch_split_rows(x, int64_t(D) * 4, offsets, cand_start, hoff, coff, B, T, xh, Th, x_cand_out, Tc,
                              stream)));
  if (n_cand_only == 0) return RR_OK;
  RR_TRY(rr_cand_only_plan(hoff, coff, B, Th, Tc, H, d, RR_BF16, wc, wc_bytes, stream));
  // candidate_only_layers_update_user_token: the user tokens (each user's first rows) keep
  // being updated, reading the user's [user tokens | frozen history] keys; their states
  // move to a compact block xp for the candidate-only layers
  float* xp = at<float>(ws, w.xp);
  int32_t* poff = at<int32_t>(ws, w.poff);
  void* wu = at<void>(ws, w.utok);
  const size_t wu_bytes = w.total - w.utok;
  if (Tp > 0) {
    RR_TRY(st(launch_prefix_offsets(user_tokens, hoff, B, poff, stream)));
    RR_TRY(st(launch_prefix_rows(xp, xh, int64_t(D) * 4, hoff, poff, B, Tp, Th, 1, stream)));
    RR_TRY(rr_user_token_attn_plan(hoff, poff, B, Th, Tp, H, d, RR_BF16, wu, wu_bytes, stream));
  }
  for (int l = n_full; l < n_layers; ++l) {
    const rr_layer& L = layers[l];
    void* kh = cache ? static_cast<void*>(cache + (2 * l) * layer_elems) : at<void>(ws, w.kh);
    void* vh = cache ? static_cast<void*>(cache + (2 * l + 1) * layer_elems) : at<void>(ws, w.vh);
    void* kv[3] = {kh, vh, nullptr};
    // the frozen history's keys and values through this layer's norm and projections,
    // its rows at positions 0 .. h_b - 1 (cand_start = the next user's first row)
    RR_TRY(st(launch_rms_norm(xh, L.norm_gain, h, Th, D, kRmsEps, stream)));
    RR_TRY(st(launch_gemm_bt(h, static_cast<const u16*>(L.w_qkv) + int64_t(D) * D, Th, 2 * D, D, kv, D,
                             nullptr, stream)));
    if (Tp > 0) {   // the user tokens from their current states, into their key and value slots
      RR_TRY(st(launch_rms_norm(xp, L.norm_gain, h, Tp, D, kRmsEps, stream)));
      RR_TRY(st(launch_gemm_bt(h, L.w_qkv, Tp, 3 * D, D, qkv, D, nullptr, stream)));
      RR_TRY(st(launch_prefix_rows(k, kh, int64_t(D) * 2, hoff, poff, B, Tp, Th, 0, stream)));
      RR_TRY(st(launch_prefix_rows(v, vh, int64_t(D) * 2, hoff, poff, B, Tp, Th, 0, stream)));
    }
    RR_TRY(st(launch_rope_qk(nullptr, kh, nullptr, kh, hoff, hoff + 1, nullptr, B, Th, H, d, RR_BF16, lb,
                             stream)));
    if (Tp > 0) {   // user tokens at positions 0 .. p_b - 1, reading [user tokens | history]
      RR_TRY(st(launch_rope_qk(q, nullptr, q, nullptr, poff, poff + 1, nullptr, B, Tp, H, d, RR_BF16, lb,
                               stream)));
      RR_TRY(rr_user_token_attn_run(q, kh, vh, o, B, Th, Tp, H, d, RR_BF16, 0.f, wu, wu_bytes, stream));
      RR_TRY(st(launch_gemm_bt(o, L.w_o, Tp, D, D, nullptr, 0, xp, stream)));
    }
    RR_TRY(cand_layer(x_cand_out, L, kh, vh, coff, hlen, B, Th, Tc, H, d, lb, ws, w, wc, wc_bytes, stream));
  }
  if (Tp > 0) RR_TRY(st(launch_prefix_rows(xp, xh, int64_t(D) * 4, hoff, poff, B, Tp, Th, 0, stream)));
  return RR_OK;
}

size_t rr_ranker_cached_workspace_bytes(int32_t B, int32_t Th, int32_t Tc, int32_t H, int32_t d) {
  if (Th < 0 || Tc < 0 || int64_t(Th) + Tc > 0x7fffffff) return 0;
  if (ranker_sizes(B, Th + Tc, Tc, H, d) != RR_OK) return 0;
  return cached_layout(B, Th, Tc, H, d).total;
}

int rr_ranker_cached_fwd(float* x_cand, const rr_layer* layers, int32_t n_layers, const void* kv_cache,
                         const int32_t* hist_offsets, const int32_t* cand_offsets, int32_t B, int32_t Th,
                         int32_t Tc, int32_t H, int32_t d, float theta_base, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (Th < 0 || Tc < 0 || int64_t(Th) + Tc > 0x7fffffff) return RR_EINVAL;
  RR_TRY(ranker_sizes(B, Th + Tc, Tc, H, d));
  if (!layers_ok(layers, n_layers)) return RR_EINVAL;
  if (B == 0 || Tc == 0) return RR_OK;
  if (!x_cand || !kv_cache || !hist_offsets || !cand_offsets) return RR_EINVAL;
  const RankerWs w = cached_layout(B, Th, Tc, H, d);
  if (!workspace || workspace_bytes < w.total) return RR_EWORKSPACE;
  void* ws = workspace;
  const int32_t D = H * d;
  const double lb = log2_theta(theta_base);
  void* wc = at<void>(ws, w.cand);
  const size_t wc_bytes = w.total - w.cand;
  // history lengths from the history offsets (the split kernel with no candidates)
  int32_t* hlen = at<int32_t>(ws, w.hlen);
  RR_TRY(st(launch_split_offsets(hist_offsets, hist_offsets + 1, B, at<int32_t>(ws, w.hoff),
                                 at<int32_t>(ws, w.coff), hlen, stream)));
  RR_TRY(rr_cand_only_plan(hist_offsets, cand_offsets, B, Th, Tc, H, d, RR_BF16, wc, wc_bytes, stream));
  const u16* cache = static_cast<const u16*>(kv_cache);
  const int64_t layer_elems = int64_t(Th) * D;
  for (int l = 0; l < n_layers; ++l)
    RR_TRY(cand_layer(x_cand, layers[l], cache + (2 * l) * layer_elems, cache + (2 * l + 1) * layer_elems,
                      cand_offsets, hlen, B, Th, Tc, H, d, lb, ws, w, wc, wc_bytes, stream));
  return RR_OK;
}

}  // extern "C"
