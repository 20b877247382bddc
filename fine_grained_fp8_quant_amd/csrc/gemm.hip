// Block-scaled FP8 GEMM for gfx950, dense and ragged grouped (MoE).
//
//   C[m, n] = bf16( sum_kb  sa[m, kb] * sw[n/128, kb] * sum_{k in chunk kb} qa[m, k] * qw[n, k] )
//
// Source pages (no section numbers; located by page and paragraph):
//   P2 Q&A board page (xn--9g3bo1gtkw0l8ubf92bgle.kr), paragraph 3: per-group
//      scaling factors along K, multiplied in as the dequantisation step;
//      paragraph 2: on H800 one warpgroup promotes while another multiplies.
//   P4 "How Google Is Changing How We Method Deepseek"
//      (xn--jj0bz6z98ct0a29q.com), paragraph 4: MMA accumulation has a
//      limited bit width, so partial sums are promoted to FP32.
//   P2 paragraph 4 and P3 "How I Improved My Deepseek In In The Future"
//      (youlimart.com), paragraph 4: FP8 forward GEMMs of the MoE experts.
//
// CDNA4 design (not the pages' Hopper design):
//   * One 128-wide K chunk is exactly one v_mfma_f32_16x16x128_f8f6f4 per
//     16x16 output sub-tile, so the chunk's FP8 sum lands in a fresh FP32
//     temporary (C operand = inline 0) and is promoted at once:
//     acc = fma(t, sa * sw, acc) on the vector ALU.  The promotion interval
//     is the scale group, 128, since the scales change every 128 along K.
//     The vector FMAs of one sub-tile overlap the matrix core's work on the
//     next (they are independent instructions of the same wave), the
//     register-level counterpart of the pages' two-warpgroup overlap.
//   * Operands are K-contiguous in HBM and in LDS.  Each lane feeds 32
//     contiguous K bytes of one row to the MFMA; A and B use the same lane
//     layout, so whatever order the unit pairs the 128 K positions in, the
//     sum is the full chunk dot product.
//   * LDS rows are 128 bytes (one chunk); the 16-byte column c of row r is
//     stored at column c ^ (r & 7) so that 16 lanes reading 16 different
//     rows at one logical column hit different banks.
//   * Global -> register -> LDS double buffering: chunk kb+1 is in flight
//     while chunk kb is multiplied.
#include "fgq_device.h"
#include "fgq_launch.h"

namespace fgq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// 16x16 output, K = 128 FP8 (E4M3) for both operands, no block scales (zero
// scale operands select the unscaled instruction).  The unit sums each group
// of 8 products in a fixed-point window about 13 bits below the group's
// largest product, truncating what falls below it.
__device__ __forceinline__ v4f mfma_16x16x128_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// 16x16 output, K = 32 FP16.  Products of E4M3 values are exact in it and
// the sum keeps binary32-level precision.
__device__ __forceinline__ v4f mfma_16x16x32_f16(const v8h& a, const v8h& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Eight E4M3 codes (two words) -> eight FP16 values; exact (every finite
// E4M3 value, subnormals included, is an FP16 value).
__device__ __forceinline__ v8h e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return (v8h){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 16 bytes global -> LDS without registers; `lds` is the wave-uniform base of
// the 64 x 16-byte slots this instruction fills, lane i writing slot i.
__device__ __forceinline__ void dma16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)lds, 4, 0, 0);
}
// wait for this wave's outstanding global loads (LDS DMA included)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int NBW = BN >= 128 ? BN / 128 : 1;  // weight-scale blocks per tile
  static constexpr int SA_OFF = A_BYTES + B_BYTES;
  static constexpr int SW_OFF = SA_OFF + BM * 4;
  static constexpr int STAGE = SW_OFF + 256;
  static constexpr int A_INS = BM / 8, B_INS = BN / 8;       // 1 KB DMA instructions per stage
  static constexpr int A_PER_W = (A_INS + NW - 1) / NW, B_PER_W = (B_INS + NW - 1) / NW;
  static constexpr int SA_INS = (BM + 63) / 64;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile is a multiple of 16x16");
  static_assert(BM % 8 == 0 && BN % 8 == 0, "whole DMA instructions");
  static_assert(WN <= 128 && (128 % WN == 0), "a wave's columns share one weight-scale block");
  static_assert(SA_INS + 1 <= NW, "scale loads need a wave each");
  static_assert(NBW <= 64, "weight scales fit one instruction");
};

// One output tile [row_begin, row_begin + BM) x [n0, n0 + BN); rows >= row_end
// are neither read (their loads repeat row row_end - 1) nor written.
template <class C, int MODE>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ qa, int64_t lda,
                                          const float* __restrict__ sa, int64_t sa_sm, int64_t sa_skb,
                                          int64_t row_begin, int64_t row_end,
                                          const uint8_t* __restrict__ qw, int64_t ldw,
                                          const float* __restrict__ sw, int64_t sw_snb, int64_t sw_skb,
                                          int64_t n0, uint16_t* __restrict__ c, int64_t ldc, int KB,
                                          uint8_t* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int l16 = lane & 15, lgrp = lane >> 4;

  // ---- this lane's DMA sources: slot s = ins * 64 + lane holds row s / 8,
  // physical column s % 8 = logical column (s % 8) ^ (row & 7).  Rows of one
  // lane differ by multiples of 8 * NW, so (row & 7) = (lane / 8) & 7 for all
  // of them; sources are the tile base plus 32-bit offsets.
  const int dcol = ((lane & 7) ^ ((lane >> 3) & 7)) * 16;
  const uint8_t* a_tile = qa + row_begin * lda;
  const int64_t a_last = row_end - 1 - row_begin;
  uint32_t a_src[C::A_PER_W];
#pragma unroll
  for (int j = 0; j < C::A_PER_W; ++j) {
    const int r = (wave + j * C::NW) * 8 + (lane >> 3);
    a_src[j] = (uint32_t)((r < a_last ? r : a_last) * lda) + dcol;
  }
  const uint8_t* b_tile = qw + n0 * ldw;
  uint32_t b_src[C::B_PER_W];
#pragma unroll
  for (int j = 0; j < C::B_PER_W; ++j) {
    const int r = (wave + j * C::NW) * 8 + (lane >> 3);
    b_src[j] = (uint32_t)((r < C::BN ? r : 0) * ldw) + dcol;
  }
  const float* s_src = nullptr;  // activation scales (waves < SA_INS) or weight scales (wave SA_INS)
  if (wave < C::SA_INS) {
    int64_t gr = row_begin + wave * 64 + lane;
    gr = gr < row_end ? gr : row_end - 1;
    s_src = sa + gr * sa_sm;
  } else if (wave == C::SA_INS) {
    s_src = sw + ((n0 >> 7) + (lane < C::NBW ? lane : 0)) * sw_snb;
  }

  auto issue = [&](int kb, int stage) {
    uint8_t* base = lds + stage * C::STAGE;
    const uint8_t* at = a_tile + (int64_t)kb * 128;
    const uint8_t* bt = b_tile + (int64_t)kb * 128;
#pragma unroll
    for (int j = 0; j < C::A_PER_W; ++j) {
      const int ins = wave + j * C::NW;
      if (C::A_INS % C::NW == 0 || ins < C::A_INS) dma16(at + a_src[j], base + ins * 1024);
    }
#pragma unroll
    for (int j = 0; j < C::B_PER_W; ++j) {
      const int ins = wave + j * C::NW;
      if (C::B_INS % C::NW == 0 || ins < C::B_INS) dma16(bt + b_src[j], base + C::A_BYTES + ins * 1024);
    }
    if (wave < C::SA_INS) {
      dma4(s_src + (int64_t)kb * sa_skb, base + C::SA_OFF + wave * 256);
    } else if (wave == C::SA_INS && lane < C::NBW) {
      dma4(s_src + (int64_t)kb * sw_skb, base + C::SW_OFF);
    }
  };

  v4f acc[C::TM][C::TN];
#pragma unroll
  for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::TN; ++ni) acc[mi][ni] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  // LDS byte offsets of this lane's fragment rows: 32 contiguous code bytes
  // (logical columns 2*lgrp, 2*lgrp + 1 of the 128-byte chunk row).  Sub-tile
  // rows step by 16, which keeps (row & 7), so sub-tiles are base + 2048 * i.
  const int c0 = lgrp * 2, rsw = l16 & 7;
  const int a_off0 = (wm * C::WM + l16) * 128 + ((c0 ^ rsw) << 4);
  const int a_off1 = (wm * C::WM + l16) * 128 + (((c0 + 1) ^ rsw) << 4);
  const int b_off0 = C::A_BYTES + (wn * C::WN + l16) * 128 + ((c0 ^ rsw) << 4);
  const int b_off1 = C::A_BYTES + (wn * C::WN + l16) * 128 + (((c0 + 1) ^ rsw) << 4);
  const int sa_off = C::SA_OFF + (wm * C::WM + lgrp * 4) * 4;
  const int sw_idx = (wn * C::WN) / 128;

  issue(0, 0);
  wait_vmem();
  __syncthreads();
  for (int kb = 0; kb < KB; ++kb) {
    if (kb + 1 < KB) issue(kb + 1, (kb + 1) & 1);
    const uint8_t* base = lds + (kb & 1) * C::STAGE;
    const float swv = reinterpret_cast<const float*>(base + C::SW_OFF)[sw_idx];
    if constexpr (MODE == 1) {
      // FP8 matrix core: one instruction per 16x16 sub-tile and chunk
      v8i bf[C::TN];
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) {
        const uint4 lo = *reinterpret_cast<const uint4*>(base + b_off0 + ni * 2048);
        const uint4 hi = *reinterpret_cast<const uint4*>(base + b_off1 + ni * 2048);
        bf[ni] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int mi = 0; mi < C::TM; ++mi) {
        const uint4 lo = *reinterpret_cast<const uint4*>(base + a_off0 + mi * 2048);
        const uint4 hi = *reinterpret_cast<const uint4*>(base + a_off1 + mi * 2048);
        const v8i af = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        const v4f sa4 = *reinterpret_cast<const v4f*>(base + sa_off + mi * 64);
        const float s0 = sa4[0] * swv, s1 = sa4[1] * swv, s2 = sa4[2] * swv, s3 = sa4[3] * swv;
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) {
          const v4f t = mfma_16x16x128_fp8(af, bf[ni]);
          acc[mi][ni][0] = __builtin_fmaf(t[0], s0, acc[mi][ni][0]);
          acc[mi][ni][1] = __builtin_fmaf(t[1], s1, acc[mi][ni][1]);
          acc[mi][ni][2] = __builtin_fmaf(t[2], s2, acc[mi][ni][2]);
          acc[mi][ni][3] = __builtin_fmaf(t[3], s3, acc[mi][ni][3]);
        }
      }
    } else {
      // exact products: codes -> FP16 in registers, four K = 32 steps per chunk
      v8h bh[C::TN][4];
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) {
        const uint4 lo = *reinterpret_cast<const uint4*>(base + b_off0 + ni * 2048);
        const uint4 hi = *reinterpret_cast<const uint4*>(base + b_off1 + ni * 2048);
        bh[ni][0] = e4m3x8_to_f16(lo.x, lo.y);
        bh[ni][1] = e4m3x8_to_f16(lo.z, lo.w);
        bh[ni][2] = e4m3x8_to_f16(hi.x, hi.y);
        bh[ni][3] = e4m3x8_to_f16(hi.z, hi.w);
      }
#pragma unroll
      for (int mi = 0; mi < C::TM; ++mi) {
        const uint4 lo = *reinterpret_cast<const uint4*>(base + a_off0 + mi * 2048);
        const uint4 hi = *reinterpret_cast<const uint4*>(base + a_off1 + mi * 2048);
        v8h ah[4];
        ah[0] = e4m3x8_to_f16(lo.x, lo.y);
        ah[1] = e4m3x8_to_f16(lo.z, lo.w);
        ah[2] = e4m3x8_to_f16(hi.x, hi.y);
        ah[3] = e4m3x8_to_f16(hi.z, hi.w);
        const v4f sa4 = *reinterpret_cast<const v4f*>(base + sa_off + mi * 64);
        const float s0 = sa4[0] * swv, s1 = sa4[1] * swv, s2 = sa4[2] * swv, s3 = sa4[3] * swv;
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) {
          // one chunk of one sub-tile: four chained K = 32 steps, then promote
          v4f t = mfma_16x16x32_f16(ah[0], bh[ni][0], (v4f){0.0f, 0.0f, 0.0f, 0.0f});
          t = mfma_16x16x32_f16(ah[1], bh[ni][1], t);
          t = mfma_16x16x32_f16(ah[2], bh[ni][2], t);
          t = mfma_16x16x32_f16(ah[3], bh[ni][3], t);
          acc[mi][ni][0] = __builtin_fmaf(t[0], s0, acc[mi][ni][0]);
          acc[mi][ni][1] = __builtin_fmaf(t[1], s1, acc[mi][ni][1]);
          acc[mi][ni][2] = __builtin_fmaf(t[2], s2, acc[mi][ni][2]);
          acc[mi][ni][3] = __builtin_fmaf(t[3], s3, acc[mi][ni][3]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  }

  // epilogue: lane holds rows lgrp*4 + i, column l16 of each 16x16 sub-tile
#pragma unroll
  for (int mi = 0; mi < C::TM; ++mi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t gr = row_begin + wm * C::WM + mi * 16 + lgrp * 4 + i;
      if (gr < row_end) {
        uint16_t* crow = c + gr * ldc + n0 + wn * C::WN + l16;
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) crow[ni * 16] = (uint16_t)bf16_rne(acc[mi][ni][i]);
      }
    }
  }
}

// Linear workgroup id -> (m-tile, n-tile).  Workgroups are dealt to the 8
// XCDs round-robin; renumber so each XCD owns a contiguous run of tiles, and
// walk tiles in groups of kGroupM m-tiles so that the tiles resident at once
// on one XCD share A row blocks and W column blocks in that XCD's L2.
constexpr int kXcds = 8, kGroupM = 8;
__device__ __forceinline__ void tile_of(int bid, int G, int tiles_m, int& tm, int& tn) {
  const int q = G / kXcds, r = G % kXcds;
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int logical = xcd * q + (xcd < r ? xcd : r) + local;
  const int tiles_n = G / tiles_m;
  const int group = kGroupM * tiles_n;
  const int g = logical / group, in = logical % group;
  const int first_m = g * kGroupM;
  const int gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  tm = first_m + in % gm;
  tn = in / gm;
}

using BigCfg = TileCfg<256, 256, 2, 4>;
using SmallCfg = TileCfg<64, 128, 1, 4>;

template <class C, int MODE>
__global__ __launch_bounds__(C::NT) void k_gemm_fp8_bs(const uint8_t* __restrict__ qa, int64_t lda,
                                                       const float* __restrict__ sa, int64_t sa_sm,
                                                       int64_t sa_skb, const uint8_t* __restrict__ qw,
                                                       int64_t ldw, const float* __restrict__ sw,
                                                       int64_t sw_snb, int64_t sw_skb,
                                                       uint16_t* __restrict__ c, int64_t ldc, int64_t M,
                                                       int tiles_m, int KB) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * C::STAGE];
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tm, tn);
  gemm_tile<C, MODE>(qa, lda, sa, sa_sm, sa_skb, (int64_t)tm * C::BM, M, qw, ldw, sw, sw_snb, sw_skb,
                     (int64_t)tn * C::BN, c, ldc, KB, lds);
}

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

template <class C, int MODE>
static void launch_dense(const uint8_t* qa, int64_t lda, const float* sa, int64_t sa_sm, int64_t sa_skb,
                         const uint8_t* qw, int64_t ldw, const float* sw, int64_t sw_snb, int64_t sw_skb,
                         uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int tiles_m = (int)((M + C::BM - 1) / C::BM);
  const int tiles_n = (int)(N / C::BN);
  hipLaunchKernelGGL((k_gemm_fp8_bs<C, MODE>), dim3(tiles_m * tiles_n), dim3(C::NT), 0, st, qa, lda, sa, sa_sm,
                     sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, tiles_m, (int)(K / 128));
}

hipError_t launch_gemm_fp8_blockscaled(const uint8_t* qa, int64_t lda, const float* sa, int64_t sa_sm,
                                       int64_t sa_skb, const uint8_t* qw, int64_t ldw, const float* sw,
                                       int64_t sw_snb, int64_t sw_skb, uint16_t* c, int64_t ldc,
                                       int64_t M, int64_t N, int64_t K, int mode, void*, size_t,
                                       hipStream_t st) {
  const bool big = M > 128 && N % 256 == 0;
  if (mode == 1) {
    if (big) launch_dense<BigCfg, 1>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, st);
    else launch_dense<SmallCfg, 1>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, st);
  } else {
    if (big) launch_dense<BigCfg, 0>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, st);
    else launch_dense<SmallCfg, 0>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, st);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped (MoE) variant.  The linear workgroup id maps (as above) to an
// (m-tile slot, n-tile) pair; slots run over all experts in expert order.
// The slot -> (expert, rows) map is computed on the GPU from offsets[] with
// a workgroup-wide prefix sum over the per-expert tile counts, so the host
// never reads the routing result.  Slots past the last real tile leave at once.
template <class C, int MODE>
__global__ __launch_bounds__(C::NT) void k_grouped_gemm_fp8_bs(
    const uint8_t* __restrict__ qa, int64_t lda, const float* __restrict__ sa, int64_t sa_sm,
    int64_t sa_skb, const uint8_t* __restrict__ qw, int64_t ldw, int64_t w_es,
    const float* __restrict__ sw, int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
    const int32_t* __restrict__ offsets, int E, int64_t total_rows, uint16_t* __restrict__ c,
    int64_t ldc, int slots, int KB) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * C::STAGE];
  int* scan = reinterpret_cast<int*>(lds);  // reused before the tile loop starts
  __shared__ int found[3];
  const int tid = threadIdx.x;
  int slot, tn;
  tile_of(blockIdx.x, gridDim.x, slots, slot, tn);
  if (tid == 0) found[0] = -1;
  int carried = 0;  // tiles of the experts before this batch
  for (int e0 = 0; e0 < E; e0 += C::NT) {
    const int e = e0 + tid;
    int tiles = 0;
    int64_t r0 = 0, r1 = 0;
    if (e < E) {
      r0 = offsets[e];
      r1 = offsets[e + 1];
      r0 = r0 < 0 ? 0 : (r0 > total_rows ? total_rows : r0);
      r1 = r1 < r0 ? r0 : (r1 > total_rows ? total_rows : r1);
      tiles = (int)((r1 - r0 + C::BM - 1) / C::BM);
    }
    scan[tid] = tiles;
    __syncthreads();
    for (int d = 1; d < C::NT; d <<= 1) {  // inclusive Hillis-Steele scan
      const int v = tid >= d ? scan[tid - d] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int incl = carried + scan[tid];
    const int excl = incl - tiles;
    if (tiles > 0 && slot >= excl && slot < incl) {
      found[0] = e;
      found[1] = (int)(r0 + (int64_t)(slot - excl) * C::BM);
      found[2] = (int)r1;
    }
    carried += scan[C::NT - 1];
    __syncthreads();
    if (found[0] >= 0 || slot < carried) break;
  }
  __syncthreads();
  const int e = found[0];
  if (e < 0) return;  // slot past the last tile: the whole workgroup leaves
  const int64_t row_begin = found[1], row_end = found[2];
  gemm_tile<C, MODE>(qa, lda, sa, sa_sm, sa_skb, row_begin, row_end, qw + (int64_t)e * w_es, ldw,
                     sw + (int64_t)e * sw_es, sw_snb, sw_skb, (int64_t)tn * C::BN, c, ldc, KB, lds);
}

template <class C, int MODE>
static void launch_grouped(const uint8_t* qa, int64_t lda, const float* sa, int64_t sa_sm, int64_t sa_skb,
                           const uint8_t* qw, int64_t ldw, int64_t w_es, const float* sw, int64_t sw_snb,
                           int64_t sw_skb, int64_t sw_es, const int32_t* offsets, int64_t E,
                           int64_t total_rows, uint16_t* c, int64_t ldc, int64_t N, int64_t K, hipStream_t st) {
  // each non-empty expert adds at most one partial m-tile
  const int64_t nonempty = E < total_rows ? E : total_rows;
  const int slots = (int)((total_rows + C::BM - 1) / C::BM + nonempty);
  const int tiles_n = (int)(N / C::BN);
  hipLaunchKernelGGL((k_grouped_gemm_fp8_bs<C, MODE>), dim3(slots * tiles_n), dim3(C::NT), 0, st, qa, lda, sa,
                     sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets, (int)E, total_rows, c,
                     ldc, slots, (int)(K / 128));
}

hipError_t launch_grouped_gemm_fp8_blockscaled(const uint8_t* qa, int64_t lda, const float* sa,
                                               int64_t sa_sm, int64_t sa_skb, const uint8_t* qw,
                                               int64_t ldw, int64_t w_es, const float* sw,
                                               int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
                                               const int32_t* offsets, int64_t E, int64_t total_rows,
                                               uint16_t* c, int64_t ldc, int64_t N, int64_t K, int mode,
                                               hipStream_t st) {
  const bool big = N % 256 == 0 && total_rows > 128;
  if (mode == 1) {
    if (big) launch_grouped<BigCfg, 1>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets, E, total_rows, c, ldc, N, K, st);
    else launch_grouped<SmallCfg, 1>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets, E, total_rows, c, ldc, N, K, st);
  } else {
    if (big) launch_grouped<BigCfg, 0>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets, E, total_rows, c, ldc, N, K, st);
    else launch_grouped<SmallCfg, 0>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets, E, total_rows, c, ldc, N, K, st);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Diagnostic: one v_mfma_f32_16x16x128_f8f6f4 on caller data, one wave.
// a, b: E4M3 [16][128] row-major (row = output row / column); cin, d:
// float [16][16] row-major.  d = a * b^T + cin as the matrix core computes it,
// with the same operand lane layout the GEMM uses.
__global__ __launch_bounds__(64) void k_debug_mfma(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                   const float* __restrict__ cin, float* __restrict__ d) {
  const int lane = threadIdx.x, l16 = lane & 15, lgrp = lane >> 4;
  const uint4 alo = *reinterpret_cast<const uint4*>(a + l16 * 128 + lgrp * 32);
  const uint4 ahi = *reinterpret_cast<const uint4*>(a + l16 * 128 + lgrp * 32 + 16);
  const uint4 blo = *reinterpret_cast<const uint4*>(b + l16 * 128 + lgrp * 32);
  const uint4 bhi = *reinterpret_cast<const uint4*>(b + l16 * 128 + lgrp * 32 + 16);
  const v8i av = (v8i){(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
  const v8i bv = (v8i){(int)blo.x, (int)blo.y, (int)blo.z, (int)blo.w, (int)bhi.x, (int)bhi.y, (int)bhi.z, (int)bhi.w};
  v4f c;
  for (int i = 0; i < 4; ++i) c[i] = cin[(lgrp * 4 + i) * 16 + l16];
  c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
  for (int i = 0; i < 4; ++i) d[(lgrp * 4 + i) * 16 + l16] = c[i];
}

hipError_t launch_debug_mfma(const uint8_t* a, const uint8_t* b, const float* cin, float* d, hipStream_t st) {
  hipLaunchKernelGGL(k_debug_mfma, dim3(1), dim3(64), 0, st, a, b, cin, d);
  return hipGetLastError();
}

}  // namespace fgq
