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

// 16x16 output, K = 128 FP8 (E4M3) for both operands, no block scales
// (the scale operands are zero, which selects the unscaled instruction).
__device__ __forceinline__ v4f mfma_16x16x128_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int NBW = BN >= 128 ? BN / 128 : 1;  // weight-scale blocks per tile
  static constexpr int SA_OFF = A_BYTES + B_BYTES;
  static constexpr int SW_OFF = SA_OFF + BM * 4;
  static constexpr int STAGE = SW_OFF + ((NBW * 4 + 15) / 16) * 16;
  static constexpr int A_CH = BM * 8 / NT, B_CH = BN * 8 / NT;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile is a multiple of 16x16");
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "even split of the chunk loads");
  static_assert(WN <= 128 && (128 % WN == 0 || WN % 128 == 0), "a wave's columns share one weight-scale block");
  static_assert(BM <= NT, "one thread per activation-scale row");
};

// One output tile [row_begin, row_begin + BM) x [n0, n0 + BN), rows >= row_end
// are neither read (loads clamp to row_end - 1) nor written.
template <class C>
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

  // per-thread global sources for the chunk loads
  const uint8_t* a_src[C::A_CH];
  int a_dst[C::A_CH];
#pragma unroll
  for (int j = 0; j < C::A_CH; ++j) {
    const int g = tid + j * C::NT, r = g >> 3, cc = g & 7;
    int64_t gr = row_begin + r;
    gr = gr < row_end ? gr : row_end - 1;
    a_src[j] = qa + gr * lda + cc * 16;
    a_dst[j] = r * 128 + ((cc ^ (r & 7)) << 4);
  }
  const uint8_t* b_src[C::B_CH];
  int b_dst[C::B_CH];
#pragma unroll
  for (int j = 0; j < C::B_CH; ++j) {
    const int g = tid + j * C::NT, r = g >> 3, cc = g & 7;
    b_src[j] = qw + (n0 + r) * ldw + cc * 16;
    b_dst[j] = C::A_BYTES + r * 128 + ((cc ^ (r & 7)) << 4);
  }
  const float* sa_src = nullptr;
  if (tid < C::BM) {
    int64_t gr = row_begin + tid;
    gr = gr < row_end ? gr : row_end - 1;
    sa_src = sa + gr * sa_sm;
  }
  const float* sw_src = nullptr;
  if (tid < C::NBW) sw_src = sw + ((n0 >> 7) + tid) * sw_snb;

  uint4 ra[C::A_CH], rb[C::B_CH];
  float rsa = 0.0f, rsw = 0.0f;
  auto load_chunk = [&](int kb) {
    const int64_t ko = (int64_t)kb * 128;
#pragma unroll
    for (int j = 0; j < C::A_CH; ++j) ra[j] = *reinterpret_cast<const uint4*>(a_src[j] + ko);
#pragma unroll
    for (int j = 0; j < C::B_CH; ++j) rb[j] = *reinterpret_cast<const uint4*>(b_src[j] + ko);
    if (tid < C::BM) rsa = sa_src[(int64_t)kb * sa_skb];
    if (tid < C::NBW) rsw = sw_src[(int64_t)kb * sw_skb];
  };
  auto store_chunk = [&](int stage) {
    uint8_t* base = lds + stage * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::A_CH; ++j) *reinterpret_cast<uint4*>(base + a_dst[j]) = ra[j];
#pragma unroll
    for (int j = 0; j < C::B_CH; ++j) *reinterpret_cast<uint4*>(base + b_dst[j]) = rb[j];
    if (tid < C::BM) reinterpret_cast<float*>(base + C::SA_OFF)[tid] = rsa;
    if (tid < C::NBW) reinterpret_cast<float*>(base + C::SW_OFF)[tid] = rsw;
  };

  v4f acc[C::TM][C::TN];
#pragma unroll
  for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::TN; ++ni) acc[mi][ni] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  // LDS byte offsets of this lane's fragment rows (two 16-byte columns each)
  const int c0 = lgrp * 2;
  int a_off[C::TM][2], b_off[C::TN][2];
#pragma unroll
  for (int mi = 0; mi < C::TM; ++mi) {
    const int r = wm * C::WM + mi * 16 + l16;
    a_off[mi][0] = r * 128 + ((c0 ^ (r & 7)) << 4);
    a_off[mi][1] = r * 128 + (((c0 + 1) ^ (r & 7)) << 4);
  }
#pragma unroll
  for (int ni = 0; ni < C::TN; ++ni) {
    const int r = wn * C::WN + ni * 16 + l16;
    b_off[ni][0] = C::A_BYTES + r * 128 + ((c0 ^ (r & 7)) << 4);
    b_off[ni][1] = C::A_BYTES + r * 128 + (((c0 + 1) ^ (r & 7)) << 4);
  }
  const int sw_idx = (wn * C::WN) / 128;

  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int kb = 0; kb < KB; ++kb) {
    const bool more = kb + 1 < KB;
    if (more) load_chunk(kb + 1);
    const uint8_t* base = lds + (kb & 1) * C::STAGE;
    v8i bf[C::TN];
#pragma unroll
    for (int ni = 0; ni < C::TN; ++ni) {
      const uint4 lo = *reinterpret_cast<const uint4*>(base + b_off[ni][0]);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + b_off[ni][1]);
      bf[ni] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    const float swv = reinterpret_cast<const float*>(base + C::SW_OFF)[sw_idx];
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi) {
      const uint4 lo = *reinterpret_cast<const uint4*>(base + a_off[mi][0]);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + a_off[mi][1]);
      const v8i af = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const v4f sa4 = *reinterpret_cast<const v4f*>(base + C::SA_OFF + (wm * C::WM + mi * 16 + lgrp * 4) * 4);
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
    if (more) store_chunk((kb + 1) & 1);
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

using DenseCfg = TileCfg<128, 128, 2, 2>;

template <class C>
__global__ __launch_bounds__(C::NT) void k_gemm_fp8_bs(const uint8_t* __restrict__ qa, int64_t lda,
                                                       const float* __restrict__ sa, int64_t sa_sm,
                                                       int64_t sa_skb, const uint8_t* __restrict__ qw,
                                                       int64_t ldw, const float* __restrict__ sw,
                                                       int64_t sw_snb, int64_t sw_skb,
                                                       uint16_t* __restrict__ c, int64_t ldc, int64_t M,
                                                       int KB) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::STAGE];
  const int64_t row_begin = (int64_t)blockIdx.x * C::BM;
  const int64_t n0 = (int64_t)blockIdx.y * C::BN;
  gemm_tile<C>(qa, lda, sa, sa_sm, sa_skb, row_begin, M, qw, ldw, sw, sw_snb, sw_skb, n0, c, ldc, KB, lds);
}

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm_fp8_blockscaled(const uint8_t* qa, int64_t lda, const float* sa, int64_t sa_sm,
                                       int64_t sa_skb, const uint8_t* qw, int64_t ldw, const float* sw,
                                       int64_t sw_snb, int64_t sw_skb, uint16_t* c, int64_t ldc,
                                       int64_t M, int64_t N, int64_t K, void*, size_t, hipStream_t st) {
  using C = DenseCfg;
  const dim3 grid((unsigned)((M + C::BM - 1) / C::BM), (unsigned)(N / C::BN));
  hipLaunchKernelGGL(k_gemm_fp8_bs<C>, grid, dim3(C::NT), 0, st, qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw,
                     sw_snb, sw_skb, c, ldc, M, (int)(K / 128));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped (MoE) variant.  blockIdx.x is an m-tile slot over all experts in
// expert order, blockIdx.y the n-tile.  The slot -> (expert, m-tile) map is
// computed on the GPU from offsets[] (a workgroup-wide prefix sum over the
// per-expert tile counts), so the host never reads the routing result.
// Slots beyond the real tile count leave at once.
template <class C>
__global__ __launch_bounds__(C::NT) void k_grouped_gemm_fp8_bs(
    const uint8_t* __restrict__ qa, int64_t lda, const float* __restrict__ sa, int64_t sa_sm,
    int64_t sa_skb, const uint8_t* __restrict__ qw, int64_t ldw, int64_t w_es,
    const float* __restrict__ sw, int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
    const int32_t* __restrict__ offsets, int E, int64_t total_rows, uint16_t* __restrict__ c,
    int64_t ldc, int KB) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::STAGE];
  __shared__ int scan[C::NT];
  __shared__ int found[3];
  const int tid = threadIdx.x;
  const int slot = blockIdx.x;
  if (tid == 0) found[0] = -1;
  int carried = 0;  // tiles of experts before this batch
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
  if (e < 0) return;  // slot past the last tile: whole workgroup leaves
  const int64_t row_begin = found[1], row_end = found[2];
  const int64_t n0 = (int64_t)blockIdx.y * C::BN;
  gemm_tile<C>(qa, lda, sa, sa_sm, sa_skb, row_begin, row_end, qw + (int64_t)e * w_es, ldw,
               sw + (int64_t)e * sw_es, sw_snb, sw_skb, n0, c, ldc, KB, lds);
}

hipError_t launch_grouped_gemm_fp8_blockscaled(const uint8_t* qa, int64_t lda, const float* sa,
                                               int64_t sa_sm, int64_t sa_skb, const uint8_t* qw,
                                               int64_t ldw, int64_t w_es, const float* sw,
                                               int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
                                               const int32_t* offsets, int64_t E, int64_t total_rows,
                                               uint16_t* c, int64_t ldc, int64_t N, int64_t K,
                                               hipStream_t st) {
  using C = DenseCfg;
  // each non-empty expert adds at most one partial m-tile
  const int64_t nonempty = E < total_rows ? E : total_rows;
  const int64_t slots = (total_rows + C::BM - 1) / C::BM + nonempty;
  const dim3 grid((unsigned)slots, (unsigned)(N / C::BN));
  hipLaunchKernelGGL(k_grouped_gemm_fp8_bs<C>, grid, dim3(C::NT), 0, st, qa, lda, sa, sa_sm, sa_skb, qw,
                     ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets, (int)E, total_rows, c, ldc,
                     (int)(K / 128));
  return hipGetLastError();
}

}  // namespace fgq
