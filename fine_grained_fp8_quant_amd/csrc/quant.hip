// Online max-abs E4M3 quantisation kernels for gfx950:
//   k_quant_act_1x128      one scale per 1x128 activation tile
//   k_quant_w_128x128      one scale per 128x128 weight block (batched)
//   k_fused_rmsnorm_quant  RMSNorm in binary32 fused with the 1x128 cast
//
// Source pages (no section numbers; located by page and paragraph):
//   P1 "DeepSeek core readings" notes page (why-be.why-be.co.kr), paragraph 1:
//      1x128 activation tiles, 128x128 weight blocks.
//   P2 Q&A board page (xn--9g3bo1gtkw0l8ubf92bgle.kr), paragraphs 1, 3, 4: the
//      quantisation reads 128 BF16 values from HBM and writes FP8 back; the
//      scale maps the max-abs value onto the largest FP8 value and is derived
//      online; normalisation stays in higher precision.
//   P3 "How I Improved My Deepseek In In The Future" (youlimart.com),
//      paragraph 3: fusing layer normalisation with the FP8 cast.
//
// Each kernel comes in two scale formats: a binary32 scale s = a / 448, and
// a power-of-two scale stored as an E8M0 byte (the microscaling block-scale
// format that the pages relate the method to: P1 paragraph 4, P4 paragraph 3;
// gfx950's matrix core applies such scales itself).
//
// All three are HBM-bound streaming kernels: 16-byte coalesced loads, a lane
// group reduction for the max-abs, one correctly rounded division pair per
// group, then multiply / clamp / hardware E4M3 convert.  This file is built
// with -ffp-contract=off: the binary32 results must be bit-identical to the
// written definition (no fused multiply-add anywhere).
#include "fgq_device.h"
#include "fgq_launch.h"

namespace fgq {

// ---------------------------------------------------------------------------
// 1x128 activation tiles.  A tile is 256 bytes of BF16: 16 lanes x 16 bytes,
// one DPP row.  A workgroup of 256 lanes owns a block of 16 rows x 4
// consecutive K blocks: each 16-lane group one row, its 1 KB read as four
// tiles, all loads issued before any arithmetic.  With K-block-major scales
// (the layout the GEMM prefers) the block's scales of one K block are 16
// consecutive values, so a wave's scale stores cover one 16-byte run and the
// workgroup's a 64-byte run.  Measured against 64 consecutive tiles in row
// order (whose scales land in 56 different lines): 8192 x 7168 33.8 -> 31.2
// us, 32768 x 7168 117.4 -> 111.5 us; 16 x 2 and 16 x 8 blocks ran at the old
// speed, 8 tiles per group in row order slower.
constexpr int kActRows = 16, kActKB = 4;

template <class SF>
__global__ __launch_bounds__(256) void k_quant_act_1x128(
    const uint16_t* __restrict__ x, int64_t ldx, uint32_t KB, uint32_t M,
    uint8_t* __restrict__ q, int64_t ldq, typename SF::T* __restrict__ s, int64_t s_sm, int64_t s_skb) {
  // workgroup block: rows m0 .. m0 + 15 (one per 16-lane group) x K blocks kb0 .. kb0 + 3
  const uint32_t lane16 = threadIdx.x & 15u;
  const uint32_t grp = threadIdx.x >> 4;
  const uint32_t KBB = (KB + kActKB - 1u) / kActKB;
  const uint32_t m0 = (blockIdx.x / KBB) * kActRows, kb0 = (blockIdx.x % KBB) * kActKB;
  uint32_t m = m0 + grp;
  const bool row_ok = m < M;
  m = row_ok ? m : M - 1u;  // clamped rows: loads stay in bounds
  uint4 v[kActKB];
#pragma unroll
  for (int u = 0; u < kActKB; ++u) {
    uint32_t kb = kb0 + u;
    kb = kb < KB ? kb : KB - 1u;
    v[u] = load_nt16(x + (int64_t)m * ldx + kb * 128u + lane16 * 8u);
  }
  if (!row_ok) return;  // uniform per 16-lane group
#pragma unroll
  for (int u = 0; u < kActKB; ++u) {
    const uint32_t kb = kb0 + u;
    if (kb >= KB) break;
    float f[8];
    unpack8(v[u], f);
    const float a = max16(absmax8(f));
    typename SF::T sc;
    float r;
    SF::derive(a, sc, r);
    store_nt8(q + (int64_t)m * ldq + kb * 128u + lane16 * 8u, cast8(f, r));
    if (lane16 == 0) s[(int64_t)m * s_sm + (int64_t)kb * s_skb] = sc;
  }
}

template <class SF>
static hipError_t launch_act(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, uint8_t* q, int64_t ldq,
                             typename SF::T* s, int64_t s_sm, int64_t s_skb, hipStream_t st) {
  const uint32_t KB = (uint32_t)(K / 128);
  const uint32_t grid = (uint32_t)((M + kActRows - 1) / kActRows) * ((KB + kActKB - 1u) / kActKB);
  hipLaunchKernelGGL(k_quant_act_1x128<SF>, dim3(grid), dim3(256), 0, st, x, ldx, KB, (uint32_t)M, q, ldq, s,
                     s_sm, s_skb);
  return hipGetLastError();
}

hipError_t launch_quant_act_1x128(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, uint8_t* q,
                                  int64_t ldq, float* s, int64_t s_sm, int64_t s_skb, hipStream_t st) {
  return launch_act<ScaleF32>(x, ldx, M, K, q, ldq, s, s_sm, s_skb, st);
}

hipError_t launch_quant_act_1x128_e8m0(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, uint8_t* q,
                                       int64_t ldq, uint8_t* s, int64_t s_sm, int64_t s_skb, hipStream_t st) {
  return launch_act<ScaleE8M0>(x, ldx, M, K, q, ldq, s, s_sm, s_skb, st);
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks.  One workgroup per block: lane t reads 16 bytes of
// rows (t/16) + 16p, p = 0..7, keeps the 64 values in registers, and the
// block max-abs goes 16-lane DPP -> wave shuffle -> LDS across the 4 waves.
// NT: the codes bypass the caches (for outputs too large for the 256 MB
// last-level cache; smaller ones are left there for the GEMM that follows).
template <class SF, bool NT>
__global__ __launch_bounds__(256) void k_quant_w_128x128(
    const uint16_t* __restrict__ w, int64_t ldw, int64_t w_bs, uint32_t NB, uint32_t KB,
    uint8_t* __restrict__ q, int64_t ldq, int64_t q_bs, typename SF::T* __restrict__ s, int64_t s_snb,
    int64_t s_skb, int64_t s_bs) {
  __shared__ float red[4];
  uint32_t id = blockIdx.x;
  const uint32_t kb = id % KB;
  id /= KB;
  const uint32_t nb = id % NB;
  const uint32_t b = id / NB;
  const uint32_t c = threadIdx.x & 15u;
  const uint32_t r0 = threadIdx.x >> 4;
  const uint16_t* src = w + (int64_t)b * w_bs + ((int64_t)nb * 128 + r0) * ldw + kb * 128u + c * 8u;
  uint4 v[8];
#pragma unroll
  for (int p = 0; p < 8; ++p)
    v[p] = load_nt16(src + (int64_t)(16 * p) * ldw);
  float m = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    float f[8];
    unpack8(v[p], f);
    m = fmaxf(m, absmax8(f));
  }
  m = max16(m);
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  if ((threadIdx.x & 63u) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  typename SF::T sc;
  float r;
  SF::derive(a, sc, r);
  uint8_t* dst = q + (int64_t)b * q_bs + ((int64_t)nb * 128 + r0) * ldq + kb * 128u + c * 8u;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    float f[8];
    unpack8(v[p], f);
    if constexpr (NT) store_nt8(dst + (int64_t)(16 * p) * ldq, cast8(f, r));
    else *reinterpret_cast<uint2*>(dst + (int64_t)(16 * p) * ldq) = cast8(f, r);
  }
  if (threadIdx.x == 0) s[(int64_t)b * s_bs + (int64_t)nb * s_snb + (int64_t)kb * s_skb] = sc;
}

template <class SF>
static hipError_t launch_w(const uint16_t* w, int64_t ldw, int64_t w_bs, int64_t B, int64_t N, int64_t K,
                           uint8_t* q, int64_t ldq, int64_t q_bs, typename SF::T* s, int64_t s_snb,
                           int64_t s_skb, int64_t s_bs, hipStream_t st) {
  const uint32_t NB = (uint32_t)(N / 128), KB = (uint32_t)(K / 128);
  const uint32_t grid = (uint32_t)(B * NB * KB);
  // measured: non-temporal stores 4% faster for 940 MB of codes, 7% slower
  // for 132 MB (and the GEMM after it then misses the cache)
  if (B * N * K > ((int64_t)256 << 20))
    hipLaunchKernelGGL((k_quant_w_128x128<SF, true>), dim3(grid), dim3(256), 0, st, w, ldw, w_bs, NB, KB, q, ldq,
                       q_bs, s, s_snb, s_skb, s_bs);
  else
    hipLaunchKernelGGL((k_quant_w_128x128<SF, false>), dim3(grid), dim3(256), 0, st, w, ldw, w_bs, NB, KB, q, ldq,
                       q_bs, s, s_snb, s_skb, s_bs);
  return hipGetLastError();
}

hipError_t launch_quant_w_128x128(const uint16_t* w, int64_t ldw, int64_t w_bs, int64_t B, int64_t N,
                                  int64_t K, uint8_t* q, int64_t ldq, int64_t q_bs, float* s,
                                  int64_t s_snb, int64_t s_skb, int64_t s_bs, hipStream_t st) {
  return launch_w<ScaleF32>(w, ldw, w_bs, B, N, K, q, ldq, q_bs, s, s_snb, s_skb, s_bs, st);
}

hipError_t launch_quant_w_128x128_e8m0(const uint16_t* w, int64_t ldw, int64_t w_bs, int64_t B, int64_t N,
                                       int64_t K, uint8_t* q, int64_t ldq, int64_t q_bs, uint8_t* s,
                                       int64_t s_snb, int64_t s_skb, int64_t s_bs, hipStream_t st) {
  return launch_w<ScaleE8M0>(w, ldw, w_bs, B, N, K, q, ldq, q_bs, s, s_snb, s_skb, s_bs, st);
}

// ---------------------------------------------------------------------------
// Fused RMSNorm + 1x128 quantisation: one wave per row, the row held in
// registers (NI 16-byte vectors per lane, lane l owning vectors l + 64 i).
// That ownership is the summation order of the definition: lane l's partial
// adds the squares of its vectors in turn, value by value, then a butterfly
// over lane xor 32, 16, ..., 1.  In iteration i the lanes 16g..16g+15 hold
// exactly tile 4i + g, so the tile max is a 16-lane DPP reduction.
//
// Short rows (NI <= 16): the row is widened to binary32 once and normalised
// in place, and the tile maxima go through a per-wave LDS slot so that lane
// t does the two correctly rounded divisions of tile t (once per tile rather
// than once per lane of each 16-lane group).  gamma is widened into LDS once
// per workgroup; FULL drops the bounds guards when K = 512 NI.
template <class SF, int NI, bool FULL>
__global__ __launch_bounds__(256) void k_fused_rmsnorm_quant_regs(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ gamma, float eps,
    uint32_t M, uint32_t K, uint8_t* __restrict__ q, int64_t ldq, typename SF::T* __restrict__ s,
    int64_t s_sm, int64_t s_skb) {
  static_assert(NI <= 16, "one tile per lane in the scale pass");
  __shared__ float tile_slot[4][64];
  // gamma widened once per workgroup (not once per row): plane 0 holds
  // values 0..3 of each 8-value vector, plane 1 values 4..7, so a lane's
  // 16-byte reads sit at a 16-byte stride (no bank conflicts)
  __shared__ __attribute__((aligned(16))) float gsh[2][NI * 64 * 4];
  const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
  // FULL: K == 512 NI, every lane owns all NI of its vectors
  const uint32_t V = FULL ? NI * 64u : K / 8u, ntiles = K / 128u;
  for (uint32_t vi = threadIdx.x; vi < V; vi += 256u) {
    float g[8];
    unpack8(*reinterpret_cast<const uint4*>(gamma + vi * 8u), g);
    *reinterpret_cast<float4*>(&gsh[0][vi * 4u]) = make_float4(g[0], g[1], g[2], g[3]);
    *reinterpret_cast<float4*>(&gsh[1][vi * 4u]) = make_float4(g[4], g[5], g[6], g[7]);
  }
  __syncthreads();  // before any wave of the workgroup may leave
  const uint32_t row0 = blockIdx.x * 4u, row = row0 + w;
  const bool row_ok = row < M;
  __shared__ typename SF::T sc_sh[64][4];   // [tile][row of the workgroup]
  float* slot = tile_slot[w];
  if (row_ok) {
  float y[NI][8];
  {
    uint4 v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t vi = lane + 64u * i;
      v[i] = (FULL || vi < V) ? load_nt16(x + (int64_t)row * ldx + vi * 8u) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) unpack8(v[i], y[i]);
  }
  {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (FULL || lane + 64u * i < V) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = acc + y[i][j] * y[i][j];  // contraction is off in this file
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc = acc + __shfl_xor(acc, d);
    const float mean = acc / (float)K;
    const float var = mean + eps;
    const float rstd = 1.0f / sqrtf(var);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t vi = lane + 64u * i;
      if (FULL || vi < V) {  // V is a multiple of 16: whole 16-lane rows
        const float4 g0 = *reinterpret_cast<const float4*>(&gsh[0][vi * 4u]);
        const float4 g1 = *reinterpret_cast<const float4*>(&gsh[1][vi * 4u]);
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) y[i][j] = (y[i][j] * rstd) * g[j];
        const float a = max16(absmax8(y[i]));
        if ((lane & 15u) == 0) slot[vi >> 4] = a;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (lane < ntiles) {
      typename SF::T sc;
      float r;
      SF::derive(slot[lane], sc, r);
      sc_sh[lane][w] = sc;
      slot[lane] = r;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    uint8_t* qr = q + (int64_t)row * ldq;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t vi = lane + 64u * i;
      if (FULL || vi < V) store_nt8(qr + vi * 8u, cast8(y[i], slot[vi >> 4]));
    }
  }
  }
  // the workgroup's four rows' scales of tile t, stored together: with
  // K-block-major scales (s_sm == 1) they are four consecutive values, one
  // 16-byte store instead of four stores to four lines (16384 x 7168: 65.7
  // -> 63.3 us)
  __syncthreads();
  const uint32_t t = threadIdx.x;
  if (t < ntiles) {
    typename SF::T* st = s + (int64_t)row0 * s_sm + (int64_t)t * s_skb;
    if (sizeof(typename SF::T) == 4 && s_sm == 1 && row0 + 4u <= M && (reinterpret_cast<uintptr_t>(st) & 15) == 0) {
      const float4 v4 = make_float4(sc_sh[t][0], sc_sh[t][1], sc_sh[t][2], sc_sh[t][3]);
      *reinterpret_cast<float4*>(st) = v4;
    } else {
      for (uint32_t r = 0; r < 4u && row0 + r < M; ++r) st[(int64_t)r * s_sm] = sc_sh[t][r];
    }
  }
}

// Long rows (K up to 16384): the row stays packed BF16 in registers and is
// widened again for each pass; scales are computed per 16-lane group.
template <class SF, int NI>
__global__ __launch_bounds__(256) void k_fused_rmsnorm_quant_long(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ gamma, float eps,
    uint32_t M, uint32_t K, uint8_t* __restrict__ q, int64_t ldq, typename SF::T* __restrict__ s,
    int64_t s_sm, int64_t s_skb) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t row = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (row >= M) return;  // whole wave leaves together
  const uint32_t V = K / 8u;
  const uint16_t* xr = x + (int64_t)row * ldx;
  uint4 v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t vi = lane + 64u * i;
    if (vi < V) v[i] = load_nt16(xr + vi * 8u);
    else v[i] = make_uint4(0, 0, 0, 0);
  }
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (lane + 64u * i < V) {
      float f[8];
      unpack8(v[i], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = acc + f[j] * f[j];  // contraction is off in this file
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc = acc + __shfl_xor(acc, d);
  const float mean = acc / (float)K;
  const float var = mean + eps;
  const float rstd = 1.0f / sqrtf(var);
  uint8_t* qr = q + (int64_t)row * ldq;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t vi = lane + 64u * i;
    if (vi < V) {  // V is a multiple of 16: whole 16-lane rows
      const uint4 gv = *reinterpret_cast<const uint4*>(gamma + vi * 8u);
      float f[8], g[8], y[8];
      unpack8(v[i], f);
      unpack8(gv, g);
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = (f[j] * rstd) * g[j];
      const float a = max16(absmax8(y));
      typename SF::T sc;
      float r;
      SF::derive(a, sc, r);
      store_nt8(qr + vi * 8u, cast8(y, r));
      if ((lane & 15u) == 0) s[(int64_t)row * s_sm + (int64_t)(vi >> 4) * s_skb] = sc;
    }
  }
}

template <class SF, int NI>
static void launch_fused_regs(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, int64_t M,
                              int64_t K, uint8_t* q, int64_t ldq, typename SF::T* s, int64_t s_sm,
                              int64_t s_skb, hipStream_t st) {
  const dim3 grid((uint32_t)((M + 3) / 4));
  if (K == 512 * NI)  // rows that fill the registers exactly: no per-vector guards
    hipLaunchKernelGGL((k_fused_rmsnorm_quant_regs<SF, NI, true>), grid, dim3(256), 0, st, x, ldx,
                       gamma, eps, (uint32_t)M, (uint32_t)K, q, ldq, s, s_sm, s_skb);
  else
    hipLaunchKernelGGL((k_fused_rmsnorm_quant_regs<SF, NI, false>), grid, dim3(256), 0, st, x, ldx,
                       gamma, eps, (uint32_t)M, (uint32_t)K, q, ldq, s, s_sm, s_skb);
}

template <class SF>
static hipError_t launch_fused(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, int64_t M,
                               int64_t K, uint8_t* q, int64_t ldq, typename SF::T* s, int64_t s_sm,
                               int64_t s_skb, hipStream_t st) {
  const int64_t ni = (K / 8 + 63) / 64;
  if (ni <= 2) launch_fused_regs<SF, 2>(x, ldx, gamma, eps, M, K, q, ldq, s, s_sm, s_skb, st);
  else if (ni <= 4) launch_fused_regs<SF, 4>(x, ldx, gamma, eps, M, K, q, ldq, s, s_sm, s_skb, st);
  else if (ni <= 8) launch_fused_regs<SF, 8>(x, ldx, gamma, eps, M, K, q, ldq, s, s_sm, s_skb, st);
  else if (ni <= 12) launch_fused_regs<SF, 12>(x, ldx, gamma, eps, M, K, q, ldq, s, s_sm, s_skb, st);
  else if (ni <= 14) launch_fused_regs<SF, 14>(x, ldx, gamma, eps, M, K, q, ldq, s, s_sm, s_skb, st);
  else if (ni <= 16) launch_fused_regs<SF, 16>(x, ldx, gamma, eps, M, K, q, ldq, s, s_sm, s_skb, st);
  else
    hipLaunchKernelGGL((k_fused_rmsnorm_quant_long<SF, 32>), dim3((uint32_t)((M + 3) / 4)), dim3(256), 0, st, x,
                       ldx, gamma, eps, (uint32_t)M, (uint32_t)K, q, ldq, s, s_sm, s_skb);
  return hipGetLastError();
}

hipError_t launch_fused_rmsnorm_quant(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps,
                                      int64_t M, int64_t K, uint8_t* q, int64_t ldq, float* s,
                                      int64_t s_sm, int64_t s_skb, hipStream_t st) {
  return launch_fused<ScaleF32>(x, ldx, gamma, eps, M, K, q, ldq, s, s_sm, s_skb, st);
}

hipError_t launch_fused_rmsnorm_quant_e8m0(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps,
                                           int64_t M, int64_t K, uint8_t* q, int64_t ldq, uint8_t* s,
                                           int64_t s_sm, int64_t s_skb, hipStream_t st) {
  return launch_fused<ScaleE8M0>(x, ldx, gamma, eps, M, K, q, ldq, s, s_sm, s_skb, st);
}

// ---------------------------------------------------------------------------
// Diagnostics.
__global__ __launch_bounds__(256) void k_debug_encode_e4m3(uint32_t start, uint64_t n,
                                                           uint8_t* __restrict__ out) {
  const uint64_t i0 = ((uint64_t)blockIdx.x * 256u + threadIdx.x) * 4u;
  if (i0 >= n) return;
  float f[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) f[j] = clamp448(__uint_as_float(start + (uint32_t)(i0 + j)));
  const uint32_t w = e4m3x4(f[0], f[1], f[2], f[3]);
  if (i0 + 4 <= n) {
    uint8_t* p = out + i0;
    if ((reinterpret_cast<uintptr_t>(p) & 3u) == 0) {
      *reinterpret_cast<uint32_t*>(p) = w;
      return;
    }
  }
  for (int j = 0; j < 4 && i0 + j < n; ++j) out[i0 + j] = (uint8_t)(w >> (8 * j));
}

hipError_t launch_debug_encode_e4m3(uint32_t start, int64_t n, uint8_t* out, hipStream_t st) {
  const uint64_t threads = ((uint64_t)n + 3) / 4;
  const uint32_t grid = (uint32_t)((threads + 255) / 256);
  hipLaunchKernelGGL(k_debug_encode_e4m3, dim3(grid), dim3(256), 0, st, start, (uint64_t)n, out);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_debug_copy(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                    uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * 256u;
  for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

hipError_t launch_debug_copy(const void* src, void* dst, int64_t bytes, hipStream_t st) {
  const uint64_t n16 = (uint64_t)bytes / 16;
  uint64_t grid = (n16 + 255) / 256;
  if (grid > 65536) grid = 65536;
  if (grid == 0) grid = 1;
  hipLaunchKernelGGL(k_debug_copy, dim3((uint32_t)grid), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace fgq
