// Quantise-then-dispatch for gfx950: BF16 token rows and their top-k expert
// ids in, expert-ordered E4M3 rows with 1x128 scales out.
//
// Source pages (no section numbers; located by page and paragraph):
//   P2 Q&A board page (xn--9g3bo1gtkw0l8ubf92bgle.kr), paragraph 4: the
//      activations entering the MoE up-projection are quantised to FP8
//      first, then dispatched.
//   P3 "How I Improved My Deepseek In In The Future" (youlimart.com),
//      paragraph 4: 8 routed experts per token.
//
// Layout (the pages fix none of it): pair i = t * topk + j with an expert id
// in [0, E) becomes one row; rows are grouped by expert, and inside an
// expert ordered by i, so the result is unique and deterministic.
//
// Four launches on one stream:
//   1. k_dispatch_count    per block of 256 pairs, a histogram over experts
//                          (LDS atomics: counts do not depend on order);
//   2. k_dispatch_scan     one workgroup: expert totals, the exclusive scan
//                          that gives offsets[], and each block's first row
//                          per expert;
//   3. k_dispatch_scatter  one wave per block walks its pairs in index order
//                          64 at a time; a lane's rank among the lanes with
//                          the same expert is counted lane by lane, so
//                          positions follow i;
//   4. k_dispatch_quant    1x128 quantisation, each token tile read once and
//                          its codes and scale stored to every routed row of
//                          that token (the per-tile arithmetic is the
//                          activation quantiser's, bit for bit).
// This file is built with -ffp-contract=off, like the other quantisers.
#include "fgq_device.h"
#include "fgq_launch.h"

namespace fgq {

constexpr int kPairsPerBlock = 256;

// 1. per-block expert histogram: counts[b * E + e]
__global__ __launch_bounds__(256) void k_dispatch_count(const int32_t* __restrict__ ids, int64_t N, int E,
                                                        int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t i0 = (int64_t)blockIdx.x * kPairsPerBlock;
#pragma unroll
  for (int u = 0; u < kPairsPerBlock / 256; ++u) {
    const int64_t i = i0 + u * 256 + threadIdx.x;
    if (i < N) {
      const int32_t e = ids[i];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Exclusive scan of one value per thread across a 1024-thread workgroup;
// returns the sum of the values of the lower threads, `total` gets the sum.
__device__ int32_t block_exclusive_scan(int32_t v, int32_t* sh, int32_t& total) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int32_t add = t >= d ? sh[t - d] : 0;
    __syncthreads();
    sh[t] += add;
    __syncthreads();
  }
  const int32_t incl = sh[t];
  total = sh[1023];
  __syncthreads();
  return incl - v;
}

__device__ __forceinline__ int32_t wave_sum(int32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t y = __shfl_up(v, d);
    if (lane >= d) v += y;
  }
  return v;
}

// 2. offsets[0..E] and base[b * E + e] = first row of expert e in block b.
// 16 waves; wave w handles experts w, w + 16, ...: its lanes sum (then
// prefix-sum) the expert's block counts 64 blocks at a time.  E <= 4096.
__global__ __launch_bounds__(1024) void k_dispatch_scan(const int32_t* __restrict__ counts, int nb, int E,
                                                        int32_t* __restrict__ base, int32_t* __restrict__ offsets) {
  __shared__ int32_t first_row[4096];  // expert totals, then expert offsets
  __shared__ int32_t sh[1024];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int e = w; e < E; e += 16) {
    int32_t t = 0;
    for (int b = lane; b < nb; b += 64) t += counts[(int64_t)b * E + e];
    t = wave_sum(t);
    if (lane == 0) first_row[e] = t;
  }
  __syncthreads();
  // offsets: exclusive scan over experts; thread t owns experts 4t .. 4t + 3
  int32_t v[4], local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * (int)threadIdx.x + j;
    v[j] = e < E ? first_row[e] : 0;
    local += v[j];
  }
  int32_t total;
  int32_t run = block_exclusive_scan(local, sh, total);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * (int)threadIdx.x + j;
    if (e < E) {
      offsets[e] = run;
      first_row[e] = run;
    }
    run += v[j];
  }
  if (threadIdx.x == 0) offsets[E] = total;
  __syncthreads();
  for (int e = w; e < E; e += 16) {
    int32_t carry = first_row[e];
    for (int b0 = 0; b0 < nb; b0 += 64) {
      const int b = b0 + lane;
      const int32_t c = b < nb ? counts[(int64_t)b * E + e] : 0;
      const int32_t incl = wave_inclusive_scan(c, lane);
      if (b < nb) base[(int64_t)b * E + e] = carry + incl - c;
      carry += __shfl(incl, 63);
    }
  }
}

// 3. one wave per block: dest[i] (row or -1) and row_src[row] = i.  Each
// lane compares its expert with every lane of the 64-pair round: its rank is
// the number of lower lanes with the same expert, and the highest such lane
// moves the expert's LDS counter past the round.
__global__ __launch_bounds__(64) void k_dispatch_scatter(const int32_t* __restrict__ ids, int64_t N, int E,
                                                         const int32_t* __restrict__ base,
                                                         int32_t* __restrict__ dest, int32_t* __restrict__ row_src) {
  extern __shared__ int32_t cnt[];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) cnt[e] = base[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  const int64_t i0 = (int64_t)blockIdx.x * kPairsPerBlock;
  constexpr int kRounds = kPairsPerBlock / 64;
  int32_t ev[kRounds];  // all of the block's ids in flight at once
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t i = i0 + r * 64 + lane;
    ev[r] = i < N ? ids[i] : -1;
  }
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t i = i0 + r * 64 + lane;
    const int32_t e = ev[r];
    const bool valid = i < N && e >= 0 && e < E;
    const int32_t key = valid ? e : -1 - lane;  // lanes that are not routed match nobody
    int rank = 0, later = 0;
#pragma unroll 16
    for (int l = 0; l < 64; ++l) {
      const int32_t kl = __builtin_amdgcn_readlane(key, l);
      rank += (l < lane) & (kl == key);
      later += (l > lane) & (kl == key);
    }
    int32_t pos = -1;
    if (valid) {
      // one LDS read for all routed lanes, then one write by the last lane
      // of each expert (the wave executes them in this order)
      const int32_t c0 = cnt[e];
      pos = c0 + rank;
      if (later == 0) cnt[e] = c0 + rank + 1;
    }
    if (i < N) dest[i] = pos;
    if (valid) row_src[pos] = (int32_t)i;
  }
}

// 4. 1x128 quantisation of token tiles stored to each routed row.  A
// workgroup of 256 lanes owns 16 * kDispU consecutive (token, kb) tiles;
// a 16-lane group holds one tile (16 x 8 BF16 values).
constexpr int kDispU = 4;

// MAXK > 0: topk <= MAXK, the destination rows of each tile's token are
// loaded with the tile (no dependent load before each store); MAXK = 0: any topk.
template <class SF, int MAXK>
__global__ __launch_bounds__(256) void k_dispatch_quant(const uint16_t* __restrict__ x, int64_t ldx, uint32_t KB,
                                                        uint32_t n_tiles, int topk, const int32_t* __restrict__ dest,
                                                        uint8_t* __restrict__ q, int64_t ldq,
                                                        typename SF::T* __restrict__ s, int64_t s_sm, int64_t s_skb) {
  const uint32_t lane16 = threadIdx.x & 15u;
  const uint32_t grp = threadIdx.x >> 4;
  const uint32_t first = blockIdx.x * (16u * kDispU) + grp;
  uint4 v[kDispU];
  uint32_t tt[kDispU], kk[kDispU];
  int32_t dr[kDispU][MAXK > 0 ? MAXK : 1];
#pragma unroll
  for (int u = 0; u < kDispU; ++u) {
    uint32_t g = first + 16u * u;
    g = g < n_tiles ? g : n_tiles - 1u;  // clamped tail: loads stay in bounds
    tt[u] = g / KB;
    kk[u] = g - tt[u] * KB;
    v[u] = load_nt16(x + (int64_t)tt[u] * ldx + kk[u] * 128u + lane16 * 8u);
    if constexpr (MAXK > 0) {
#pragma unroll
      for (int j = 0; j < MAXK; ++j) dr[u][j] = j < topk ? dest[(int64_t)tt[u] * topk + j] : -1;
    }
  }
#pragma unroll
  for (int u = 0; u < kDispU; ++u) {
    if (first + 16u * u >= n_tiles) break;  // uniform across each 16-lane row
    float f[8];
    unpack8(v[u], f);
    const float a = max16(absmax8(f));
    typename SF::T sc;
    float r;
    SF::derive(a, sc, r);
    const uint2 codes = cast8(f, r);
    const int nk = MAXK > 0 ? MAXK : topk;
    for (int j = 0; j < nk; ++j) {
      const int32_t row = MAXK > 0 ? dr[u][MAXK > 0 ? j : 0] : dest[(int64_t)tt[u] * topk + j];
      if (row < 0) continue;
      store_nt8(q + (int64_t)row * ldq + kk[u] * 128u + lane16 * 8u, codes);
      if (lane16 == 0) s[(int64_t)row * s_sm + (int64_t)kk[u] * s_skb] = sc;
    }
  }
}

size_t dispatch_workspace_bytes(int64_t T, int64_t topk, int64_t E) {
  const int64_t N = T * topk;
  if (N <= 0 || E <= 0) return 0;
  const int64_t nb = (N + kPairsPerBlock - 1) / kPairsPerBlock;
  return (size_t)(2 * nb * E) * sizeof(int32_t);
}

template <class SF>
static hipError_t launch_dispatch(const uint16_t* x, int64_t ldx, int64_t T, int64_t K, const int32_t* ids,
                                  int64_t topk, int64_t E, uint8_t* q, int64_t ldq, typename SF::T* s, int64_t s_sm,
                                  int64_t s_skb, int32_t* offsets, int32_t* row_src, int32_t* dest, void* workspace,
                                  hipStream_t st) {
  const int64_t N = T * topk;
  const int nb = (int)((N + kPairsPerBlock - 1) / kPairsPerBlock);
  int32_t* counts = static_cast<int32_t*>(workspace);
  int32_t* base = counts + (int64_t)nb * E;
  const size_t lds = (size_t)E * sizeof(int32_t);
  if (nb > 0) hipLaunchKernelGGL(k_dispatch_count, dim3(nb), dim3(256), lds, st, ids, N, (int)E, counts);
  hipLaunchKernelGGL(k_dispatch_scan, dim3(1), dim3(1024), 0, st, counts, nb, (int)E, base, offsets);
  if (nb > 0) {
    hipLaunchKernelGGL(k_dispatch_scatter, dim3(nb), dim3(64), lds, st, ids, N, (int)E, base, dest, row_src);
    const uint32_t KB = (uint32_t)(K / 128);
    const uint32_t n_tiles = (uint32_t)(T * KB);
    if (n_tiles > 0) {
      const uint32_t grid = (n_tiles + 16u * kDispU - 1) / (16u * kDispU);
      if (topk <= 8)
        hipLaunchKernelGGL((k_dispatch_quant<SF, 8>), dim3(grid), dim3(256), 0, st, x, ldx, KB, n_tiles, (int)topk,
                           dest, q, ldq, s, s_sm, s_skb);
      else
        hipLaunchKernelGGL((k_dispatch_quant<SF, 0>), dim3(grid), dim3(256), 0, st, x, ldx, KB, n_tiles, (int)topk,
                           dest, q, ldq, s, s_sm, s_skb);
    }
  }
  return hipGetLastError();
}

hipError_t launch_quant_dispatch_1x128(const uint16_t* x, int64_t ldx, int64_t T, int64_t K,
                                       const int32_t* ids, int64_t topk, int64_t E, uint8_t* q, int64_t ldq,
                                       float* s, int64_t s_sm, int64_t s_skb, int32_t* offsets,
                                       int32_t* row_src, int32_t* dest, void* workspace, hipStream_t st) {
  return launch_dispatch<ScaleF32>(x, ldx, T, K, ids, topk, E, q, ldq, s, s_sm, s_skb, offsets, row_src, dest,
                                   workspace, st);
}

hipError_t launch_quant_dispatch_1x128_e8m0(const uint16_t* x, int64_t ldx, int64_t T, int64_t K,
                                            const int32_t* ids, int64_t topk, int64_t E, uint8_t* q, int64_t ldq,
                                            uint8_t* s, int64_t s_sm, int64_t s_skb, int32_t* offsets,
                                            int32_t* row_src, int32_t* dest, void* workspace, hipStream_t st) {
  return launch_dispatch<ScaleE8M0>(x, ldx, T, K, ids, topk, E, q, ldq, s, s_sm, s_skb, offsets, row_src, dest,
                                    workspace, st);
}

}  // namespace fgq
