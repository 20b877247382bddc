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
// Launches on one stream:
//   1. k_dispatch_count    per block of 256 pairs, a histogram over experts
//                          (LDS atomics: counts do not depend on order);
//   2. k_dispatch_scan     one workgroup: expert totals, the exclusive scan
//                          that gives offsets[], and each block's first row
//                          per expert.  Skipped when blocks x experts is
//                          small: each scatter block then derives its own
//                          first rows from the counts;
//   3. k_dispatch_scatter  one wave per block walks its pairs in index order
//                          64 at a time; a lane's rank among the lanes with
//                          the same expert comes from one ballot per bit of
//                          the expert id, so positions follow i;
//   4. k_dispatch_quant    1x128 quantisation, each token tile read once and
//                          its codes stored to every routed row of that token
//                          (the per-tile arithmetic is the activation
//                          quantiser's, bit for bit).  Scales go to every
//                          routed row too when a row's scales are contiguous;
//                          otherwise once per token into the workspace, and
//   5. k_dispatch_gather_scales spreads them to the routed rows in row order
//                          (scattered 4-byte stores to K-block-major scales
//                          cost the quantiser a fifth of its time).
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
// prefix-sum) the expert's block counts 64 blocks at a time.  The expert
// offsets are one wave's scan, with no workgroup barrier inside: lane l owns
// experts l * per .. l * per + per - 1.  E <= 4096.
__global__ __launch_bounds__(1024) void k_dispatch_scan(const int32_t* __restrict__ counts, int nb, int E,
                                                        int32_t* __restrict__ base, int32_t* __restrict__ offsets) {
  __shared__ int32_t first_row[4096];  // expert totals, then expert offsets
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int e = w; e < E; e += 16) {
    int32_t t = 0;
    for (int b = lane; b < nb; b += 64) t += counts[(int64_t)b * E + e];
    t = wave_sum(t);
    if (lane == 0) first_row[e] = t;
  }
  __syncthreads();
  if (w == 0) {
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int32_t local = 0;
    for (int j = 0; j < per; ++j)
      if (e0 + j < E) local += first_row[e0 + j];
    const int32_t incl = wave_inclusive_scan(local, lane);
    int32_t run = incl - local;
    for (int j = 0; j < per; ++j) {
      const int e = e0 + j;
      if (e < E) {
        const int32_t v = first_row[e];
        offsets[e] = run;
        first_row[e] = run;
        run += v;
      }
    }
    if (lane == 63) offsets[E] = incl;
  }
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

// 3. one wave per block: dest[i] (row or -1) and row_src[row] = i.  A lane's
// rank among the 64 pairs of a round is the number of lower lanes routed to
// the same expert: the lanes with an equal expert id are found one id bit at
// a time with ballots, and the highest such lane moves the expert's LDS
// counter past the round.
//
// FUSED (small problems, nb * E <= kFusedScan): the block derives its own
// starting rows from the block counts instead of a separate scan: the pairs
// of expert e in earlier blocks, plus the expert offset (an exclusive scan of
// the totals); block 0 also writes offsets.  `counts` is read in place of
// `base`.
constexpr int kFusedScan = 8192;
template <bool FUSED>
__global__ __launch_bounds__(64) void k_dispatch_scatter(const int32_t* __restrict__ ids, int64_t N, int E,
                                                         const int32_t* __restrict__ base,
                                                         int32_t* __restrict__ dest, int32_t* __restrict__ row_src,
                                                         int nb, int32_t* __restrict__ offsets) {
  extern __shared__ int32_t cnt[];  // [E] running row of each expert (+ [E] totals when FUSED)
  const int lane = threadIdx.x;
  if constexpr (FUSED) {
    int32_t* tot = cnt + E;
    if (64 % E == 0) {
      // the table read flat, 64 consecutive entries per load: entry idx
      // belongs to block idx / E and expert idx mod E, which is lane mod E
      // for every load; the 64 / E lanes of one expert then add up
      const int e = lane % E;
      const int total = nb * E;
      int32_t all = 0, before = 0;
      constexpr int kU = 32;
      for (int i0 = 0; i0 < total; i0 += 64 * kU) {
        int32_t c[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int idx = i0 + u * 64 + lane;
          c[u] = idx < total ? base[idx] : 0;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int idx = i0 + u * 64 + lane;
          all += c[u];
          before += idx / E < (int)blockIdx.x ? c[u] : 0;
        }
      }
      for (int d = E; d < 64; d <<= 1) {
        all += __shfl_xor(all, d);
        before += __shfl_xor(before, d);
      }
      if (lane < E) {
        tot[e] = all;
        cnt[e] = before;
      }
    } else {
      // lane l sums expert e = l (then l + 64, ...) over all blocks and
      // over the blocks before this one, no atomics
      for (int e = lane; e < E; e += 64) {
        int32_t all = 0, before = 0;
        constexpr int kU = 16;
        for (int b0 = 0; b0 < nb; b0 += kU) {
          int32_t c[kU];
#pragma unroll
          for (int u = 0; u < kU; ++u) c[u] = b0 + u < nb ? base[(int64_t)(b0 + u) * E + e] : 0;
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            all += c[u];
            before += b0 + u < (int)blockIdx.x ? c[u] : 0;
          }
        }
        tot[e] = all;
        cnt[e] = before;
      }
    }
    __syncthreads();
    // expert offsets: lane l owns experts l * per .. l * per + per - 1
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int32_t local = 0;
    for (int j = 0; j < per; ++j)
      if (e0 + j < E) local += tot[e0 + j];
    const int32_t incl = wave_inclusive_scan(local, lane);
    int32_t run = incl - local;
    for (int j = 0; j < per; ++j) {
      const int e = e0 + j;
      if (e < E) {
        cnt[e] += run;
        if (blockIdx.x == 0) offsets[e] = run;
        run += tot[e];
      }
    }
    if (blockIdx.x == 0 && lane == 63) offsets[E] = incl;
  } else {
    for (int e = lane; e < E; e += 64) cnt[e] = base[(int64_t)blockIdx.x * E + e];
  }
  __syncthreads();
  const int64_t i0 = (int64_t)blockIdx.x * kPairsPerBlock;
  constexpr int kRounds = kPairsPerBlock / 64;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;  // bits of an expert id
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
    uint64_t same = __ballot(valid);  // routed lanes whose id agrees with this lane's in every bit
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(valid && bit);
      same &= bit ? ones : ~ones;
    }
    const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(same >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)same, 0u));
    const int later = __popcll(same) - rank - 1;
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
// TOKEN_SCALES: each tile's scale is written once, to s[t * KB + kb] (a
// token-major scratch array that k_dispatch_gather_scales spreads to the
// routed rows), instead of to every routed row.
template <class SF, int MAXK, bool TOKEN_SCALES>
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
    if (TOKEN_SCALES && lane16 == 0) s[(int64_t)tt[u] * KB + kk[u]] = sc;
    const int nk = MAXK > 0 ? MAXK : topk;
    for (int j = 0; j < nk; ++j) {
      const int32_t row = MAXK > 0 ? dr[u][MAXK > 0 ? j : 0] : dest[(int64_t)tt[u] * topk + j];
      if (row < 0) continue;
      store_nt8(q + (int64_t)row * ldq + kk[u] * 128u + lane16 * 8u, codes);
      if (!TOKEN_SCALES && lane16 == 0) s[(int64_t)row * s_sm + (int64_t)kk[u] * s_skb] = sc;
    }
  }
}

// 5. (with TOKEN_SCALES) s[r, kb] = tok[row_src[r] / topk, kb] for the routed
// rows r < offsets[E].  Thread r handles kGatherKB consecutive kb (from
// kGatherKB * blockIdx.y): consecutive threads write consecutive rows, which
// are contiguous when the caller's scales are K-block-major (the layout the
// GEMM reads best); the per-row stores of the quantiser would land
// 4 * rows bytes apart.
constexpr uint32_t kGatherKB = 8;
// row_src is read before the routed count is known (rows past it hold old
// values), so the token index is clamped into [0, T) and only the stores wait
// for r < offsets[E]: two dependent loads instead of three.
template <class SF>
__global__ __launch_bounds__(256) void k_dispatch_gather_scales(const typename SF::T* __restrict__ tok, uint32_t KB,
                                                                int topk, int32_t T, int32_t N,
                                                                const int32_t* __restrict__ row_src,
                                                                const int32_t* __restrict__ offsets, int E,
                                                                typename SF::T* __restrict__ s, int64_t s_sm,
                                                                int64_t s_skb) {
  const int32_t r = (int32_t)(blockIdx.x * 256u + threadIdx.x);
  if (r >= N) return;
  const int32_t R = offsets[E];
  int32_t t = row_src[r] / topk;
  t = t < 0 ? 0 : (t >= T ? T - 1 : t);
  const uint32_t kb0 = blockIdx.y * kGatherKB;
  const typename SF::T* src = tok + (int64_t)t * KB;
  typename SF::T v[kGatherKB];
#pragma unroll
  for (uint32_t j = 0; j < kGatherKB; ++j) v[j] = kb0 + j < KB ? src[kb0 + j] : typename SF::T{};
#pragma unroll
  for (uint32_t j = 0; j < kGatherKB; ++j)
    if (r < R && kb0 + j < KB) s[(int64_t)r * s_sm + (int64_t)(kb0 + j) * s_skb] = v[j];
}

// Workspace: the routing counts (2 nb E int32), then, from a 256-byte
// boundary, one 4-byte slot per token tile for the token-major scales.
static int64_t routing_bytes(int64_t N, int64_t E) {
  const int64_t nb = (N + kPairsPerBlock - 1) / kPairsPerBlock;
  return (2 * nb * E * (int64_t)sizeof(int32_t) + 255) / 256 * 256;
}

size_t dispatch_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t K) {
  const int64_t N = T * topk;
  if (N <= 0 || E <= 0) return 0;
  return (size_t)(routing_bytes(N, E) + T * (K / 128) * 4);
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
  const bool fused = nb > 0 && (int64_t)nb * E <= kFusedScan;
  if (!fused) hipLaunchKernelGGL(k_dispatch_scan, dim3(1), dim3(1024), 0, st, counts, nb, (int)E, base, offsets);
  if (nb > 0) {
    if (fused)
      hipLaunchKernelGGL(k_dispatch_scatter<true>, dim3(nb), dim3(64), 2 * lds, st, ids, N, (int)E, counts, dest,
                         row_src, nb, offsets);
    else
      hipLaunchKernelGGL(k_dispatch_scatter<false>, dim3(nb), dim3(64), lds, st, ids, N, (int)E, base, dest,
                         row_src, nb, offsets);
    const uint32_t KB = (uint32_t)(K / 128);
    const uint32_t n_tiles = (uint32_t)(T * KB);
    if (n_tiles > 0) {
      const uint32_t grid = (n_tiles + 16u * kDispU - 1) / (16u * kDispU);
      // a row's scales not contiguous: write them per token, then gather
      const bool token_scales = s_skb != 1;
      using ST = typename SF::T;
      ST* tok = reinterpret_cast<ST*>(static_cast<uint8_t*>(workspace) + routing_bytes(N, E));
      ST* s_q = token_scales ? tok : s;
      if (topk <= 8) {
        if (token_scales)
          hipLaunchKernelGGL((k_dispatch_quant<SF, 8, true>), dim3(grid), dim3(256), 0, st, x, ldx, KB, n_tiles,
                             (int)topk, dest, q, ldq, s_q, s_sm, s_skb);
        else
          hipLaunchKernelGGL((k_dispatch_quant<SF, 8, false>), dim3(grid), dim3(256), 0, st, x, ldx, KB, n_tiles,
                             (int)topk, dest, q, ldq, s_q, s_sm, s_skb);
      } else {
        if (token_scales)
          hipLaunchKernelGGL((k_dispatch_quant<SF, 0, true>), dim3(grid), dim3(256), 0, st, x, ldx, KB, n_tiles,
                             (int)topk, dest, q, ldq, s_q, s_sm, s_skb);
        else
          hipLaunchKernelGGL((k_dispatch_quant<SF, 0, false>), dim3(grid), dim3(256), 0, st, x, ldx, KB, n_tiles,
                             (int)topk, dest, q, ldq, s_q, s_sm, s_skb);
      }
      if (token_scales)
        hipLaunchKernelGGL((k_dispatch_gather_scales<SF>), dim3((unsigned)((N + 255) / 256), (KB + kGatherKB - 1) / kGatherKB),
                           dim3(256), 0, st,
                           tok, KB, (int)topk, (int32_t)T, (int32_t)N, row_src, offsets, (int)E, s, s_sm, s_skb);
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
