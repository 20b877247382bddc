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
//   * FP8 matrix-core mode: one 128-wide K chunk is exactly one
//     v_mfma_f32_16x16x128_f8f6f4 per 16x16 output sub-tile, so the chunk's
//     FP8 sum lands in a fresh FP32 temporary (C operand = inline 0) and is
//     promoted at once: acc = fma(t, sa * sw, acc) on the vector ALU.  The
//     promotion interval is the scale group, 128, since the scales change
//     every 128 along K.  The vector FMAs of one sub-tile overlap the matrix
//     core's work on the next (independent instructions of the same wave),
//     the register-level counterpart of the pages' two-warpgroup overlap.
//   * Exact mode (default): the same chunk as four K = 32 steps on the FP16
//     matrix core after an exact E4M3 -> FP16 conversion in registers, then
//     the same FP32 promotion.  gfx950's FP8 unit truncates inside groups of
//     eight products; its FP16 unit does not.
//   * Operands are K-contiguous in HBM and in LDS.  Each lane feeds 32
//     contiguous K bytes of one row to the MFMA; A and B use the same lane
//     layout, so whatever order the unit pairs the 128 K positions in, the
//     sum is the full chunk dot product.
//   * LDS rows are 128 bytes (one chunk); the 16-byte column c of row r is
//     stored at column c ^ s(r), a swizzle that keeps the fragment reads
//     (16 consecutive rows at one logical column) free of bank conflicts.
//   * Staging is LDS DMA (global_load_lds, no registers) into NSTAGE stages:
//     chunk kb + NSTAGE - 1 is in flight while chunk kb is multiplied.  The
//     per-chunk activation scales are one 4-byte load per row; stored
//     K-block-major ([K/128][M]) they are contiguous, which is the layout the
//     quantisers' callers should prefer.
//   * Power-of-two (E8M0) scales, the microscaling block-scale format the
//     pages relate the method to (P1 paragraph 4, P4 paragraph 3): the FP8
//     matrix core applies them itself (v_mfma_scale_f32_16x16x128_f8f6f4,
//     one byte per lane = per row of A or column of B and 32-value K block;
//     every lane of a row gets the same byte, as the block is 128 wide).
//     Two ways to accumulate: promote (each chunk into a zero C, then an
//     FP32 add on the vector ALU, the pages' promotion), or in the matrix
//     core (C = the running sum, no vector work).  Measured: the unit aligns
//     C and the chunk's 8-product group sums to the largest of them and
//     truncates about 24 bits below it, so keeping the sum in the matrix
//     core costs at most ~2^-20 of it per chunk, unlike the ~14 bits the
//     pages report for H800.
//     Scale bytes travel in the same 4-byte DMA slots as binary32 scales
//     (the aligned word holding the byte) and are read back as single bytes.
#include <mutex>
#include <type_traits>

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

// The same with E8M0 block scales (byte 127 = 1.0): D = 2^(sa - 127) *
// 2^(sb - 127) * A B^T + C, sa from the lane's row of A, sb from the lane's
// column of B.  With C = 0 the result is the unscaled one times the two
// powers of two, exactly.  C and the scaled group sums are added in a window
// about 24 bits below the largest of them (truncating below it).
__device__ __forceinline__ v4f mfma_16x16x128_fp8_e8m0(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Scale element type of a mode: binary32 for exact (0) and FP8 core (1),
// E8M0 bytes for the scaled matrix-core modes (2: promote, 3: in-core).
template <int MODE>
using ScaleOf = typename std::conditional<(MODE >= 2), uint8_t, float>::type;

// Aligned 32-bit word that holds the scale at p (the DMA moves words).
template <class S>
__device__ __forceinline__ const void* word_of(const S* p) {
  return reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(p) & ~(uintptr_t)3);
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
// s_waitcnt immediate: at most n of this wave's vector memory operations (LDS
// DMA included) outstanding and every LDS operation finished (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 left at 7, lgkmcnt 11:8 = 0).
constexpr int waitcnt_vm_lds(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Workgroup barrier without the implicit wait for all outstanding global
// loads that __syncthreads() adds (it would drain the DMA pipeline).  LDS
// visibility is the caller's job (waitcnt before it); the memory clobber
// keeps the compiler from moving memory operations across it.
__device__ __forceinline__ void barrier_no_drain() { asm volatile("s_barrier" ::: "memory"); }

// SKIP: the tile's waves all span its rows (WAVES_M = 1), so a tile with
// fewer rows than BM runs only the 16-row sub-tiles that hold rows (in
// quarter steps, chosen once per workgroup).
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int NSTAGE_ = 2, bool SKIP_ = false>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, NSTAGE = NSTAGE_;
  static constexpr bool SKIP = SKIP_;
  static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int NBW = BN >= 128 ? BN / 128 : 1;  // weight-scale blocks per tile
  static constexpr int SA_OFF = A_BYTES + B_BYTES;
  static constexpr int SW_OFF = SA_OFF + BM * 4;
  static constexpr int STAGE = SW_OFF + 256;   // weight scales, then a dummy slot at +128
  static constexpr int A_INS = BM / 8, B_INS = BN / 8;       // 1 KB DMA instructions per stage
  static constexpr int A_PER_W = (A_INS + NW - 1) / NW, B_PER_W = (B_INS + NW - 1) / NW;
  static constexpr int SA_INS = (BM + 63) / 64;
  // every wave issues the same DMA instructions per chunk: its A and B
  // slices and one 4-byte load (activation scales, weight scales, or a dummy)
  static constexpr int DMA_PER_CHUNK = A_PER_W + B_PER_W + 1;
  static_assert(A_INS % NW == 0 && B_INS % NW == 0, "uniform DMA count per wave");
  static_assert(NSTAGE >= 2 && (NSTAGE - 2) * DMA_PER_CHUNK <= 63, "vmcnt range");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile is a multiple of 16x16");
  static_assert(BM % 8 == 0 && BN % 8 == 0, "whole DMA instructions");
  static_assert(WN <= 128 && (128 % WN == 0), "a wave's columns share one weight-scale block");
  static_assert(SA_INS + 1 <= NW, "scale loads need a wave each");
  static_assert(BM % 64 == 0, "activation-scale loads fill whole 64-row slots");
  static_assert(NBW <= 64, "weight scales fit one instruction");
  static_assert(!SKIP || (WAVES_M == 1 && TM % 4 == 0), "row skipping needs full-height waves");
};

// Physical 16-byte column of logical column c in LDS row r.  Measured on
// gfx950: a 16-byte-per-lane LDS read runs at full rate (256 B/clk per CU)
// only when its 64 lanes fall in 64 different 16-byte slots modulo 1 KB.  A
// fragment read has rows r = 0 .. 15 (mod 16) at logical columns 2 g + h
// (g = 0 .. 3, h fixed); with 128-byte rows its slot is 8 (r mod 8) + the
// physical column, so rows r and r + 8 must share the eight physical columns
// between them.  Swizzle s(r) = (bit 3 of r) | (r & 6) does it (bit 0 of s
// differs between r and r + 8); c ^ (r / 2 mod 8), whose bit 0 does not,
// measured 142 B/clk.  s depends only on r mod 16, and c -> c ^ s is its own
// inverse.
__device__ __forceinline__ int lds_col(int c, int r) { return c ^ (((r >> 3) & 1) | (r & 6)); }

// ---- per-chunk arithmetic of one wave.  An engine holds the wave's
// accumulators; chunk() multiplies the K chunk staged at `base` (layout of
// TileCfg) into them and store() writes the wave's part of the tile.

// 16x16 sub-tiles: FP8 matrix core (MODE 1), exact products as four K = 32
// steps on the FP16 matrix core (MODE 0), or the FP8 matrix core with E8M0
// scales applied by the unit (MODE 2 promote, MODE 3 in-core).  Lane
// (l16, lgrp) feeds row l16 of a sub-tile with code bytes 32 lgrp ...
// 32 lgrp + 31 of the chunk.
template <class C, int MODE, bool LATE = true, bool IL = true>
struct Engine16 {
  v4f acc[C::TM][C::TN];
  int wm, wn, l16, lgrp;
  int a_off0, a_off1, b_off0, b_off1, sa_off, sw_idx;
  // E8M0 modes: low address bits of this lane's A scale and the wave's
  // weight scale at chunk 0, and the per-chunk strides; the byte sits at
  // (address mod 4) inside its DMA slot.
  uint32_t sa_lo = 0, sa_step = 0, sw_lo = 0, sw_step = 0;
  // Promoting modes (FP8 core, E8M0 promote, and the exact mode on
  // row-skipping tiles): the chunk sums of a chunk's last sub-tile row and their
  // scales wait here and are added at the start of the next chunk (after its
  // fragment loads are issued, so the wait on the matrix core overlaps LDS
  // latency instead of stalling every wave just before the barrier), or by
  // flush() after the last chunk.  Each accumulator still takes its chunk
  // terms in chunk order.
  v4f carry_t[C::TN];
  v4f carry_s;
  // Exact mode on full-height tiles: the chunk's last sub-tile row is
  // multiplied at the start of the next chunk (or by flush()), after the
  // barrier, so its matrix-core work covers the latency of the next chunk's
  // fragment loads.  Its operands wait in registers: the chunk's B fragments
  // (FP16), the row's A codes and its promotion scales.  Every accumulator
  // still takes its chunk terms in chunk order.
  static constexpr bool DEFER = MODE == 0 && !C::SKIP;
  // The fixed-order exact path takes the B part of the next chunk's DMA
  // request as a hook and issues it after the deferred row; the A codes and
  // scales still go out at the chunk top.  The larger B request then queues
  // behind the chunk's fragment reads instead of in front of them (about 2%
  // shorter than issuing everything at the top, on the dense and grouped
  // prefill shapes).
  static constexpr bool ISSUE_IN_CHUNK = DEFER && LATE && IL && C::TN == 4;
  v8h bhm[C::TN][4];
  uint4 pa_lo, pa_hi;
  v4f psc;

  __device__ __forceinline__ Engine16(int wave, int lane) {
    wm = wave / C::WAVES_N;
    wn = wave % C::WAVES_N;
    l16 = lane & 15;
    lgrp = lane >> 4;
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) acc[mi][ni] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ni = 0; ni < C::TN; ++ni) carry_t[ni] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    carry_s = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    // the first chunk's deferred row multiplies zeros into zero sums
#pragma unroll
    for (int ni = 0; ni < C::TN; ++ni)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bhm[ni][ks] = (v8h){};
    pa_lo = pa_hi = (uint4){0u, 0u, 0u, 0u};
    psc = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    // LDS byte offsets of this lane's fragment rows: logical columns 2 lgrp
    // and 2 lgrp + 1 of the 128-byte chunk row.  Sub-tile rows step by 16,
    // which keeps row & 15, so sub-tiles are base + 2048 * i; wave tile
    // origins are multiples of 16 rows as well.
    const int c0 = lgrp * 2;
    a_off0 = (wm * C::WM + l16) * 128 + (lds_col(c0, l16) << 4);
    a_off1 = (wm * C::WM + l16) * 128 + (lds_col(c0 + 1, l16) << 4);
    b_off0 = C::A_BYTES + (wn * C::WN + l16) * 128 + (lds_col(c0, l16) << 4);
    b_off1 = C::A_BYTES + (wn * C::WN + l16) * 128 + (lds_col(c0 + 1, l16) << 4);
    sa_off = MODE >= 2 ? C::SA_OFF + (wm * C::WM + l16) * 4 : C::SA_OFF + (wm * C::WM + lgrp * 4) * 4;
    sw_idx = (wn * C::WN) / 128;
  }

  // adds the carried row (the last chunk's last sub-tile row); call once
  // after the last chunk, with the TMA the chunks used
  template <int TMA = C::TM>
  __device__ __forceinline__ void flush() {
    if constexpr (DEFER) {
      exact_row(acc[TMA - 1], pa_lo, pa_hi, psc);
    } else if constexpr (MODE == 2) {
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) add4(acc[TMA - 1][ni], carry_t[ni]);
    } else if constexpr (MODE != 3) {
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) fma4(acc[TMA - 1][ni], carry_t[ni], carry_s);
    }
  }

  // TMA: sub-tile rows that hold rows of the tile (the rest are skipped)
  // With ISSUE_IN_CHUNK, `issue` (callable, no arguments) is run exactly
  // once inside the chunk; otherwise it must be null.
  template <int TMA = C::TM, class F = int>
  __device__ __forceinline__ void chunk(const uint8_t* base, int kb, F* issue = nullptr) {
    if constexpr (MODE >= 2) chunk_e8m0<TMA>(base, kb);
    else chunk_f32<TMA>(base, issue);
  }

  // E8M0: one scale byte per sub-tile row (this lane's row l16) and one per
  // wave for the weights; the unit multiplies them in
  template <int TMA>
  __device__ __forceinline__ void chunk_e8m0(const uint8_t* base, int kb) {
    const int swv = base[C::SW_OFF + sw_idx * 4 + ((sw_lo + (uint32_t)kb * sw_step) & 3u)];
    const int a_byte = sa_off + (int)((sa_lo + (uint32_t)kb * sa_step) & 3u);
    v8i bf[C::TN];
#pragma unroll
    for (int ni = 0; ni < C::TN; ++ni) {
      const uint4 lo = *reinterpret_cast<const uint4*>(base + b_off0 + ni * 2048);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + b_off1 + ni * 2048);
      bf[ni] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    uint4 alo = *reinterpret_cast<const uint4*>(base + a_off0);
    uint4 ahi = *reinterpret_cast<const uint4*>(base + a_off1);
    int sav = base[a_byte];
    if constexpr (MODE == 2 && IL && C::TN == 4 && !C::SKIP) {
      // fixed order, as in the FP8-core rows: each matrix operation is
      // followed by the previous row's four adds in its column; the first
      // row adds the previous chunk's carried row
      v4f tp[C::TN];
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) tp[ni] = carry_t[ni];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mi = 0; mi < TMA; ++mi) {
        uint4 nlo = alo, nhi = ahi;
        int nsa = sav;
        if (mi + 1 < TMA) {
          nlo = *reinterpret_cast<const uint4*>(base + a_off0 + (mi + 1) * 2048);
          nhi = *reinterpret_cast<const uint4*>(base + a_off1 + (mi + 1) * 2048);
          nsa = base[a_byte + (mi + 1) * 64];
        }
        const v8i af = (v8i){(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
        const int pr = mi > 0 ? mi - 1 : TMA - 1;  // the row added now
        v4f tc[C::TN];
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) {
          tc[ni] = mfma_16x16x128_fp8_e8m0(af, bf[ni], (v4f){0.0f, 0.0f, 0.0f, 0.0f}, sav, swv);
          add4(acc[pr][ni], tp[ni]);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) tp[ni] = tc[ni];
        alo = nlo;
        ahi = nhi;
        sav = nsa;
      }
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) carry_t[ni] = tp[ni];
      return;
    }
    if constexpr (MODE == 2) {
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) add4(acc[TMA - 1][ni], carry_t[ni]);  // the previous chunk's last row
    }
    // promote: the chunk sums of sub-tile row mi are added one row later,
    // after the next row's operations are issued, so no add waits on the
    // operation that produces its input
    v4f tp[C::TN];
#pragma unroll
    for (int mi = 0; mi < TMA; ++mi) {
      uint4 nlo = alo, nhi = ahi;
      int nsa = sav;
      if (mi + 1 < TMA) {
        nlo = *reinterpret_cast<const uint4*>(base + a_off0 + (mi + 1) * 2048);
        nhi = *reinterpret_cast<const uint4*>(base + a_off1 + (mi + 1) * 2048);
        nsa = base[a_byte + (mi + 1) * 64];
      }
      const v8i af = (v8i){(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
      if constexpr (MODE == 2) {
        v4f tc[C::TN];
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni)
          tc[ni] = mfma_16x16x128_fp8_e8m0(af, bf[ni], (v4f){0.0f, 0.0f, 0.0f, 0.0f}, sav, swv);
        // keep this order: the scheduler would otherwise pull the adds up
        // against the operations that produce them
        __builtin_amdgcn_sched_barrier(0);
        if (mi > 0) {
#pragma unroll
          for (int ni = 0; ni < C::TN; ++ni) add4(acc[mi - 1][ni], tp[ni]);
        }
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) tp[ni] = tc[ni];
      } else {
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) acc[mi][ni] = mfma_16x16x128_fp8_e8m0(af, bf[ni], acc[mi][ni], sav, swv);
      }
      alo = nlo;
      ahi = nhi;
      sav = nsa;
    }
    if constexpr (MODE == 2) {
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) carry_t[ni] = tp[ni];
    }
  }

  // a += t * s elementwise, four binary32 fused multiply-adds
  static __device__ __forceinline__ void fma4(v4f& a, const v4f& t, const v4f& s) {
    a[0] = __builtin_fmaf(t[0], s[0], a[0]);
    a[1] = __builtin_fmaf(t[1], s[1], a[1]);
    a[2] = __builtin_fmaf(t[2], s[2], a[2]);
    a[3] = __builtin_fmaf(t[3], s[3], a[3]);
  }

  // four binary32 adds (no packed instructions)
  static __device__ __forceinline__ void add4(v4f& a, const v4f& t) {
    a[0] += t[0];
    a[1] += t[1];
    a[2] += t[2];
    a[3] += t[3];
  }

  // one sub-tile row, exact products: four K = 32 steps against the B
  // fragments in bhm, then the promotion a += t * sc
  __device__ __forceinline__ void exact_row(v4f (&arow)[C::TN], const uint4& lo, const uint4& hi, const v4f& sc) {
    const uint32_t aw[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    v4f t[C::TN];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const v8h a = e4m3x8_to_f16(aw[2 * ks], aw[2 * ks + 1]);
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni)
        t[ni] = mfma_16x16x32_f16(a, bhm[ni][ks], ks == 0 ? (v4f){0.0f, 0.0f, 0.0f, 0.0f} : t[ni]);
    }
#pragma unroll
    for (int ni = 0; ni < C::TN; ++ni) fma4(arow[ni], t[ni], sc);
  }

  // one sub-tile row's chunk sums, exact products, without the promotion
  __device__ __forceinline__ void exact_mma(v4f (&t)[C::TN], const uint4& lo, const uint4& hi) {
    const uint32_t aw[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const v8h a = e4m3x8_to_f16(aw[2 * ks], aw[2 * ks + 1]);
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni)
        t[ni] = mfma_16x16x32_f16(a, bhm[ni][ks], ks == 0 ? (v4f){0.0f, 0.0f, 0.0f, 0.0f} : t[ni]);
    }
  }

  // One full-height row of the exact path (four K = 32 steps into the
  // chunk sums tc) with the instruction order fixed in the source: each
  // matrix operation is followed by two vector instructions, fenced so the
  // compiler keeps them together.  The vector work is the conversions of
  // the next K step's A codes, the previous row's promotion arow += tp * sp,
  // and this row's scale products sc = sa4 * swv.  Both waves of a SIMD run
  // this program in step behind the chunk barrier: left to itself the
  // compiler emits matrix operations and vector work in bursts of eight or
  // more, and the two waves' bursts collide instead of overlapping.
  // (four column sub-tiles: TN = 4)
  __device__ __forceinline__ void row_interleaved(v4f (&tc)[C::TN], const uint4& lo, const uint4& hi,
                                                  v4f (&arow)[C::TN], const v4f (&tp)[C::TN], const v4f& sp,
                                                  v4f& sc, const v4f& sa4, float swv) {
    const uint32_t aw[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    v2h ap[4][4];
    // pair p of K step ks: the two conversions of word 2 ks + p
    auto cvt2 = [&](int ks, int p) {
      ap[ks][2 * p] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(aw[2 * ks + p], 1.0f, false);
      ap[ks][2 * p + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(aw[2 * ks + p], 1.0f, true);
    };
    // promotion multiply-adds 2 k and 2 k + 1 (sub-tile k / 2, elements 2 (k % 2) ..)
    auto fma2 = [&](int k) {
      const int ni = k >> 1, e = (k & 1) * 2;
      arow[ni][e] = __builtin_fmaf(tp[ni][e], sp[e], arow[ni][e]);
      arow[ni][e + 1] = __builtin_fmaf(tp[ni][e + 1], sp[e + 1], arow[ni][e + 1]);
    };
    cvt2(0, 0);
    cvt2(0, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int ks = j >> 2, ni = j & 3;
      const v8h a = (v8h){ap[ks][0][0], ap[ks][0][1], ap[ks][1][0], ap[ks][1][1],
                          ap[ks][2][0], ap[ks][2][1], ap[ks][3][0], ap[ks][3][1]};
      tc[ni] = mfma_16x16x32_f16(a, bhm[ni][ks], ks == 0 ? (v4f){0.0f, 0.0f, 0.0f, 0.0f} : tc[ni]);
      // fillers: after operations 0, 1 of steps 0-2 the next step's
      // conversions; after 2, 3 of steps 0-2 and 0, 1 of step 3 the
      // promotion; after the last two the scale products
      if (ks < 3 && ni < 2) {
        cvt2(ks + 1, ni);
      } else if (j < 14) {
        fma2(ks < 3 ? 2 * ks + (ni - 2) : 6 + ni);
      } else {
        const int e = (j - 14) * 2;
        sc[e] = sa4[e] * swv;
        sc[e + 1] = sa4[e + 1] * swv;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // The previous chunk's deferred last row (A codes pa_lo / pa_hi, old FP16
  // B fragments in bhm) into the chunk sums tp, in the fixed order of
  // row_interleaved; the fillers are the row's remaining A conversions and
  // the new chunk's B conversions from blo / bhi: fragment (ni, ks) is
  // replaced two matrix operations after the one that read it (the last two
  // after the row).
  // Row 0's A codes and scales (alo, ahi, sa4) are requested halfway
  // through, when half the B words are converted and their registers free.
  __device__ __forceinline__ void deferred_interleaved(v4f (&tp)[C::TN], const uint4 (&blo)[C::TN],
                                                       const uint4 (&bhi)[C::TN], const uint8_t* base, uint4& alo,
                                                       uint4& ahi, v4f& sa4) {
    const uint32_t aw[8] = {pa_lo.x, pa_lo.y, pa_lo.z, pa_lo.w, pa_hi.x, pa_hi.y, pa_hi.z, pa_hi.w};
    v2h ap[4][4];
    auto cvt1 = [&](int ks, int q) {
      if (q & 1) ap[ks][q] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(aw[2 * ks + (q >> 1)], 1.0f, true);
      else ap[ks][q] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(aw[2 * ks + (q >> 1)], 1.0f, false);
    };
    auto newb = [&](int j) {
      const int ks = j >> 2, ni = j & 3;
      const uint32_t w0 = ks == 0 ? blo[ni].x : ks == 1 ? blo[ni].z : ks == 2 ? bhi[ni].x : bhi[ni].z;
      const uint32_t w1 = ks == 0 ? blo[ni].y : ks == 1 ? blo[ni].w : ks == 2 ? bhi[ni].y : bhi[ni].w;
      bhm[ni][ks] = e4m3x8_to_f16(w0, w1);
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) cvt1(0, q);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int ks = j >> 2, ni = j & 3;
      const v8h a = (v8h){ap[ks][0][0], ap[ks][0][1], ap[ks][1][0], ap[ks][1][1],
                          ap[ks][2][0], ap[ks][2][1], ap[ks][3][0], ap[ks][3][1]};
      tp[ni] = mfma_16x16x32_f16(a, bhm[ni][ks], ks == 0 ? (v4f){0.0f, 0.0f, 0.0f, 0.0f} : tp[ni]);
      if (ks < 3) cvt1(ks + 1, ni);
      if (j >= 2) newb(j - 2);
      if (j == 8) {
        alo = *reinterpret_cast<const uint4*>(base + a_off0);
        ahi = *reinterpret_cast<const uint4*>(base + a_off1);
        sa4 = *reinterpret_cast<const v4f*>(base + sa_off);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    newb(14);
    newb(15);
  }

  // binary32 scales: the chunk's FP32 sum, then promotion by the vector ALU
  template <int TMA, class F = int>
  __device__ __forceinline__ void chunk_f32(const uint8_t* base, F* issue = nullptr) {
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
      // A codes and scales one sub-tile row ahead; the chunk sums of row mi
      // are promoted one row later, after row mi + 1's operations are issued
      uint4 alo = *reinterpret_cast<const uint4*>(base + a_off0);
      uint4 ahi = *reinterpret_cast<const uint4*>(base + a_off1);
      v4f sa4 = *reinterpret_cast<const v4f*>(base + sa_off);
      if constexpr (IL && C::TN == 4 && !C::SKIP) {
        // fixed order: each matrix operation (32 cycles) is followed by the
        // promotion of the previous row's sub-tile in the same column (four
        // multiply-adds) and one scale product; the first row promotes the
        // previous chunk's carried row.  Left to itself the compiler issues
        // a row's four operations back to back and then twenty vector
        // instructions, and the two waves of a SIMD collide on both.
        v4f tp[C::TN];
        v4f sp = carry_s;
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) tp[ni] = carry_t[ni];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mi = 0; mi < TMA; ++mi) {
          uint4 nlo = alo, nhi = ahi;
          v4f nsa = sa4;
          if (mi + 1 < TMA) {
            nlo = *reinterpret_cast<const uint4*>(base + a_off0 + (mi + 1) * 2048);
            nhi = *reinterpret_cast<const uint4*>(base + a_off1 + (mi + 1) * 2048);
            nsa = *reinterpret_cast<const v4f*>(base + sa_off + (mi + 1) * 64);
          }
          const v8i af = (v8i){(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
          v4f tc[C::TN];
          v4f sc;
          const int pr = mi > 0 ? mi - 1 : TMA - 1;  // the row promoted now
#pragma unroll
          for (int ni = 0; ni < C::TN; ++ni) {
            tc[ni] = mfma_16x16x128_fp8(af, bf[ni]);
            fma4(acc[pr][ni], tp[ni], sp);
            sc[ni] = sa4[ni] * swv;
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int ni = 0; ni < C::TN; ++ni) tp[ni] = tc[ni];
          sp = sc;
          alo = nlo;
          ahi = nhi;
          sa4 = nsa;
        }
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) carry_t[ni] = tp[ni];
        carry_s = sp;
        return;
      }
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) fma4(acc[TMA - 1][ni], carry_t[ni], carry_s);  // the previous chunk's last row
      v4f tp[C::TN];
      v4f sp;
#pragma unroll
      for (int mi = 0; mi < TMA; ++mi) {
        uint4 nlo = alo, nhi = ahi;
        v4f nsa = sa4;
        if (mi + 1 < TMA) {
          nlo = *reinterpret_cast<const uint4*>(base + a_off0 + (mi + 1) * 2048);
          nhi = *reinterpret_cast<const uint4*>(base + a_off1 + (mi + 1) * 2048);
          nsa = *reinterpret_cast<const v4f*>(base + sa_off + (mi + 1) * 64);
        }
        const v8i af = (v8i){(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
        v4f tc[C::TN];
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) tc[ni] = mfma_16x16x128_fp8(af, bf[ni]);
        __builtin_amdgcn_sched_barrier(0);  // as in chunk_e8m0: keep the promotion behind them
        if (mi > 0) {
#pragma unroll
          for (int ni = 0; ni < C::TN; ++ni) fma4(acc[mi - 1][ni], tp[ni], sp);
        }
        const v4f sc = {sa4[0] * swv, sa4[1] * swv, sa4[2] * swv, sa4[3] * swv};
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) tp[ni] = tc[ni];
        sp = sc;
        alo = nlo;
        ahi = nhi;
        sa4 = nsa;
      }
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) carry_t[ni] = tp[ni];
      carry_s = sp;
    } else if constexpr (ISSUE_IN_CHUNK) {
      // exact products, last row deferred, the instruction order fixed in
      // the source.  All B fragments are requested first; the previous
      // chunk's last row runs against the old FP16 B fragments while the new
      // ones are converted in its shadow, each replacing an old fragment two
      // matrix operations after the row has read it.
      uint4 blo[C::TN], bhi[C::TN];
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) {
        blo[ni] = *reinterpret_cast<const uint4*>(base + b_off0 + ni * 2048);
        bhi[ni] = *reinterpret_cast<const uint4*>(base + b_off1 + ni * 2048);
      }
      uint4 alo, ahi;
      v4f sa4;
      v4f tp[C::TN];
      deferred_interleaved(tp, blo, bhi, base, alo, ahi, sa4);
      if constexpr (!std::is_same<F, int>::value) (*issue)();
      v4f sp = psc;
      int rp = TMA - 1;  // the row whose promotion is pending
#pragma unroll
      for (int mi = 0; mi + 1 < TMA; ++mi) {
        const uint4 nlo = *reinterpret_cast<const uint4*>(base + a_off0 + (mi + 1) * 2048);
        const uint4 nhi = *reinterpret_cast<const uint4*>(base + a_off1 + (mi + 1) * 2048);
        const v4f nsa = *reinterpret_cast<const v4f*>(base + sa_off + (mi + 1) * 64);
        v4f tc[C::TN];
        v4f scn;
        if (rp == TMA - 1) row_interleaved(tc, alo, ahi, acc[TMA - 1], tp, sp, scn, sa4, swv);
        else row_interleaved(tc, alo, ahi, acc[rp], tp, sp, scn, sa4, swv);
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) tp[ni] = tc[ni];
        sp = scn;
        rp = mi;
        alo = nlo;
        ahi = nhi;
        sa4 = nsa;
      }
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) fma4(acc[rp][ni], tp[ni], sp);
      pa_lo = alo;
      pa_hi = ahi;
      psc = (v4f){sa4[0] * swv, sa4[1] * swv, sa4[2] * swv, sa4[3] * swv};
    } else if constexpr (DEFER) {
      // exact products, last row deferred.  Half the B fragments are
      // requested before the previous chunk's last row runs, the rest after
      // it has taken their registers' old values.
      constexpr int H = C::TN / 2;
      uint4 blo[H], bhi[H];
#pragma unroll
      for (int ni = 0; ni < H; ++ni) {
        blo[ni] = *reinterpret_cast<const uint4*>(base + b_off0 + ni * 2048);
        bhi[ni] = *reinterpret_cast<const uint4*>(base + b_off1 + ni * 2048);
      }
      uint4 alo = *reinterpret_cast<const uint4*>(base + a_off0);
      uint4 ahi = *reinterpret_cast<const uint4*>(base + a_off1);
      v4f sa4 = *reinterpret_cast<const v4f*>(base + sa_off);
      // the previous chunk's last row.  With LATE, its promotion (and each
      // row's below) is issued after the next row's matrix operations,
      // behind a scheduling barrier, so no multiply-add waits on the
      // operation that produces its input.
      v4f tp[C::TN];
      v4f sp = psc;
      int rp = TMA - 1;  // the row whose promotion is pending
      if constexpr (LATE) exact_mma(tp, pa_lo, pa_hi);
      else exact_row(acc[TMA - 1], pa_lo, pa_hi, psc);
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) {
        uint4 lo, hi;
        if (ni < H) {
          lo = blo[ni < H ? ni : 0];
          hi = bhi[ni < H ? ni : 0];
        } else {
          lo = *reinterpret_cast<const uint4*>(base + b_off0 + ni * 2048);
          hi = *reinterpret_cast<const uint4*>(base + b_off1 + ni * 2048);
        }
        bhm[ni][0] = e4m3x8_to_f16(lo.x, lo.y);
        bhm[ni][1] = e4m3x8_to_f16(lo.z, lo.w);
        bhm[ni][2] = e4m3x8_to_f16(hi.x, hi.y);
        bhm[ni][3] = e4m3x8_to_f16(hi.z, hi.w);
      }
#pragma unroll
      for (int mi = 0; mi + 1 < TMA; ++mi) {
        const uint4 nlo = *reinterpret_cast<const uint4*>(base + a_off0 + (mi + 1) * 2048);
        const uint4 nhi = *reinterpret_cast<const uint4*>(base + a_off1 + (mi + 1) * 2048);
        const v4f nsa = *reinterpret_cast<const v4f*>(base + sa_off + (mi + 1) * 64);
        const v4f sc = {sa4[0] * swv, sa4[1] * swv, sa4[2] * swv, sa4[3] * swv};
        if constexpr (LATE) {
          v4f tc[C::TN];
          exact_mma(tc, alo, ahi);
          __builtin_amdgcn_sched_barrier(0);
          if (rp == TMA - 1) {
#pragma unroll
            for (int ni = 0; ni < C::TN; ++ni) fma4(acc[TMA - 1][ni], tp[ni], sp);
          } else {
#pragma unroll
            for (int ni = 0; ni < C::TN; ++ni) fma4(acc[rp][ni], tp[ni], sp);
          }
#pragma unroll
          for (int ni = 0; ni < C::TN; ++ni) tp[ni] = tc[ni];
          sp = sc;
          rp = mi;
        } else {
          exact_row(acc[mi], alo, ahi, sc);
        }
        alo = nlo;
        ahi = nhi;
        sa4 = nsa;
      }
      if constexpr (LATE) {
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) fma4(acc[rp][ni], tp[ni], sp);
      }
      pa_lo = alo;
      pa_hi = ahi;
      psc = (v4f){sa4[0] * swv, sa4[1] * swv, sa4[2] * swv, sa4[3] * swv};
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
      uint4 alo = *reinterpret_cast<const uint4*>(base + a_off0);
      uint4 ahi = *reinterpret_cast<const uint4*>(base + a_off1);
      v4f sa4 = *reinterpret_cast<const v4f*>(base + sa_off);
#pragma unroll
      for (int ni = 0; ni < C::TN; ++ni) fma4(acc[TMA - 1][ni], carry_t[ni], carry_s);  // the previous chunk's last row
#pragma unroll
      for (int mi = 0; mi < TMA; ++mi) {
        uint4 nlo = alo, nhi = ahi;
        v4f nsa = sa4;
        if (mi + 1 < TMA) {
          nlo = *reinterpret_cast<const uint4*>(base + a_off0 + (mi + 1) * 2048);
          nhi = *reinterpret_cast<const uint4*>(base + a_off1 + (mi + 1) * 2048);
          nsa = *reinterpret_cast<const v4f*>(base + sa_off + (mi + 1) * 64);
        }
        const uint32_t aw[8] = {alo.x, alo.y, alo.z, alo.w, ahi.x, ahi.y, ahi.z, ahi.w};
        // K step ks: convert 8 codes of A, then one MFMA into each of the TN
        // independent sub-tile chains
        v4f t[C::TN];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const v8h a = e4m3x8_to_f16(aw[2 * ks], aw[2 * ks + 1]);
#pragma unroll
          for (int ni = 0; ni < C::TN; ++ni)
            t[ni] = mfma_16x16x32_f16(a, bh[ni][ks], ks == 0 ? (v4f){0.0f, 0.0f, 0.0f, 0.0f} : t[ni]);
        }
        const v4f sc = {sa4[0] * swv, sa4[1] * swv, sa4[2] * swv, sa4[3] * swv};
        if (mi + 1 < TMA) {
#pragma unroll
          for (int ni = 0; ni < C::TN; ++ni) fma4(acc[mi][ni], t[ni], sc);
        } else {
#pragma unroll
          for (int ni = 0; ni < C::TN; ++ni) carry_t[ni] = t[ni];
          carry_s = sc;
        }
        alo = nlo;
        ahi = nhi;
        sa4 = nsa;
      }
    }
  }

  // lane holds rows lgrp*4 + i, column l16 of each 16x16 sub-tile
  // PARTIAL 0: BF16 C; 1: binary32 sums to part[m * ldc + n]; 2: binary32
  // sums to the tile's own block, part[(m - row_begin) * BN + n - n0]
  template <int PARTIAL>
  __device__ __forceinline__ void store(int64_t row_begin, int64_t row_end, int64_t n0, uint16_t* __restrict__ c,
                                        float* __restrict__ part, int64_t ldc) {
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t gr = row_begin + wm * C::WM + mi * 16 + lgrp * 4 + i;
        if (gr < row_end) {
          if constexpr (PARTIAL == 2) {
            float* prow = part + (gr - row_begin) * C::BN + wn * C::WN + l16;
#pragma unroll
            for (int ni = 0; ni < C::TN; ++ni) prow[ni * 16] = acc[mi][ni][i];
          } else if constexpr (PARTIAL == 1) {
            float* prow = part + gr * ldc + n0 + wn * C::WN + l16;
#pragma unroll
            for (int ni = 0; ni < C::TN; ++ni) prow[ni * 16] = acc[mi][ni][i];
          } else {
            uint16_t* crow = c + gr * ldc + n0 + wn * C::WN + l16;
#pragma unroll
            for (int ni = 0; ni < C::TN; ++ni) crow[ni * 16] = (uint16_t)bf16_rne(acc[mi][ni][i]);
          }
        }
      }
    }
  }
};

// One output tile [row_begin, row_begin + BM) x [n0, n0 + BN) over the K
// chunks [kb_begin, kb_end); rows >= row_end are neither read (their loads
// repeat row row_end - 1) nor written.  Writes BF16 C, or with PARTIAL the
// binary32 sums of its chunks to part[m * ldc + n] (PARTIAL 1, split-K
// workspace) or to the tile's own BM x BN block at part (PARTIAL 2).
template <class C, int MODE, int PARTIAL = 0>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ qa, int64_t lda,
                                          const ScaleOf<MODE>* __restrict__ sa, int64_t sa_sm, int64_t sa_skb,
                                          int64_t row_begin, int64_t row_end,
                                          const uint8_t* __restrict__ qw, int64_t ldw,
                                          const ScaleOf<MODE>* __restrict__ sw, int64_t sw_snb, int64_t sw_skb,
                                          int64_t n0, uint16_t* __restrict__ c, float* __restrict__ part,
                                          int64_t ldc, int kb_begin, int kb_end, uint8_t* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- this lane's DMA sources: slot s = ins * 64 + lane holds row s / 8 at
  // physical column s % 8, i.e. the logical column whose lds_col is s % 8
  // (the XOR is its own inverse).  Row = 8 * ins + lane / 8 with ins = wave +
  // j * NW (NW even), so row & 15 = 8 * (wave & 1) + lane / 8 for every j and
  // one column offset serves all of them; sources are the tile base plus
  // 32-bit offsets.
  static_assert(C::NW % 2 == 0, "instruction parity follows the wave's");
  const int dcol = lds_col(lane & 7, ((wave & 1) << 3) | (lane >> 3)) * 16;
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
  const ScaleOf<MODE>* s_src = nullptr;  // activation scales (waves < SA_INS) or weight scales (wave SA_INS)
  if (wave < C::SA_INS) {
    int64_t gr = row_begin + wave * 64 + lane;
    gr = gr < row_end ? gr : row_end - 1;
    s_src = sa + gr * sa_sm;
  } else if (wave == C::SA_INS) {
    s_src = sw + ((n0 >> 7) + (lane < C::NBW ? lane : 0)) * sw_snb;
  }

  // what: kDmaAll, or the two parts of a split request, kDmaA (A codes and
  // both scale slots) and kDmaB (B codes)
  constexpr int kDmaAll = 0, kDmaA = 1, kDmaB = 2;
  auto issue = [&](int kb, int stage, int what = kDmaAll) {
    uint8_t* base = lds + stage * C::STAGE;
    const uint8_t* at = a_tile + (int64_t)kb * 128;
    const uint8_t* bt = b_tile + (int64_t)kb * 128;
    if (what != kDmaB) {
#pragma unroll
      for (int j = 0; j < C::A_PER_W; ++j) dma16(at + a_src[j], base + (wave + j * C::NW) * 1024);
    }
    if (what != kDmaA) {
#pragma unroll
      for (int j = 0; j < C::B_PER_W; ++j) dma16(bt + b_src[j], base + C::A_BYTES + (wave + j * C::NW) * 1024);
    }
    if (what == kDmaB) return;
    if (wave < C::SA_INS) {
      dma4(word_of(s_src + (int64_t)kb * sa_skb), base + C::SA_OFF + wave * 256);
    } else if (wave == C::SA_INS) {
      if (lane < C::NBW) dma4(word_of(s_src + (int64_t)kb * sw_skb), base + C::SW_OFF);
    } else if (lane == 0) {
      dma4(word_of(sw), base + C::SW_OFF + 128);  // dummy: keeps the per-wave DMA count uniform
    }
  };

  Engine16<C, MODE> eng(wave, lane);
  if constexpr (MODE >= 2) {
    // slot r of the A scales holds the word of tile row r (clamped rows are
    // never stored, so their byte offset does not matter)
    const int64_t ar = row_begin + eng.wm * C::WM + eng.l16;
    eng.sa_lo = (uint32_t)reinterpret_cast<uintptr_t>(sa) + (uint32_t)(ar * sa_sm);
    eng.sa_step = (uint32_t)sa_skb;
    eng.sw_lo = (uint32_t)reinterpret_cast<uintptr_t>(sw) + (uint32_t)(((n0 >> 7) + eng.sw_idx) * sw_snb);
    eng.sw_step = (uint32_t)sw_skb;
  }

  // NSTAGE-deep pipeline: chunk kb + NSTAGE - 1 is requested while chunk kb
  // is multiplied.  At the top of iteration kb, the wait leaves the chunks
  // issued after kb in flight; the barrier then publishes chunk kb to every
  // wave and frees the stage of chunk kb - 1, which the next request reuses.
#pragma unroll
  for (int p = 0; p < C::NSTAGE - 1; ++p)
    if (kb_begin + p < kb_end) issue(kb_begin + p, p);
  // tma = 0: the wave multiplies nothing but still issues its DMA share and
  // meets every barrier (one per chunk, as in the other instantiations).
  auto kloop = [&](auto tma) {
    for (int kb = kb_begin; kb < kb_end; ++kb) {
      const int it = kb - kb_begin;
      const int stage = it % C::NSTAGE;
      if (kb + C::NSTAGE - 2 < kb_end) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds((C::NSTAGE - 2) * C::DMA_PER_CHUNK));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds(0));
      barrier_no_drain();
      // every part of chunk kb + NSTAGE - 1's request goes out in this
      // iteration, so the wait at the top of the next one counts as before
      const bool more = kb + C::NSTAGE - 1 < kb_end;
      const int nstage = (it + C::NSTAGE - 1) % C::NSTAGE;
      if constexpr (decltype(eng)::ISSUE_IN_CHUNK && decltype(tma)::value > 0) {
        if (more) issue(kb + C::NSTAGE - 1, nstage, kDmaA);
        auto rest = [&]() {
          if (more) issue(kb + C::NSTAGE - 1, nstage, kDmaB);
        };
        eng.template chunk<decltype(tma)::value>(lds + stage * C::STAGE, kb, &rest);
      } else {
        if (more) issue(kb + C::NSTAGE - 1, nstage);
        if constexpr (decltype(tma)::value > 0) eng.template chunk<decltype(tma)::value>(lds + stage * C::STAGE, kb);
      }
    }
    if constexpr (decltype(tma)::value > 0) eng.template flush<decltype(tma)::value>();
  };
  // A wave whose rows all lie past the tile's last row (the short last slot
  // of a grouped expert) runs the loop without arithmetic: its SIMD partner
  // then has the matrix core and the vector ALU to itself.  Uniform per wave.
  if (C::WAVES_M > 1 && (int64_t)eng.wm * C::WM >= row_end - row_begin) {
    kloop(std::integral_constant<int, 0>{});
  } else if constexpr (C::SKIP) {
    // sub-tile rows past the tile's last row hold no rows: skip them
    const int64_t rows = row_end - row_begin;
    if (rows <= C::BM / 4) kloop(std::integral_constant<int, C::TM / 4>{});
    else if (rows <= C::BM / 2) kloop(std::integral_constant<int, C::TM / 2>{});
    else if (rows <= 3 * C::BM / 4) kloop(std::integral_constant<int, 3 * C::TM / 4>{});
    else kloop(std::integral_constant<int, C::TM>{});
  } else {
    kloop(std::integral_constant<int, C::TM>{});
  }
  eng.template store<PARTIAL>(row_begin, row_end, n0, c, part, ldc);
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

using BigCfg = TileCfg<256, 256, 2, 4>;      // FP8 matrix core, large M
using BigExactCfg = TileCfg<192, 256, 2, 4>; // exact products, large M (FP16 operands need more registers)
using SmallCfg = TileCfg<64, 128, 1, 4>;
// Exact-mode products with short K (at most 16 chunks), dense and grouped:
// with one workgroup per CU each tile's pipeline fill and C stores stand
// alone, and the large tiles end on a partly filled round.  These 67 KB
// workgroups run two per CU, so one covers the other's.  Measured (us):
// grouped, 32 experts, 16384 rows, K 2048, N 7168: 596 -> 550; dense
// 8192 x 7168 x 2048: 228 -> 218, 4096 x 7168 x 2048: 136 -> 112,
// 8192 x 4096 x 1024: 77 -> 70, 16384 x 7168 x 2048: 441 -> 432.  The FP8
// modes ran 7-14% slower with it (their operand bytes per flop double),
// and so do not use it.
using ShortKExactCfg = TileCfg<128, 128, 2, 2>;
constexpr int64_t kShortK = 2048;
using SplitCfg = TileCfg<64, 128, 1, 4, 3>;  // split-K, memory-bound small M: 3 stages, 2 per CU
// Grouped GEMM with few rows per expert (decode batches): the expert weights
// dominate the traffic.  64 x 128 tiles with full-height waves: a slot runs
// only the 16-row sub-tiles that hold rows, and two stages (49 KB of LDS)
// leave room for three workgroups per CU; the slots of one expert share each
// weight column block in L2 (the grouped kernel orders this configuration's
// tiles by column block per XCD, slot fastest).
using MoeDecodeCfg = TileCfg<64, 128, 1, 4, 2, true>;

// ---------------------------------------------------------------------------
// Activation quantisation fused into the A-load: the CDNA counterpart of the
// FP8 cast during the global -> shared transfer that the pages propose (P3
// paragraph 3), which removes the HBM round trip of quantised activations
// (P2 paragraph 1).  A arrives as BF16.  Per K chunk each 16-lane group holds
// one row's 1x128 tile in registers (16 bytes a lane), takes its max-abs,
// derives the scale pair and codes with the same helpers as
// k_quant_act_1x128, and writes codes and scale into the LDS stage in the
// layout the engine reads.  The weights keep their DMA.  With EMIT, the
// workgroups of n-tile 0 also store the codes and scales to HBM
// (bit-identical to fgq_quant_act_1x128); HBM stores count in vmcnt on this
// chip, so that variant waits for all memory operations each chunk.
template <class C>
struct FusedA {
  static constexpr int ROWS_PER_INS = 4;                 // 4 rows of 256 B per wave instruction
  static constexpr int LOADS = C::BM / (ROWS_PER_INS * C::NW);
  static constexpr int DMA_PER_CHUNK = C::B_PER_W + 1;   // W slices + one weight-scale (or dummy) load
  static_assert(C::BM % (ROWS_PER_INS * C::NW) == 0, "whole A rows per thread");
  static_assert(C::NSTAGE >= 2 && (C::NSTAGE - 2) * DMA_PER_CHUNK <= 63, "vmcnt range");
};

template <class C, int MODE, bool EMIT, bool PARTIAL = false>
__device__ __forceinline__ void gemm_tile_fused(const uint16_t* __restrict__ a, int64_t lda, int64_t row_begin,
                                                int64_t row_end, const uint8_t* __restrict__ qw, int64_t ldw,
                                                const float* __restrict__ sw, int64_t sw_snb, int64_t sw_skb,
                                                int64_t n0, uint16_t* __restrict__ c, float* __restrict__ part,
                                                int64_t ldc, int kb_begin, int kb_end, uint8_t* lds,
                                                uint8_t* __restrict__ qa_out, int64_t ldq,
                                                float* __restrict__ sa_out, int64_t sa_sm, int64_t sa_skb) {
  using F = FusedA<C>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // weight staging as in gemm_tile
  static_assert(C::NW % 2 == 0, "instruction parity follows the wave's");
  const int dcol = lds_col(lane & 7, ((wave & 1) << 3) | (lane >> 3)) * 16;
  const uint8_t* b_tile = qw + n0 * ldw;
  uint32_t b_src[C::B_PER_W];
#pragma unroll
  for (int j = 0; j < C::B_PER_W; ++j) {
    const int r = (wave + j * C::NW) * 8 + (lane >> 3);
    b_src[j] = (uint32_t)((r < C::BN ? r : 0) * ldw) + dcol;
  }
  const float* sw_src = sw + ((n0 >> 7) + (lane < C::NBW ? lane : 0)) * sw_snb;
  auto issue_w = [&](int kb, int stage) {
    uint8_t* base = lds + stage * C::STAGE;
    const uint8_t* bt = b_tile + (int64_t)kb * 128;
#pragma unroll
    for (int j = 0; j < C::B_PER_W; ++j) dma16(bt + b_src[j], base + C::A_BYTES + (wave + j * C::NW) * 1024);
    if (wave == 0) {
      if (lane < C::NBW) dma4(sw_src + (int64_t)kb * sw_skb, base + C::SW_OFF);
    } else if (lane == 0) {
      dma4(sw, base + C::SW_OFF + 128);  // dummy: keeps the per-wave DMA count uniform
    }
  };

  // this thread's A rows: tile row (wave + j NW) * 4 + lane / 16, bytes 16 l16 .. of the chunk
  const uint16_t* a_tile = a + row_begin * lda + l16 * 8;
  const int64_t a_last = row_end - 1 - row_begin;
  uint32_t a_off[F::LOADS];
  int a_row[F::LOADS];
#pragma unroll
  for (int j = 0; j < F::LOADS; ++j) {
    a_row[j] = (wave + j * C::NW) * F::ROWS_PER_INS + (lane >> 4);
    a_off[j] = (uint32_t)((a_row[j] < a_last ? a_row[j] : a_last) * lda);  // clamped rows: loads stay in bounds
  }
  auto load_a = [&](int kb, uint4* v) {
#pragma unroll
    for (int j = 0; j < F::LOADS; ++j) v[j] = *reinterpret_cast<const uint4*>(a_tile + a_off[j] + (int64_t)kb * 128);
  };
  const bool emit = EMIT && qa_out != nullptr;
  auto put_a = [&](int kb, const uint4* v, uint8_t* base) {
#pragma unroll
    for (int j = 0; j < F::LOADS; ++j) {
      float f[8];
      unpack8(v[j], f);
      const float amax = max16(absmax8(f));
      float sc, r;
      group_scales(amax, sc, r);
      const uint2 codes = cast8(f, r);
      const int rr = a_row[j];
      *reinterpret_cast<uint2*>(base + rr * 128 + (lds_col(l16 >> 1, rr) << 4) + (l16 & 1) * 8) = codes;
      if (l16 == 0) *reinterpret_cast<float*>(base + C::SA_OFF + rr * 4) = sc;
      if (emit && rr <= a_last) {
        const int64_t gr = row_begin + rr;
        *reinterpret_cast<uint2*>(qa_out + gr * ldq + (int64_t)kb * 128 + l16 * 8) = codes;
        if (l16 == 0) sa_out[gr * sa_sm + (int64_t)kb * sa_skb] = sc;
      }
    }
  };

  // the exact engine's late promotion would spill here, beside the A ring
  Engine16<C, MODE, false> eng(wave, lane);
  // A tiles travel two chunks ahead in a two-slot register ring: chunk k
  // lives in ring[(k - kb_begin) & 1].  Within an iteration the weight
  // request goes out before the A loads, and the prologue keeps that order,
  // so at the top of iteration kb the operations issued after the weight
  // request of chunk kb are exactly the next iteration's: (NSTAGE - 2)
  // weight requests and one set of A loads (none in the last iteration).
  static_assert(C::NSTAGE == 2 || C::NSTAGE == 3, "ring and wait counts are laid out for 2 or 3 stages");
  uint4 ring[2][F::LOADS];
  if constexpr (C::NSTAGE == 2) {
    load_a(kb_begin, ring[0]);
    issue_w(kb_begin, 0);
    if (kb_begin + 1 < kb_end) load_a(kb_begin + 1, ring[1]);
  } else {
    issue_w(kb_begin, 0);
    load_a(kb_begin, ring[0]);
    if (kb_begin + 1 < kb_end) {
      issue_w(kb_begin + 1, 1);
      load_a(kb_begin + 1, ring[1]);
    }
  }
  put_a(kb_begin, ring[0], lds);
  constexpr int kAhead = (C::NSTAGE - 2) * F::DMA_PER_CHUNK + F::LOADS;
  static_assert(kAhead <= 63, "vmcnt range");

  auto step = [&](auto par, int kb) {
    constexpr int P = decltype(par)::value;  // (kb - kb_begin) & 1
    const int it = kb - kb_begin;
    const int stage = it % C::NSTAGE;
    if (!emit && kb + 1 < kb_end) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds(kAhead));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds(0));
    barrier_no_drain();
    if (kb + C::NSTAGE - 1 < kb_end) issue_w(kb + C::NSTAGE - 1, (it + C::NSTAGE - 1) % C::NSTAGE);
    if (kb + 2 < kb_end) load_a(kb + 2, ring[P]);  // slot of chunk kb, written to LDS last iteration
    eng.chunk(lds + stage * C::STAGE, kb);
    // the next chunk's A goes to the stage every wave finished before this
    // iteration's barrier
    if (kb + 1 < kb_end) put_a(kb + 1, ring[P ^ 1], lds + ((it + 1) % C::NSTAGE) * C::STAGE);
  };
  for (int kb = kb_begin; kb < kb_end; kb += 2) {
    step(std::integral_constant<int, 0>{}, kb);
    if (kb + 1 < kb_end) step(std::integral_constant<int, 1>{}, kb + 1);
  }
  eng.flush();
  eng.template store<PARTIAL>(row_begin, row_end, n0, c, part, ldc);
}

template <class C, int MODE, bool EMIT>
__global__ __launch_bounds__(C::NT) void k_gemm_fused_a(const uint16_t* __restrict__ a, int64_t lda,
                                                        const uint8_t* __restrict__ qw, int64_t ldw,
                                                        const float* __restrict__ sw, int64_t sw_snb, int64_t sw_skb,
                                                        uint16_t* __restrict__ c, int64_t ldc, int64_t M, int tiles_m,
                                                        int KB, uint8_t* __restrict__ qa_out, int64_t ldq,
                                                        float* __restrict__ sa_out, int64_t sa_sm, int64_t sa_skb) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::NSTAGE * C::STAGE];
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tm, tn);
  gemm_tile_fused<C, MODE, EMIT>(a, lda, (int64_t)tm * C::BM, M, qw, ldw, sw, sw_snb, sw_skb, (int64_t)tn * C::BN, c,
                                 nullptr, ldc, 0, KB, lds, tn == 0 ? qa_out : nullptr, ldq, sa_out, sa_sm, sa_skb);
}

template <class C, int MODE, bool EMIT>
__global__ __launch_bounds__(C::NT) void k_gemm_fused_a_splitk(const uint16_t* __restrict__ a, int64_t lda,
                                                               const uint8_t* __restrict__ qw, int64_t ldw,
                                                               const float* __restrict__ sw, int64_t sw_snb,
                                                               int64_t sw_skb, float* __restrict__ part, int64_t M,
                                                               int64_t N, int tiles_m, int tiles, int KB, int S,
                                                               uint8_t* __restrict__ qa_out, int64_t ldq,
                                                               float* __restrict__ sa_out, int64_t sa_sm,
                                                               int64_t sa_skb) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::NSTAGE * C::STAGE];
  const int split = blockIdx.x / tiles;
  int tm, tn;
  tile_of(blockIdx.x % tiles, tiles, tiles_m, tm, tn);
  const int kb0 = (int)((int64_t)split * KB / S), kb1 = (int)((int64_t)(split + 1) * KB / S);
  gemm_tile_fused<C, MODE, EMIT, true>(a, lda, (int64_t)tm * C::BM, M, qw, ldw, sw, sw_snb, sw_skb,
                                       (int64_t)tn * C::BN, nullptr, part + (int64_t)split * M * N, N, kb0, kb1, lds,
                                       tn == 0 ? qa_out : nullptr, ldq, sa_out, sa_sm, sa_skb);
}

template <class C, int MODE>
__global__ __launch_bounds__(C::NT) void k_gemm_fp8_bs(const uint8_t* __restrict__ qa, int64_t lda,
                                                       const ScaleOf<MODE>* __restrict__ sa, int64_t sa_sm,
                                                       int64_t sa_skb, const uint8_t* __restrict__ qw,
                                                       int64_t ldw, const ScaleOf<MODE>* __restrict__ sw,
                                                       int64_t sw_snb, int64_t sw_skb,
                                                       uint16_t* __restrict__ c, int64_t ldc, int64_t M,
                                                       int tiles_m, int KB, int G) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::NSTAGE * C::STAGE];
  // G: the tiles of the whole product; the grid may cover only the first
  // ones (k_gemm_fp8_bs_tail takes the rest)
  int tm, tn;
  tile_of(blockIdx.x, G, tiles_m, tm, tn);
  gemm_tile<C, MODE>(qa, lda, sa, sa_sm, sa_skb, (int64_t)tm * C::BM, M, qw, ldw, sw, sw_snb, sw_skb,
                     (int64_t)tn * C::BN, c, nullptr, ldc, 0, KB, lds);
}

// Split-K for small M (memory-bound shapes): workgroup (tile, split) sums
// chunks [split * KB / S, (split + 1) * KB / S) into part[split][M][N].
template <class C, int MODE>
__global__ __launch_bounds__(C::NT) void k_gemm_fp8_bs_splitk(const uint8_t* __restrict__ qa, int64_t lda,
                                                              const ScaleOf<MODE>* __restrict__ sa, int64_t sa_sm,
                                                              int64_t sa_skb, const uint8_t* __restrict__ qw,
                                                              int64_t ldw, const ScaleOf<MODE>* __restrict__ sw,
                                                              int64_t sw_snb, int64_t sw_skb,
                                                              float* __restrict__ part, int64_t M, int64_t N,
                                                              int tiles_m, int tiles, int KB, int S) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::NSTAGE * C::STAGE];
  const int split = blockIdx.x / tiles;
  int tm, tn;
  tile_of(blockIdx.x % tiles, tiles, tiles_m, tm, tn);
  const int kb0 = (int)((int64_t)split * KB / S), kb1 = (int)((int64_t)(split + 1) * KB / S);
  gemm_tile<C, MODE, 1>(qa, lda, sa, sa_sm, sa_skb, (int64_t)tm * C::BM, M, qw, ldw, sw, sw_snb, sw_skb,
                           (int64_t)tn * C::BN, nullptr, part + (int64_t)split * M * N, N, kb0, kb1, lds);
}

// C[m, n] = bf16(sum over splits s = 0, 1, ... of part[s][m][n]), in split
// order (deterministic).  Eight consecutive outputs per thread.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int S, int64_t M,
                                                       int64_t N, uint16_t* __restrict__ c, int64_t ldc) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= M * N) return;
  const int64_t m = i / N, n = i - m * N;
  float v[8];
  const float4* p = reinterpret_cast<const float4*>(part + i);
  float4 x = p[0], y = p[1];
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  for (int s = 1; s < S; ++s) {
    p = reinterpret_cast<const float4*>(part + (int64_t)s * M * N + i);
    x = p[0];
    y = p[1];
    v[0] += x.x; v[1] += x.y; v[2] += x.z; v[3] += x.w; v[4] += y.x; v[5] += y.y; v[6] += y.z; v[7] += y.w;
  }
  uint4 o;
  o.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
  o.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
  o.z = bf16_rne(v[4]) | (bf16_rne(v[5]) << 16);
  o.w = bf16_rne(v[6]) | (bf16_rne(v[7]) << 16);
  *reinterpret_cast<uint4*>(c + m * ldc + n) = o;
}

// The last, partly filled round of a large dense product: its `rem` tiles
// (the last ones of the tile order) are split S ways along K so that they
// spread over the compute units the round would leave idle.  Workgroup i
// takes tile t = i mod rem and K part s = i / rem, and writes its binary32
// sums to the tile's own BM x BN block part[s * rem + t].
template <class C, int MODE>
__global__ __launch_bounds__(C::NT) void k_gemm_fp8_bs_tail(const uint8_t* __restrict__ qa, int64_t lda,
                                                            const ScaleOf<MODE>* __restrict__ sa, int64_t sa_sm,
                                                            int64_t sa_skb, const uint8_t* __restrict__ qw,
                                                            int64_t ldw, const ScaleOf<MODE>* __restrict__ sw,
                                                            int64_t sw_snb, int64_t sw_skb,
                                                            float* __restrict__ part, int64_t M, int tiles_m,
                                                            int G, int rem, int KB, int S) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::NSTAGE * C::STAGE];
  const int t = (int)blockIdx.x % rem, split = (int)blockIdx.x / rem;
  int tm, tn;
  tile_of(G - rem + t, G, tiles_m, tm, tn);
  const int kb0 = (int)((int64_t)split * KB / S), kb1 = (int)((int64_t)(split + 1) * KB / S);
  gemm_tile<C, MODE, 2>(qa, lda, sa, sa_sm, sa_skb, (int64_t)tm * C::BM, M, qw, ldw, sw, sw_snb, sw_skb,
                        (int64_t)tn * C::BN, nullptr, part + ((int64_t)split * rem + t) * C::BM * C::BN, C::BN,
                        kb0, kb1, lds);
}

// C of the tail tiles: the sum of their S partial blocks in split order
// (deterministic), eight consecutive outputs per thread; tile t = blockIdx.y.
template <class C>
__global__ __launch_bounds__(256) void k_tail_reduce(const float* __restrict__ part, int S, int rem, int G,
                                                     int tiles_m, int64_t M, uint16_t* __restrict__ c, int64_t ldc) {
  const int t = (int)blockIdx.y;
  const int e = ((int)blockIdx.x * 256 + (int)threadIdx.x) * 8;
  if (e >= C::BM * C::BN) return;
  int tm, tn;
  tile_of(G - rem + t, G, tiles_m, tm, tn);
  const int r = e / C::BN, col = e - r * C::BN;
  const int64_t row = (int64_t)tm * C::BM + r;
  if (row >= M) return;
  float v[8];
  const int64_t blk = (int64_t)C::BM * C::BN;
  const float4* p = reinterpret_cast<const float4*>(part + (int64_t)t * blk + e);
  float4 x = p[0], y = p[1];
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  for (int sp = 1; sp < S; ++sp) {
    p = reinterpret_cast<const float4*>(part + ((int64_t)sp * rem + t) * blk + e);
    x = p[0];
    y = p[1];
    v[0] += x.x; v[1] += x.y; v[2] += x.z; v[3] += x.w; v[4] += y.x; v[5] += y.y; v[6] += y.z; v[7] += y.w;
  }
  uint4 o;
  o.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
  o.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
  o.z = bf16_rne(v[4]) | (bf16_rne(v[5]) << 16);
  o.w = bf16_rne(v[6]) | (bf16_rne(v[7]) << 16);
  *reinterpret_cast<uint4*>(c + row * ldc + (int64_t)tn * C::BN + col) = o;
}

// Split-K plan for a dense shape: S > 1 when M is small enough that the
// output tiles alone cannot fill the 256 compute units several times over.
// The same function decides the workspace size and the launch.
struct SplitPlan {
  int S;
  int tiles_m, tiles_n;
};
static SplitPlan split_plan(int64_t M, int64_t N, int64_t K) {
  SplitPlan p{1, 0, 0};
  if (M > 128 || N % SplitCfg::BN != 0) return p;
  p.tiles_m = (int)((M + SplitCfg::BM - 1) / SplitCfg::BM);
  p.tiles_n = (int)(N / SplitCfg::BN);
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  const int KB = (int)(K / 128);
  // one round of workgroups at two per CU (512): a second, partly filled
  // round and short splits both cost more than the deeper reduction saves
  int S = (int)(512 / tiles);
  if (S > KB / 4) S = KB / 4;                 // at least 4 chunks per split
  if (S > 16) S = 16;
  p.S = S < 2 ? 1 : S;
  return p;
}

// Large dense products run one workgroup per compute unit (gfx950 has
// 256), so a product of G tiles takes G / 256 rounds.  When the last round
// holds at most half the units' worth of tiles, those rem tiles are split
// S ways along K (k_gemm_fp8_bs_tail, k_tail_reduce) if the caller's
// workspace holds their partial blocks; otherwise the plain launch runs.
constexpr int kComputeUnits = 256;
struct TailPlan {
  int S = 1;
  int G = 0, rem = 0, tiles_m = 0;
};
template <class C>
static TailPlan tail_plan(int64_t M, int64_t N, int64_t K) {
  static_assert(C::NSTAGE * C::STAGE > 80 * 1024, "one workgroup per compute unit");
  TailPlan p;
  if (M <= 128 || N % C::BN != 0) return p;
  p.tiles_m = (int)((M + C::BM - 1) / C::BM);
  p.G = p.tiles_m * (int)(N / C::BN);
  p.rem = p.G % kComputeUnits;
  const int KB = (int)(K / 128);
  if (p.G < kComputeUnits || p.rem == 0 || p.rem > kComputeUnits / 2) return p;
  int S = kComputeUnits / p.rem;
  if (S > KB / 4) S = KB / 4;  // at least 4 chunks per part
  if (S > 16) S = 16;
  p.S = S < 2 ? 1 : S;
  return p;
}
template <class C>
static size_t tail_bytes(const TailPlan& p) {
  return p.S > 1 ? (size_t)p.S * (size_t)p.rem * C::BM * C::BN * sizeof(float) : 0;
}

size_t gemm_workspace_required(int64_t M, int64_t N, int64_t K) {
  const SplitPlan p = split_plan(M, N, K);
  return p.S > 1 ? (size_t)p.S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  size_t b = gemm_workspace_required(M, N, K);
  // exact products with short K take ShortKExactCfg, which is not split
  const size_t t0 = K > kShortK ? tail_bytes<BigExactCfg>(tail_plan<BigExactCfg>(M, N, K)) : 0;
  const size_t t1 = tail_bytes<BigCfg>(tail_plan<BigCfg>(M, N, K));
  if (t0 > b) b = t0;
  if (t1 > b) b = t1;
  return b;
}

template <class C, int MODE>
static void launch_dense(const uint8_t* qa, int64_t lda, const ScaleOf<MODE>* sa, int64_t sa_sm, int64_t sa_skb,
                         const uint8_t* qw, int64_t ldw, const ScaleOf<MODE>* sw, int64_t sw_snb, int64_t sw_skb,
                         uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int tiles_m = (int)((M + C::BM - 1) / C::BM);
  const int tiles_n = (int)(N / C::BN);
  hipLaunchKernelGGL((k_gemm_fp8_bs<C, MODE>), dim3(tiles_m * tiles_n), dim3(C::NT), 0, st, qa, lda, sa, sa_sm,
                     sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, tiles_m, (int)(K / 128), tiles_m * tiles_n);
}

template <class C, int MODE>
static void launch_dense_tail(const TailPlan& p, const uint8_t* qa, int64_t lda, const ScaleOf<MODE>* sa,
                              int64_t sa_sm, int64_t sa_skb, const uint8_t* qw, int64_t ldw, const ScaleOf<MODE>* sw,
                              int64_t sw_snb, int64_t sw_skb, uint16_t* c, int64_t ldc, int64_t M, int64_t K,
                              float* part, hipStream_t st) {
  const int KB = (int)(K / 128);
  hipLaunchKernelGGL((k_gemm_fp8_bs<C, MODE>), dim3(p.G - p.rem), dim3(C::NT), 0, st, qa, lda, sa, sa_sm, sa_skb,
                     qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, p.tiles_m, KB, p.G);
  hipLaunchKernelGGL((k_gemm_fp8_bs_tail<C, MODE>), dim3(p.rem * p.S), dim3(C::NT), 0, st, qa, lda, sa, sa_sm,
                     sa_skb, qw, ldw, sw, sw_snb, sw_skb, part, M, p.tiles_m, p.G, p.rem, KB, p.S);
  hipLaunchKernelGGL((k_tail_reduce<C>), dim3((C::BM * C::BN / 8 + 255) / 256, p.rem), dim3(256), 0, st, part, p.S,
                     p.rem, p.G, p.tiles_m, M, c, ldc);
}

template <int MODE>
static void launch_splitk(const SplitPlan& p, const uint8_t* qa, int64_t lda, const ScaleOf<MODE>* sa, int64_t sa_sm,
                          int64_t sa_skb, const uint8_t* qw, int64_t ldw, const ScaleOf<MODE>* sw, int64_t sw_snb,
                          int64_t sw_skb, uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                          float* part, hipStream_t st) {
  using C = SplitCfg;
  const int tiles = p.tiles_m * p.tiles_n;
  hipLaunchKernelGGL((k_gemm_fp8_bs_splitk<C, MODE>), dim3(tiles * p.S), dim3(C::NT), 0, st, qa, lda, sa, sa_sm,
                     sa_skb, qw, ldw, sw, sw_snb, sw_skb, part, M, N, p.tiles_m, tiles, (int)(K / 128), p.S);
  const int64_t groups = (M * N + 7) / 8;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st, part, p.S, M, N,
                     c, ldc);
}

// Large-M tile of a mode: FP16 operands (exact mode) need more registers.
template <int MODE>
using BigOf = typename std::conditional<MODE == 0, BigExactCfg, BigCfg>::type;

// Dense in-core products: the same 256x256 tile over sixteen waves (64x64
// each, four per SIMD, at most 128 VGPRs).  Only the in-core mode, which
// keeps its sums in the matrix core, fits that without spills.  Measured on
// 8192 x 18432 x 7168 in two runs: 873 -> 840 us and 873 -> 859 us
// (bit-identical); the grouped kernel ran 4% slower with it (937 -> 976 us
// on 32 experts), so it stays dense.
using BigIncoreCfg = TileCfg<256, 256, 4, 4>;
static_assert(BigIncoreCfg::BM == BigCfg::BM && BigIncoreCfg::BN == BigCfg::BN,
              "gemm_workspace_bytes sizes the last-round split from BigCfg's tiles");
template <int MODE>
using DenseBigOf = typename std::conditional<MODE == 3, BigIncoreCfg, BigOf<MODE>>::type;

template <int MODE>
static hipError_t gemm_dispatch(const uint8_t* qa, int64_t lda, const ScaleOf<MODE>* sa, int64_t sa_sm,
                                int64_t sa_skb, const uint8_t* qw, int64_t ldw, const ScaleOf<MODE>* sw,
                                int64_t sw_snb, int64_t sw_skb, uint16_t* c, int64_t ldc, int64_t M, int64_t N,
                                int64_t K, void* workspace, size_t workspace_bytes, hipStream_t st) {
  const SplitPlan p = split_plan(M, N, K);
  float* part = static_cast<float*>(workspace);
  const bool big = M > 128 && N % 256 == 0;
  if (p.S > 1) {
    launch_splitk<MODE>(p, qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, part, st);
  } else if (MODE == 0 && K <= kShortK && M > 128) {
    if constexpr (MODE == 0)
      launch_dense<ShortKExactCfg, 0>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, st);
  } else if (big) {
    using C = DenseBigOf<MODE>;
    const TailPlan tp = tail_plan<C>(M, N, K);
    const bool room = workspace && (reinterpret_cast<uintptr_t>(workspace) & 15) == 0 &&
                      workspace_bytes >= tail_bytes<C>(tp);
    if (tp.S > 1 && room)
      launch_dense_tail<C, MODE>(tp, qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, K, part, st);
    else
      launch_dense<C, MODE>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, st);
  } else {
    launch_dense<SmallCfg, MODE>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, st);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_fp8_blockscaled(const uint8_t* qa, int64_t lda, const float* sa, int64_t sa_sm,
                                       int64_t sa_skb, const uint8_t* qw, int64_t ldw, const float* sw,
                                       int64_t sw_snb, int64_t sw_skb, uint16_t* c, int64_t ldc,
                                       int64_t M, int64_t N, int64_t K, int mode, void* workspace,
                                       size_t workspace_bytes, hipStream_t st) {
  if (mode == 1)
    return gemm_dispatch<1>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, workspace,
                            workspace_bytes, st);
  return gemm_dispatch<0>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, workspace,
                            workspace_bytes, st);
}

// ---------------------------------------------------------------------------
// Scratch for callers that cannot allocate device memory (code under graph
// capture, allocation-free serving loops): fgq_gemm_fp8_blockscaled_noalloc
// runs the products of fgq_gemm_fp8_blockscaled with this file-scope array as
// their workspace.  Every GPU holds its own copy at its own address, resolved
// once per device with hipGetSymbolAddress; host code never passes the
// array's name itself to a kernel (on the host it is only a stand-in).
// Nothing in it needs to start at zero: every call writes the partial sums
// it reads back.  Calls that overlap on one GPU share it and race.  48 MiB
// holds the split-K partial sums of every small-M shape (at most 256 tiles of
// 64 x 128, split at most 512 / tiles ways: at most 16.8 MB) and the
// last-round split of an 8192 x 18432 product (47.2 MB).
constexpr size_t kNoAllocScratchBytes = (size_t)48 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

hipError_t launch_gemm_fp8_e8m0(const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t sa_sm, int64_t sa_skb,
                                const uint8_t* qw, int64_t ldw, const uint8_t* sw, int64_t sw_snb, int64_t sw_skb,
                                uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, int in_core,
                                void* workspace, size_t workspace_bytes, hipStream_t st) {
  if (in_core)
    return gemm_dispatch<3>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, workspace,
                            workspace_bytes, st);
  return gemm_dispatch<2>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, workspace,
                            workspace_bytes, st);
}

// BF16 activations quantised inside the GEMM (see gemm_tile_fused).  Same
// split plan and workspace as the FP8-operand GEMM; large M uses 128 x 256
// tiles, which leave the registers for the A tile in flight.
using FusedBigCfg = TileCfg<128, 256, 2, 4>;

template <int MODE, bool EMIT>
static void fused_dispatch(const uint16_t* a, int64_t lda, const uint8_t* qw, int64_t ldw, const float* sw,
                           int64_t sw_snb, int64_t sw_skb, uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                           void* workspace, uint8_t* qa_out, int64_t ldq, float* sa_out, int64_t sa_sm,
                           int64_t sa_skb, hipStream_t st) {
  const SplitPlan p = split_plan(M, N, K);
  const int KB = (int)(K / 128);
  if (p.S > 1) {
    using C = SplitCfg;
    const int tiles = p.tiles_m * p.tiles_n;
    float* part = static_cast<float*>(workspace);
    hipLaunchKernelGGL((k_gemm_fused_a_splitk<C, MODE, EMIT>), dim3(tiles * p.S), dim3(C::NT), 0, st, a, lda, qw, ldw,
                       sw, sw_snb, sw_skb, part, M, N, p.tiles_m, tiles, KB, p.S, qa_out, ldq, sa_out, sa_sm, sa_skb);
    const int64_t groups = (M * N + 7) / 8;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st, part, p.S, M, N, c,
                       ldc);
    return;
  }
  if (M > 128 && N % 256 == 0) {
    using C = FusedBigCfg;
    const int tiles_m = (int)((M + C::BM - 1) / C::BM);
    hipLaunchKernelGGL((k_gemm_fused_a<C, MODE, EMIT>), dim3(tiles_m * (int)(N / C::BN)), dim3(C::NT), 0, st, a, lda,
                       qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, tiles_m, KB, qa_out, ldq, sa_out, sa_sm, sa_skb);
    return;
  }
  using C = SmallCfg;
  const int tiles_m = (int)((M + C::BM - 1) / C::BM);
  hipLaunchKernelGGL((k_gemm_fused_a<C, MODE, EMIT>), dim3(tiles_m * (int)(N / C::BN)), dim3(C::NT), 0, st, a, lda, qw,
                     ldw, sw, sw_snb, sw_skb, c, ldc, M, tiles_m, KB, qa_out, ldq, sa_out, sa_sm, sa_skb);
}

hipError_t launch_gemm_bf16a_fp8_blockscaled(const uint16_t* a, int64_t lda, const uint8_t* qw, int64_t ldw,
                                             const float* sw, int64_t sw_snb, int64_t sw_skb, uint16_t* c,
                                             int64_t ldc, int64_t M, int64_t N, int64_t K, int mode,
                                             uint8_t* qa_out, int64_t ldq, float* sa_out, int64_t sa_sm,
                                             int64_t sa_skb, void* workspace, hipStream_t st) {
  const bool emit = qa_out != nullptr;
  if (mode == 1) {
    if (emit) fused_dispatch<1, true>(a, lda, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, workspace, qa_out, ldq, sa_out, sa_sm, sa_skb, st);
    else fused_dispatch<1, false>(a, lda, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, workspace, nullptr, 0, nullptr, 0, 0, st);
  } else {
    if (emit) fused_dispatch<0, true>(a, lda, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, workspace, qa_out, ldq, sa_out, sa_sm, sa_skb, st);
    else fused_dispatch<0, false>(a, lda, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, workspace, nullptr, 0, nullptr, 0, 0, st);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped (MoE) variant.  The linear workgroup id maps (as above) to an
// (m-tile slot, n-tile) pair; slots run over all experts in expert order.
// The slot -> (expert, rows) map is computed on the GPU from offsets[] (a
// running sum of the per-expert slot counts, done by every wave), so the
// host never reads the routing result.  The grid is sized for the most
// slots the sizes allow; workgroup ids are dealt over the real tiles and
// the rest leave at once.
template <class C, int MODE>
__global__ __launch_bounds__(C::NT) void k_grouped_gemm_fp8_bs(
    const uint8_t* __restrict__ qa, int64_t lda, const ScaleOf<MODE>* __restrict__ sa, int64_t sa_sm,
    int64_t sa_skb, const uint8_t* __restrict__ qw, int64_t ldw, int64_t w_es,
    const ScaleOf<MODE>* __restrict__ sw, int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
    const int32_t* __restrict__ offsets, int E, int64_t total_rows, uint16_t* __restrict__ c,
    int64_t ldc, int slots, int KB) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::NSTAGE * C::STAGE];
  // Every wave resolves the tile by itself on the scalar unit: the offsets
  // are read with uniform addresses (scalar loads through the scalar cache),
  // with no LDS and no barrier, so each wave starts its first requests as
  // soon as it can.  (A workgroup-wide scan here cost about 15%: workgroups
  // started unevenly and lost the L2 sharing of their neighbours.)
  constexpr int kBatch = 16;  // experts per batch of scalar loads
  // slots of expert e0 + j from the batch o[0..kBatch], rows clamped to [0, total_rows)
  auto batch = [&](int e0, int32_t* o) {
#pragma unroll
    for (int j = 0; j <= kBatch; ++j) o[j] = offsets[e0 + j < E ? e0 + j : E];
  };
  const int32_t nrows = (int32_t)total_rows;  // < 2^31 (checked on the host)
  auto clamp_rows = [&](int32_t a, int32_t b, int32_t& r0, int32_t& r1) {
    r0 = a < 0 ? 0 : (a > nrows ? nrows : a);
    r1 = b < r0 ? r0 : (b > nrows ? nrows : b);
    return (int)((uint32_t)(r1 - r0 + C::BM - 1) / (uint32_t)C::BM);
  };
  // the real number of row slots first: workgroup ids are dealt over the
  // real tiles only, so they spread evenly over the XCDs and the
  // launch-size bound's spare slots do not leave a partial last round
  int real_slots = 0;
  for (int e0 = 0; e0 < E; e0 += kBatch) {
    int32_t o[kBatch + 1];
    batch(e0, o);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      int32_t r0, r1;
      if (e0 + j < E) real_slots += clamp_rows(o[j], o[j + 1], r0, r1);
    }
  }
  const int tiles_n = (int)gridDim.x / slots;
  const int G = real_slots * tiles_n;
  if ((int)blockIdx.x >= G) return;  // no tile for this workgroup: the whole workgroup leaves
  int slot, tn;
  if constexpr (C::SKIP) {
    // decode-shaped experts, weight-bound: each XCD owns a range of weight
    // column blocks over all slots, slot fastest, so every (expert, column
    // block) is fetched by one XCD and an expert's slots share it in L2
    // (with m-tile groups an expert's slots could straddle two XCDs)
    const int q = G / kXcds, r = G % kXcds;
    const int xcd = (int)blockIdx.x % kXcds, local = (int)blockIdx.x / kXcds;
    const int logical = xcd * q + (xcd < r ? xcd : r) + local;
    tn = logical / real_slots;
    slot = logical - tn * real_slots;
  } else {
    tile_of(blockIdx.x, G, real_slots, slot, tn);
  }
  int e = -1;
  int64_t row_begin = 0, row_end = 0;
  int carried = 0;  // slots of the experts before e0 + j
  for (int e0 = 0; e0 < E && e < 0; e0 += kBatch) {
    int32_t o[kBatch + 1];
    batch(e0, o);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      int32_t r0 = 0, r1 = 0;
      const int t = e0 + j < E ? clamp_rows(o[j], o[j + 1], r0, r1) : 0;
      if (e < 0 && slot < carried + t) {
        e = e0 + j;
        row_begin = r0 + (int64_t)(slot - carried) * C::BM;
        row_end = r1;
      }
      carried += t;
    }
  }
  if (e < 0) return;  // unreachable for slot < real_slots
  gemm_tile<C, MODE>(qa, lda, sa, sa_sm, sa_skb, row_begin, row_end, qw + (int64_t)e * w_es, ldw,
                     sw + (int64_t)e * sw_es, sw_snb, sw_skb, (int64_t)tn * C::BN, c, nullptr, ldc, 0, KB, lds);
}

template <class C, int MODE>
static void launch_grouped(const uint8_t* qa, int64_t lda, const ScaleOf<MODE>* sa, int64_t sa_sm, int64_t sa_skb,
                           const uint8_t* qw, int64_t ldw, int64_t w_es, const ScaleOf<MODE>* sw, int64_t sw_snb,
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

template <int MODE>
static hipError_t grouped_dispatch(const uint8_t* qa, int64_t lda, const ScaleOf<MODE>* sa, int64_t sa_sm,
                                   int64_t sa_skb, const uint8_t* qw, int64_t ldw, int64_t w_es,
                                   const ScaleOf<MODE>* sw, int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
                                   const int32_t* offsets, int64_t E, int64_t total_rows, uint16_t* c, int64_t ldc,
                                   int64_t N, int64_t K, hipStream_t st) {
  // decode regime: at most 128 rows per expert on average (the host decides
  // from the sizes alone; offsets stay on the device)
  const bool decode = total_rows <= 128 * E && N % MoeDecodeCfg::BN == 0;
  if constexpr (MODE == 0) {
    if (!decode && K <= kShortK && total_rows > 128) {
      launch_grouped<ShortKExactCfg, 0>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es,
                                        offsets, E, total_rows, c, ldc, N, K, st);
      return hipGetLastError();
    }
  }
  if (decode)
    launch_grouped<MoeDecodeCfg, MODE>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets,
                                       E, total_rows, c, ldc, N, K, st);
  else if (N % 256 == 0 && total_rows > 128)
    launch_grouped<BigOf<MODE>, MODE>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets,
                                      E, total_rows, c, ldc, N, K, st);
  else
    launch_grouped<SmallCfg, MODE>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets, E,
                                   total_rows, c, ldc, N, K, st);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_fp8_blockscaled(const uint8_t* qa, int64_t lda, const float* sa,
                                               int64_t sa_sm, int64_t sa_skb, const uint8_t* qw,
                                               int64_t ldw, int64_t w_es, const float* sw,
                                               int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
                                               const int32_t* offsets, int64_t E, int64_t total_rows,
                                               uint16_t* c, int64_t ldc, int64_t N, int64_t K, int mode,
                                               hipStream_t st) {
  if (mode == 1)
    return grouped_dispatch<1>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets, E,
                               total_rows, c, ldc, N, K, st);
  return grouped_dispatch<0>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets, E,
                             total_rows, c, ldc, N, K, st);
}

hipError_t launch_grouped_gemm_fp8_e8m0(const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t sa_sm,
                                        int64_t sa_skb, const uint8_t* qw, int64_t ldw, int64_t w_es,
                                        const uint8_t* sw, int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
                                        const int32_t* offsets, int64_t E, int64_t total_rows, uint16_t* c,
                                        int64_t ldc, int64_t N, int64_t K, int in_core, hipStream_t st) {
  if (in_core)
    return grouped_dispatch<3>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets, E,
                               total_rows, c, ldc, N, K, st);
  return grouped_dispatch<2>(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es, offsets, E,
                             total_rows, c, ldc, N, K, st);
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

// Diagnostic: one v_mfma_scale_f32_16x16x128_f8f6f4 as the E8M0 GEMMs issue
// it (the lane's row / column byte, the same for its four 32-value blocks).
__global__ __launch_bounds__(64) void k_debug_mfma_e8m0(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                        const uint8_t* __restrict__ sa, const uint8_t* __restrict__ sb,
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
  c = mfma_16x16x128_fp8_e8m0(av, bv, c, sa[l16], sb[l16]);
  for (int i = 0; i < 4; ++i) d[(lgrp * 4 + i) * 16 + l16] = c[i];
}

hipError_t launch_debug_mfma_e8m0(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                                  const float* cin, float* d, hipStream_t st) {
  hipLaunchKernelGGL(k_debug_mfma_e8m0, dim3(1), dim3(64), 0, st, a, b, sa, sb, cin, d);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Diagnostic: the matrix cores' sustained rate and the shader clock under
// load.  Every wave runs `iters` rounds of 8 independent matrix operations on
// register operands (no memory traffic in the loop) and records the shader
// clock counter (s_memtime) and the constant 100 MHz counter (s_memrealtime)
// before and after, so the host gets both the operation rate and the clock
// the chip held while running it.  kind 0: v_mfma_f32_16x16x128_f8f6f4 (FP8,
// 65536 flops); 1: v_mfma_f32_16x16x32_f16 (16384 flops); 2:
// v_mfma_f32_32x32x16_f16 (32768 flops).  out[4 * wave + 0..3] = clock start,
// clock end, real start, real end; sink receives a reduction of the results.
typedef float v16f __attribute__((ext_vector_type(16)));

template <int KIND>
__global__ __launch_bounds__(256) void k_debug_mfma_loop(int64_t iters, uint64_t* __restrict__ out,
                                                         float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  // operands from the lane id so the compiler cannot fold them
  const int seed = lane * 0x01010101 + 0x3C3C3C3C;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  float red = 0.0f;
  if constexpr (KIND == 0) {
    const v8i a = (v8i){seed, seed ^ 1, seed ^ 2, seed ^ 3, seed ^ 4, seed ^ 5, seed ^ 6, seed ^ 7};
    const v8i b = (v8i){seed ^ 8, seed ^ 9, seed ^ 10, seed ^ 11, seed ^ 12, seed ^ 13, seed ^ 14, seed ^ 15};
    v4f acc[8];
    for (int j = 0; j < 8; ++j) acc[j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 0, 0, 0, 0, 0, 0);
    for (int j = 0; j < 8; ++j) red += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else if constexpr (KIND == 1) {
    const _Float16 h = (_Float16)(float)(lane & 7);
    const v8h a = (v8h){h, h, h, h, h, h, h, h};
    const v8h b = (v8h){h, (_Float16)1.0f, h, h, h, h, h, h};
    v4f acc[8];
    for (int j = 0; j < 8; ++j) acc[j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
    for (int j = 0; j < 8; ++j) red += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else {
    const _Float16 h = (_Float16)(float)(lane & 7);
    const v8h a = (v8h){h, h, h, h, h, h, h, h};
    const v8h b = (v8h){h, (_Float16)1.0f, h, h, h, h, h, h};
    v16f acc[4];
    for (int j = 0; j < 4; ++j)
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    for (int64_t i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
      }
    for (int j = 0; j < 4; ++j)
      for (int e = 0; e < 16; ++e) red += acc[j][e];
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    out[4 * wave + 0] = c0;
    out[4 * wave + 1] = c1;
    out[4 * wave + 2] = r0;
    out[4 * wave + 3] = r1;
  }
  sink[(int64_t)wave * 64 + lane] = red;
}

hipError_t launch_debug_mfma_loop(int kind, int64_t iters, int64_t waves, uint64_t* out, float* sink,
                                  hipStream_t st) {
  const dim3 grid((uint32_t)(waves / 4));
  if (kind == 0) hipLaunchKernelGGL(k_debug_mfma_loop<0>, grid, dim3(256), 0, st, iters, out, sink);
  else if (kind == 1) hipLaunchKernelGGL(k_debug_mfma_loop<1>, grid, dim3(256), 0, st, iters, out, sink);
  else hipLaunchKernelGGL(k_debug_mfma_loop<2>, grid, dim3(256), 0, st, iters, out, sink);
  return hipGetLastError();
}

}  // namespace fgq
