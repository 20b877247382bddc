/*
 * fgq.h -- fine-grained FP8 quantisation and block-scaled FP8 GEMM for
 * AMD Instinct MI355X (gfx950).  C ABI of libfgq.so.
 *
 * The method (DeepSeek-V3 FP8 mixed precision, as described on the source
 * pages; they have no section numbers, so passages are located by page and
 * paragraph):
 *   P1  "DeepSeek core readings" notes page (why-be.why-be.co.kr)
 *   P2  Q&A board page (xn--9g3bo1gtkw0l8ubf92bgle.kr)
 *   P3  "How I Improved My Deepseek In In The Future" (youlimart.com)
 *   P4  "How Google Is Changing How We Method Deepseek" (xn--jj0bz6z98ct0a29q.com)
 *
 * FP8 format: OCP E4M3 ("E4M3FN"; bias 7, largest finite 448, NaN 0x7F/0xFF).
 * Codes are stored as one byte each.  Scales are IEEE binary32 and are the
 * dequantisation multipliers: value ~= decode(code) * scale.
 *
 * Conventions shared by every call:
 *   - Every data pointer is a DEVICE pointer on the calling thread's current
 *     HIP device.  The caller allocates and frees every buffer; the library
 *     never allocates, frees, synchronises, or reads device data on the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is enqueued on it, in stream order; calls return before the
 *     GPU work completes.  Asynchronous faults surface at the caller's next
 *     synchronisation.
 *   - Leading dimensions (ld*) and strides are in ELEMENTS of the pointed-to
 *     type (BF16 = 2 bytes, E4M3 = 1 byte, float = 4 bytes).  Row-major,
 *     with the K (inner) dimension contiguous.
 *   - Arguments are validated on the host before any HIP call.  On an error
 *     nothing is enqueued and a status > 0 is returned.  A call with an empty
 *     problem (M == 0, rows == 0, B == 0 or E == 0) returns FGQ_OK and
 *     launches nothing.
 *   - Not checked (undefined behaviour): outputs that alias inputs or each
 *     other; NaN or Inf inputs; device data that breaks a documented
 *     invariant (e.g. grouped offsets).
 *   - Thread-safe: the library holds no mutable global state other than a
 *     thread-local copy of the last HIP error code.
 */
#ifndef FGQ_H
#define FGQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fgq_status_t;

enum {
  FGQ_OK = 0,
  FGQ_ERR_NULL = 1,        /* a required pointer is NULL */
  FGQ_ERR_SHAPE = 2,       /* a negative size, or an inconsistent shape */
  FGQ_ERR_ALIGN = 3,       /* a pointer is not aligned as documented */
  FGQ_ERR_STRIDE = 4,      /* a leading dimension / stride is too small or misaligned */
  FGQ_ERR_UNSUPPORTED = 5, /* sizes outside what the kernels support (e.g. K % 128 != 0) */
  FGQ_ERR_HIP = 6,         /* a HIP launch failed; see fgq_last_hip_error() */
  FGQ_ERR_SCRATCH = 7      /* fgq_gemm_fp8_blockscaled_noalloc: the product needs more scratch than it holds */
};

#define FGQ_ABI_VERSION 6

/*
 * fgq_quant_act_1x128 -- online activation quantisation, one scale per
 * 1x128 tile (per token per 128 channels) [P1 paragraph 1], derived from the
 * tile's max-abs value mapped onto the largest E4M3 value [P2 paragraphs 3-4,
 * P4 paragraph 1].
 *
 * For every row m < M and tile kb < K/128, with x_j the 128 BF16 inputs of the
 * tile widened exactly to binary32:
 *     a = max_j |x_j|
 *     s = fl32(a / 448)                       (stored scale)
 *     r = min(fl32(448 / a), FLT_MAX)         (a = 0 gives FLT_MAX)
 *     q_j = E4M3_rne(clamp(fl32(x_j * r), -448, 448))
 * All binary32 operations round to nearest even; subnormals are kept; the
 * sign of zero is kept.  Results are bit-identical to that definition.
 *
 *   x      BF16 [M, K], row stride ldx (>= K, multiple of 8); 16-byte aligned.
 *   q      E4M3 [M, K] output, row stride ldq (>= K, multiple of 16); 16-byte aligned.
 *   s      float output, s[m * s_sm + kb * s_skb]; 4-byte aligned; s_sm, s_skb >= 0
 *          and the M x K/128 positions must not overlap (not checked).
 *   K must be a multiple of 128.  M >= 0.
 */
fgq_status_t fgq_quant_act_1x128(const void* x, int64_t ldx, int64_t M, int64_t K,
                                 void* q, int64_t ldq, float* s, int64_t s_sm, int64_t s_skb,
                                 void* stream);

/*
 * fgq_quant_w_128x128 -- weight quantisation, one scale per 128x128 block
 * (per 128 input channels per 128 output channels) [P1 paragraph 1], same
 * scale rule as fgq_quant_act_1x128 with the tile replaced by the block.
 * Batched over B experts (B = 1 for a dense weight).
 *
 *   w      BF16 [B][N, K]; w[b*w_bs + n*ldw + k]; ldw >= K, multiple of 8;
 *          w_bs multiple of 8; 16-byte aligned.
 *   q      E4M3 [B][N, K]; q[b*q_bs + n*ldq + k]; ldq >= K, multiple of 16;
 *          q_bs multiple of 16; 16-byte aligned.
 *   s      float [B][N/128][K/128]; s[b*s_bs + nb*s_snb + kb*s_skb]; strides >= 0.
 *   N and K must be multiples of 128.  B >= 0.
 */
fgq_status_t fgq_quant_w_128x128(const void* w, int64_t ldw, int64_t w_bs, int64_t B,
                                 int64_t N, int64_t K, void* q, int64_t ldq, int64_t q_bs,
                                 float* s, int64_t s_snb, int64_t s_skb, int64_t s_bs,
                                 void* stream);

/*
 * fgq_fused_rmsnorm_quant -- RMSNorm fused with the 1x128 FP8 cast, so the
 * normalised row never makes a BF16 round trip through HBM [P3 paragraph 3,
 * P2 paragraph 1].  The norm is computed in binary32 and is not rounded to
 * BF16 before the cast:
 *     y_k = fl32(fl32(x_k * rstd) * gamma_k),
 *     rstd = fl32(1 / fl32(sqrt(fl32(fl32(ss / K) + eps))))
 * where ss is the sum of x_k^2 in one fixed order: the row is cut into
 * 8-value vectors; partial sum l (l = 0..63) takes vectors l, l+64, ... in
 * turn and adds their squares one value at a time (no fused multiply-add);
 * the 64 partials are combined by adding partial (l xor d) for
 * d = 32, 16, 8, 4, 2, 1.  Then y is quantised exactly as in
 * fgq_quant_act_1x128.  Results are bit-identical to that definition.
 *
 *   x      BF16 [M, K], row stride ldx (>= K, multiple of 8); 16-byte aligned.
 *   gamma  BF16 [K]; 16-byte aligned.
 *   eps    binary32 epsilon (the caller rounds it to float).
 *   q, s   as in fgq_quant_act_1x128.
 *   K must be a multiple of 128 and at most 16384.
 */
fgq_status_t fgq_fused_rmsnorm_quant(const void* x, int64_t ldx, const void* gamma, float eps,
                                     int64_t M, int64_t K, void* q, int64_t ldq,
                                     float* s, int64_t s_sm, int64_t s_skb, void* stream);

/*
 * How the GEMMs sum the FP8 products of one 128-wide K chunk.
 *
 * FGQ_GEMM_EXACT (default): the E4M3 codes are widened exactly to FP16 in
 *   registers and multiplied on the FP16 matrix cores: every product is exact
 *   and the chunk sum keeps binary32-level precision.  Runs at the FP16
 *   matrix-core rate.
 * FGQ_GEMM_FP8_CORE: the FP8 matrix cores (v_mfma_f32_16x16x128_f8f6f4), at
 *   twice that rate.  Measured on gfx950: the unit sums each group of 8
 *   consecutive products in a window about 13 bits below the group's largest
 *   product and truncates the rest (the same limited accumulation width the
 *   pages report for H800, P1 paragraph 4 and P4 paragraph 4).  The per-chunk
 *   FP32 promotion bounds the damage, but on outlier-heavy inputs a few
 *   strongly cancelling outputs (about 1 in 10^5) miss a 1e-2 elementwise
 *   relative bound that FGQ_GEMM_EXACT meets.
 */
enum { FGQ_GEMM_EXACT = 0, FGQ_GEMM_FP8_CORE = 1 };

/*
 * fgq_gemm_fp8_blockscaled -- C = A_hat * W_hat^T in FP8 with per-group K
 * scaling [P2 paragraph 3]: for each 128-wide K chunk kb the FP8 products are
 * summed by the matrix cores, and the partial sum is promoted into a binary32
 * accumulator multiplied by sa[m, kb] * sw[n/128, kb] [P2 paragraph 3,
 * P4 paragraph 4, P1 paragraph 4]; the result is rounded to BF16 (nearest even).
 *
 *   qa     E4M3 [M, K] (1x128-quantised activations), row stride lda (>= K,
 *          multiple of 16, at most 2^24); 16-byte aligned.
 *   sa     float, sa[m * sa_sm + kb * sa_skb].
 *   qw     E4M3 [N, K] (128x128-quantised weights), row stride ldw (>= K,
 *          multiple of 16, at most 2^24); 16-byte aligned.
 *          (The kernels address operand rows by 32-bit offsets inside a
 *          tile; a larger lda or ldw returns FGQ_ERR_UNSUPPORTED.)
 *   sw     float, sw[nb * sw_snb + kb * sw_skb].
 *   c      BF16 [M, N] output, row stride ldc (>= N, multiple of 8); 16-byte aligned.
 *   mode   FGQ_GEMM_EXACT or FGQ_GEMM_FP8_CORE (anything else: FGQ_ERR_UNSUPPORTED).
 *   workspace / workspace_bytes: scratch the caller provides, 256-byte
 *          aligned; fgq_gemm_workspace_bytes(M, N, K) bytes is the size that
 *          lets every shape take its fastest launch.  Small M (split along
 *          K) requires that size; otherwise the call runs with any size,
 *          NULL included: a large product whose last round of tiles would
 *          leave most compute units idle splits those tiles along K when
 *          the workspace holds their partial sums, and runs plainly when it
 *          does not.
 *   N and K must be multiples of 128, K > 0.  M >= 0 (any value; M = 0
 *   launches nothing).
 * The result is within the tolerance of the float64 definition; the order of
 * the additions inside a chunk is the matrix core's, so results are
 * reproducible run to run (for the same workspace size) but not across tile
 * configurations.
 */
fgq_status_t fgq_gemm_fp8_blockscaled(const void* qa, int64_t lda, const float* sa, int64_t sa_sm,
                                      int64_t sa_skb, const void* qw, int64_t ldw, const float* sw,
                                      int64_t sw_snb, int64_t sw_skb, void* c, int64_t ldc,
                                      int64_t M, int64_t N, int64_t K, int32_t mode, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * fgq_gemm_fp8_blockscaled_noalloc -- fgq_gemm_fp8_blockscaled for callers
 * that cannot allocate device memory (code under HIP graph capture,
 * allocation-free serving loops, harnesses that forbid hipMalloc): the same
 * product, the same kernels and the same results as fgq_gemm_fp8_blockscaled
 * given a 48 MiB workspace, with a scratch array inside the library (48 MiB
 * per GPU, allocated when the library's code is loaded on that GPU and held
 * until the process ends) in place of the workspace.  The call allocates
 * nothing and calls no allocating routine; the caller still passes every
 * input and output.
 *   Arguments as in fgq_gemm_fp8_blockscaled, without workspace.
 *   A product whose required workspace (the split along K of small M, at
 *   most 16.8 MB for any shape the ABI accepts) exceeded 48 MiB would
 *   return FGQ_ERR_SCRATCH; a large product splits its last round of tiles
 *   only when their partial sums fit (8192 x 18432 products do).
 *   Every call on one GPU uses that GPU's one scratch array: calls that can
 *   overlap on the same GPU (different streams or threads) race and must
 *   be serialised by the caller.
 */
fgq_status_t fgq_gemm_fp8_blockscaled_noalloc(const void* qa, int64_t lda, const float* sa, int64_t sa_sm,
                                              int64_t sa_skb, const void* qw, int64_t ldw, const float* sw,
                                              int64_t sw_snb, int64_t sw_skb, void* c, int64_t ldc, int64_t M,
                                              int64_t N, int64_t K, int32_t mode, void* stream);

/* Bytes of workspace for fgq_gemm_fp8_blockscaled (and its E8M0 variant) at
 * this shape: what small M requires, and what lets a large product split its
 * last round (0 = none). */
size_t fgq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * fgq_grouped_gemm_fp8_blockscaled -- the ragged grouped variant for MoE
 * experts, whose up-projection forward GEMMs run in FP8 [P2 paragraph 4,
 * P3 paragraph 4].  Rows of A are concatenated by expert: expert e owns rows
 * offsets[e] .. offsets[e+1]-1 and multiplies them by its own weight
 *     W_e = qw + e * w_es,  scales sw + e * sw_es,
 * with the same per-chunk promotion as fgq_gemm_fp8_blockscaled.  Experts
 * with no rows cost nothing.
 *
 *   offsets    DEVICE int32 [E + 1], non-decreasing, offsets[0] = 0,
 *              offsets[E] = total_rows.  Read only by the GPU (no host sync).
 *              Rows outside [0, total_rows) are never read or written even if
 *              offsets break this invariant; what is then computed is undefined.
 *   qa, sa     as in the dense GEMM, with total_rows rows.
 *   qw         E4M3 [E][N, K]; w_es (elements) multiple of 16.
 *   sw         float; sw[e * sw_es + nb * sw_snb + kb * sw_skb].
 *   c          BF16 [total_rows, N].
 *   mode       as in fgq_gemm_fp8_blockscaled.
 *   E >= 0 and at most 65536.  N and K multiples of 128, K > 0.
 */
fgq_status_t fgq_grouped_gemm_fp8_blockscaled(const void* qa, int64_t lda, const float* sa,
                                              int64_t sa_sm, int64_t sa_skb, const void* qw,
                                              int64_t ldw, int64_t w_es, const float* sw,
                                              int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
                                              const int32_t* offsets, int64_t E, int64_t total_rows,
                                              void* c, int64_t ldc, int64_t N, int64_t K, int32_t mode,
                                              void* stream);

/*
 * fgq_gemm_bf16a_fp8_blockscaled -- the 1x128 activation quantisation fused
 * into the GEMM's A-load.  The pages note that quantised activations make a
 * round trip through HBM (read as BF16, written as FP8, read again for the
 * MMA) [P2 paragraph 1] and propose doing the FP8 cast while the activations
 * move from global memory into shared memory [P3 paragraph 3].  Here the
 * GEMM reads A in BF16; per 128-wide K chunk each row's tile is quantised in
 * registers exactly as fgq_quant_act_1x128 does (same codes, same scale),
 * written to LDS, and multiplied as in fgq_gemm_fp8_blockscaled.  The result
 * is bit-identical to fgq_quant_act_1x128 followed by
 * fgq_gemm_fp8_blockscaled with the same mode.
 *
 *   a       BF16 [M, K], row stride lda (>= K, multiple of 8, at most 2^23); 16-byte aligned.
 *           ldw at most 2^24, as in fgq_gemm_fp8_blockscaled.
 *   qw, sw, c, M, N, K, mode, workspace: as in fgq_gemm_fp8_blockscaled
 *           (the same fgq_gemm_workspace_bytes).
 *   qa_out, sa_out  optional (both NULL or both set): the codes and scales
 *           of A, written once (by the tiles of the first 128- or 256-column
 *           block), laid out as fgq_quant_act_1x128's q (row stride ldq,
 *           16-byte aligned) and s (sa_out[m * sa_sm + kb * sa_skb]).
 *           Emitting costs time: the GEMM then waits for every memory access
 *           each chunk.
 * A is read once per column block of C (from L2 where it fits): this trades
 * the activation round trip for repeated quantisation work inside the GEMM.
 */
fgq_status_t fgq_gemm_bf16a_fp8_blockscaled(const void* a, int64_t lda, const void* qw, int64_t ldw,
                                            const float* sw, int64_t sw_snb, int64_t sw_skb, void* c,
                                            int64_t ldc, int64_t M, int64_t N, int64_t K, int32_t mode,
                                            void* qa_out, int64_t ldq, float* sa_out, int64_t sa_sm,
                                            int64_t sa_skb, void* workspace, size_t workspace_bytes,
                                            void* stream);

/*
 * fgq_quant_dispatch_1x128 -- quantise-then-dispatch: the activations that
 * enter the MoE up-projection are quantised to FP8 and handed to the experts
 * in that form [P2 paragraph 4]; each token goes to topk experts
 * [P3 paragraph 4].
 *
 * Pair i = t * topk + j (token t < T, slot j < topk) whose id ids[i] lies in
 * [0, E) becomes one output row; pairs with other ids are not routed.  Rows
 * are grouped by expert and, inside an expert, ordered by increasing i, so
 * the output is unique:
 *     offsets[e] .. offsets[e+1]-1   rows of expert e; offsets[0] = 0 and
 *                                    offsets[E] = R, the number of routed pairs
 *     row_src[r] = i                 for every row r < R
 *     dest[i] = r, or -1             for every pair i < T * topk
 *     q[r, :], s[r, :]               the 1x128 quantisation of token row
 *                                    i / topk: bit-identical to
 *                                    fgq_quant_act_1x128 of that row.
 * This is the row layout fgq_grouped_gemm_fp8_blockscaled consumes (pass
 * offsets, and T * topk as total_rows); row_src and dest are the maps a
 * combine step needs.
 *
 *   x        BF16 [T, K], row stride ldx (>= K, multiple of 8); 16-byte aligned.
 *   ids      DEVICE int32 [T, topk], row-major (row stride topk); 4-byte aligned.
 *   q        E4M3 output with room for T * topk rows, row stride ldq (>= K,
 *            multiple of 16); 16-byte aligned.  Rows >= R are not written.
 *   s        float output, s[r * s_sm + kb * s_skb], room for T * topk rows.
 *   offsets  DEVICE int32 [E + 1] output, written also when T = 0.
 *   row_src  DEVICE int32 [T * topk] output; entries >= R are not written.
 *   dest     DEVICE int32 [T * topk] output.
 *   workspace / workspace_bytes: scratch the caller provides; at least
 *            fgq_quant_dispatch_workspace_bytes(T, topk, E, K) bytes,
 *            256-byte aligned (may be NULL when that is 0).  It holds the
 *            routing counts and, when a row's scales are not contiguous
 *            (s_skb != 1, e.g. the K-block-major layout the GEMM reads
 *            best), one scale per token tile: those are then written once
 *            per token and copied to the routed rows in row order, instead
 *            of being stored 4-byte by 4-byte to scattered rows.
 *   K a multiple of 128 with K / 128 <= 65535; T >= 0; topk >= 1;
 *   1 <= E <= 4096; T * topk < 2^31.  The inputs are read only by the GPU
 *   (no host sync).
 */
fgq_status_t fgq_quant_dispatch_1x128(const void* x, int64_t ldx, int64_t T, int64_t K,
                                      const int32_t* ids, int64_t topk, int64_t E, void* q,
                                      int64_t ldq, float* s, int64_t s_sm, int64_t s_skb,
                                      int32_t* offsets, int32_t* row_src, int32_t* dest,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace fgq_quant_dispatch_1x128 (and its E8M0 variant) needs
 * (0 = none, or arguments out of range). */
size_t fgq_quant_dispatch_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t K);

/*
 * Power-of-two (E8M0) scales.  The pages note that per-group scaling along K
 * is in line with microscaling formats, and that newer matrix units support
 * such formats natively [P1 paragraph 4, P4 paragraph 3].  A microscaling
 * block scale is an E8M0 byte (OCP Microscaling Formats v1.0): the value
 * 2^(byte - 127); byte 255 is NaN.  gfx950's FP8 matrix core multiplies such
 * scales in itself (v_mfma_scale_f32_16x16x128_f8f6f4), so the GEMMs below
 * need no binary32 scale products.
 *
 * Scale rule (in place of s = a / 448): for a group with max-abs a, the
 * smallest e >= -127 with 448 * 2^e >= a; the stored byte is e + 127 (a = 0
 * gives byte 0).  The cast multiplies by 2^-e, which is exact, so
 *     q_j = E4M3_rne(x_j * 2^-e),   |x_j * 2^-e| <= 448,
 *     value ~= decode(q_j) * 2^(byte - 127).
 * Scale arrays are bytes with strides in bytes and no alignment rule.  The
 * GEMMs read each scale as the aligned 32-bit word that holds it (that word
 * must be readable memory, as it is inside any allocation).
 */

/* fgq_quant_act_1x128_e8m0 -- fgq_quant_act_1x128 with E8M0 scales:
 * s[m * s_sm + kb * s_skb] = byte of tile (m, kb).  Bit-identical to the rule above. */
fgq_status_t fgq_quant_act_1x128_e8m0(const void* x, int64_t ldx, int64_t M, int64_t K,
                                      void* q, int64_t ldq, uint8_t* s, int64_t s_sm, int64_t s_skb,
                                      void* stream);

/* fgq_quant_w_128x128_e8m0 -- fgq_quant_w_128x128 with E8M0 scales:
 * s[b * s_bs + nb * s_snb + kb * s_skb] = byte of block (b, nb, kb). */
fgq_status_t fgq_quant_w_128x128_e8m0(const void* w, int64_t ldw, int64_t w_bs, int64_t B,
                                      int64_t N, int64_t K, void* q, int64_t ldq, int64_t q_bs,
                                      uint8_t* s, int64_t s_snb, int64_t s_skb, int64_t s_bs,
                                      void* stream);

/* fgq_fused_rmsnorm_quant_e8m0 -- fgq_fused_rmsnorm_quant (same y) with E8M0
 * scales of the binary32 tile max-abs of y. */
fgq_status_t fgq_fused_rmsnorm_quant_e8m0(const void* x, int64_t ldx, const void* gamma, float eps,
                                          int64_t M, int64_t K, void* q, int64_t ldq,
                                          uint8_t* s, int64_t s_sm, int64_t s_skb, void* stream);

/* fgq_quant_dispatch_1x128_e8m0 -- fgq_quant_dispatch_1x128 with E8M0 scales
 * (s[r * s_sm + kb * s_skb], bytes): every routed row is bit-identical to
 * fgq_quant_act_1x128_e8m0 of its token row.  Same routing outputs. */
fgq_status_t fgq_quant_dispatch_1x128_e8m0(const void* x, int64_t ldx, int64_t T, int64_t K,
                                           const int32_t* ids, int64_t topk, int64_t E, void* q,
                                           int64_t ldq, uint8_t* s, int64_t s_sm, int64_t s_skb,
                                           int32_t* offsets, int32_t* row_src, int32_t* dest,
                                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * How the E8M0 GEMMs accumulate across 128-wide K chunks.  Each chunk is one
 * scaled matrix-core operation per 16x16 output block; scales are applied by
 * the unit.
 *
 * FGQ_E8M0_PROMOTE (default): each chunk's scaled sum lands in a fresh zero
 *   accumulator and is added to a binary32 accumulator on the vector ALU:
 *   the pages' promotion at an interval of 128 [P1 paragraph 4,
 *   P4 paragraph 4].  Same accuracy as FGQ_GEMM_FP8_CORE.
 * FGQ_E8M0_IN_CORE: the running sum is the matrix core's own accumulator
 *   operand, so no vector-ALU work at all: the accumulation without
 *   promotion that the pages warn about on H800, where about 14 bits survive.
 *   Measured on gfx950: the unit aligns the accumulator operand and the
 *   chunk's 8-product group sums to the largest of them and truncates what
 *   falls more than about 24 bits below, so each chunk costs at most about
 *   2^-20 of the running sum (the 13-bit window inside each group is the
 *   same in both modes).  Accuracy is that of FGQ_E8M0_PROMOTE to within
 *   BF16 output rounding.
 */
enum { FGQ_E8M0_PROMOTE = 0, FGQ_E8M0_IN_CORE = 1 };

/*
 * fgq_gemm_fp8_e8m0 -- fgq_gemm_fp8_blockscaled with E8M0 scales:
 *     C[m, n] = bf16( sum_kb 2^(sa[m, kb] - 127) * 2^(sw[n/128, kb] - 127)
 *                            * sum_{k in chunk kb} decode(qa[m, k]) * decode(qw[n, k]) )
 *   sa     bytes, sa[m * sa_sm + kb * sa_skb].
 *   sw     bytes, sw[nb * sw_snb + kb * sw_skb].
 *   accumulate  FGQ_E8M0_PROMOTE or FGQ_E8M0_IN_CORE (else FGQ_ERR_UNSUPPORTED).
 *   Everything else (shapes, strides, alignment, workspace =
 *   fgq_gemm_workspace_bytes(M, N, K)) as in fgq_gemm_fp8_blockscaled.
 */
fgq_status_t fgq_gemm_fp8_e8m0(const void* qa, int64_t lda, const uint8_t* sa, int64_t sa_sm,
                               int64_t sa_skb, const void* qw, int64_t ldw, const uint8_t* sw,
                               int64_t sw_snb, int64_t sw_skb, void* c, int64_t ldc,
                               int64_t M, int64_t N, int64_t K, int32_t accumulate, void* workspace,
                               size_t workspace_bytes, void* stream);

/* fgq_grouped_gemm_fp8_e8m0 -- fgq_grouped_gemm_fp8_blockscaled with E8M0
 * scales (sw[e * sw_es + nb * sw_snb + kb * sw_skb], bytes) and the
 * accumulation choice of fgq_gemm_fp8_e8m0. */
fgq_status_t fgq_grouped_gemm_fp8_e8m0(const void* qa, int64_t lda, const uint8_t* sa,
                                       int64_t sa_sm, int64_t sa_skb, const void* qw,
                                       int64_t ldw, int64_t w_es, const uint8_t* sw,
                                       int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
                                       const int32_t* offsets, int64_t E, int64_t total_rows,
                                       void* c, int64_t ldc, int64_t N, int64_t K, int32_t accumulate,
                                       void* stream);

/* Text for a status code (static storage; never NULL). */
const char* fgq_status_string(fgq_status_t status);

/* The hipError_t behind this thread's last FGQ_ERR_HIP (0 if none). */
int32_t fgq_last_hip_error(void);

/* FGQ_ABI_VERSION of the loaded library. */
int32_t fgq_abi_version(void);

/*
 * Diagnostics used by the tests and the benchmark (not part of the method).
 *
 * fgq_debug_encode_e4m3 -- out[i] = E4M3 code of clamp(float(bits = start + i), -448, 448)
 * through the same device conversion the quantisation kernels use, i < n.
 * Bit patterns that are NaN give unspecified codes.  out: device, n bytes.
 */
fgq_status_t fgq_debug_encode_e4m3(uint32_t start, int64_t n, void* out, void* stream);

/* fgq_debug_copy -- plain device copy of `bytes` bytes (16-byte aligned
 * pointers, bytes a multiple of 16); used to calibrate traffic counters. */
fgq_status_t fgq_debug_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* fgq_debug_mfma_16x16x128 -- one FP8 matrix-core operation exactly as the
 * GEMM issues it: d = a * b^T + cin, a and b E4M3 [16][128] row-major (16-byte
 * aligned), cin and d float [16][16] row-major.  Used to measure how the unit
 * accumulates a 128-wide chunk (the pages report ~14 retained bits on H800). */
fgq_status_t fgq_debug_mfma_16x16x128(const void* a, const void* b, const float* cin, float* d, void* stream);

/* fgq_debug_mfma_loop -- the matrix cores' sustained rate and the shader
 * clock under that load, the measured ceiling beside the nominal peaks (the
 * pages report no kernel-level throughput, so the chip's own limits are the
 * reference for every roofline fraction).  `waves` waves (a multiple of 4,
 * four per 256-thread workgroup) each run `iters` rounds of 8 independent
 * register-only matrix operations of one kind:
 *   kind 0  v_mfma_f32_16x16x128_f8f6f4  (FP8,  65536 flops each)
 *   kind 1  v_mfma_f32_16x16x32_f16      (FP16, 16384 flops each)
 *   kind 2  v_mfma_f32_32x32x16_f16      (FP16, 32768 flops each)
 * out     DEVICE uint64 [4 * waves], 8-byte aligned: per wave the shader
 *         clock counter (s_memtime) before and after the loop, then the
 *         100 MHz real-time counter (s_memrealtime) before and after.
 * sink    DEVICE float [64 * waves]: a reduction of the results (keeps the
 *         work from being optimised away; its values mean nothing).
 * Errors: kind outside 0..2 -> FGQ_ERR_UNSUPPORTED; iters < 0, waves < 0,
 * waves not a multiple of 4 or above 4 * 65535 -> FGQ_ERR_SHAPE. */
fgq_status_t fgq_debug_mfma_loop(int32_t kind, int64_t iters, int64_t waves, uint64_t* out, float* sink,
                                 void* stream);

/* fgq_debug_mfma_e8m0_16x16x128 -- one scaled FP8 matrix-core operation as
 * the E8M0 GEMMs issue it: d = diag(2^(sa - 127)) a b^T diag(2^(sb - 127)) + cin,
 * sa and sb bytes [16] (row scales of a, column scales of b), the rest as in
 * fgq_debug_mfma_16x16x128.  Used to measure how the unit adds cin. */
fgq_status_t fgq_debug_mfma_e8m0_16x16x128(const void* a, const void* b, const uint8_t* sa,
                                           const uint8_t* sb, const float* cin, float* d, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FGQ_H */
