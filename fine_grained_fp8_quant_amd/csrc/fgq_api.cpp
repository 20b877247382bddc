// C ABI of libfgq.so (declared in include/fgq.h): host-side argument
// validation, then a launch on the caller's stream.  Validation returns an
// error code before any HIP call; nothing here allocates, synchronises or
// reads device memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fgq.h"
#include "fgq_launch.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr int64_t kMaxTiles = (int64_t)1 << 31;  // 32-bit tile indices in the kernels
// The GEMM kernels address a tile's operand rows by 32-bit byte offsets from
// the tile's first row: row (at most 255) * ld + column (at most 112), which
// stays below 2^32 for every ld <= 2^24 bytes.
constexpr int64_t kMaxOperandLd = (int64_t)1 << 24;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

fgq_status_t from_hip(hipError_t e) {
  if (e == hipSuccess) return FGQ_OK;
  g_last_hip_error = (int32_t)e;
  return FGQ_ERR_HIP;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Before a call launches its kernels: clear an error that an unrelated
// earlier HIP call left in this thread's error state, so that the
// hipGetLastError() after the launch reports this call's launch only.
void clear_stale_error() { (void)hipGetLastError(); }

// Common checks for a [rows, K] BF16 input / E4M3 + scale output pair;
// s_align is the scale element's alignment (4 for binary32, 1 for E8M0).
fgq_status_t check_act_io(const void* x, int64_t ldx, int64_t M, int64_t K, const void* q, int64_t ldq,
                          const void* s, int64_t s_sm, int64_t s_skb, uintptr_t s_align = 4) {
  if (M < 0 || K < 0) return FGQ_ERR_SHAPE;
  if (K % 128 != 0) return FGQ_ERR_UNSUPPORTED;
  if (M == 0 || K == 0) return FGQ_OK;
  if (!x || !q || !s) return FGQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, s_align)) return FGQ_ERR_ALIGN;
  if (ldx < K || ldx % 8 != 0 || ldq < K || ldq % 16 != 0) return FGQ_ERR_STRIDE;
  if (s_sm < 0 || s_skb < 0) return FGQ_ERR_STRIDE;
  if (M * (K / 128) >= kMaxTiles) return FGQ_ERR_UNSUPPORTED;
  return FGQ_OK;
}

fgq_status_t check_gemm_common(const void* qa, int64_t lda, const void* sa, int64_t sa_sm, int64_t sa_skb,
                               const void* qw, int64_t ldw, const void* sw, int64_t sw_snb,
                               int64_t sw_skb, const void* c, int64_t ldc, int64_t N, int64_t K,
                               uintptr_t s_align = 4) {
  if (!qa || !sa || !qw || !sw || !c) return FGQ_ERR_NULL;
  if (!aligned(qa, 16) || !aligned(qw, 16) || !aligned(c, 16) || !aligned(sa, s_align) || !aligned(sw, s_align))
    return FGQ_ERR_ALIGN;
  if (lda < K || lda % 16 != 0 || ldw < K || ldw % 16 != 0 || ldc < N || ldc % 8 != 0)
    return FGQ_ERR_STRIDE;
  if (sa_sm < 0 || sa_skb < 0 || sw_snb < 0 || sw_skb < 0) return FGQ_ERR_STRIDE;
  if (N / 128 > 65535 || lda > kMaxOperandLd || ldw > kMaxOperandLd) return FGQ_ERR_UNSUPPORTED;
  return FGQ_OK;
}

// Shared validation of the two scale formats' weight quantisers.
fgq_status_t check_quant_w(const void* w, int64_t ldw, int64_t w_bs, int64_t B, int64_t N, int64_t K,
                           const void* q, int64_t ldq, int64_t q_bs, const void* s, int64_t s_snb,
                           int64_t s_skb, int64_t s_bs, uintptr_t s_align) {
  if (B < 0 || N < 0 || K < 0) return FGQ_ERR_SHAPE;
  if (N % 128 != 0 || K % 128 != 0) return FGQ_ERR_UNSUPPORTED;
  if (B == 0 || N == 0 || K == 0) return FGQ_OK;
  if (!w || !q || !s) return FGQ_ERR_NULL;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(s, s_align)) return FGQ_ERR_ALIGN;
  if (ldw < K || ldw % 8 != 0 || ldq < K || ldq % 16 != 0) return FGQ_ERR_STRIDE;
  if (w_bs % 8 != 0 || q_bs % 16 != 0) return FGQ_ERR_STRIDE;
  if (B > 1 && (w_bs < N * ldw || q_bs < N * ldq)) return FGQ_ERR_STRIDE;
  if (s_snb < 0 || s_skb < 0 || s_bs < 0) return FGQ_ERR_STRIDE;
  if (B * (N / 128) * (K / 128) >= kMaxTiles) return FGQ_ERR_UNSUPPORTED;
  return FGQ_OK;
}

fgq_status_t check_fused(const void* x, int64_t ldx, const void* gamma, int64_t M, int64_t K, const void* q,
                         int64_t ldq, const void* s, int64_t s_sm, int64_t s_skb, uintptr_t s_align) {
  fgq_status_t st = check_act_io(x, ldx, M, K, q, ldq, s, s_sm, s_skb, s_align);
  if (st != FGQ_OK || M == 0 || K == 0) return st;
  if (K > 16384) return FGQ_ERR_UNSUPPORTED;
  if (!gamma) return FGQ_ERR_NULL;
  if (!aligned(gamma, 16)) return FGQ_ERR_ALIGN;
  return FGQ_OK;
}

fgq_status_t check_gemm(const void* qa, int64_t lda, const void* sa, int64_t sa_sm, int64_t sa_skb,
                        const void* qw, int64_t ldw, const void* sw, int64_t sw_snb, int64_t sw_skb,
                        const void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, bool mode_ok,
                        const void* workspace, size_t workspace_bytes, uintptr_t s_align) {
  if (M < 0 || N < 0 || K < 0) return FGQ_ERR_SHAPE;
  if (!mode_ok) return FGQ_ERR_UNSUPPORTED;
  if (N % 128 != 0 || K % 128 != 0 || K == 0) return FGQ_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return FGQ_OK;
  fgq_status_t st = check_gemm_common(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, N, K,
                                      s_align);
  if (st != FGQ_OK) return st;
  if (M >= kMaxTiles) return FGQ_ERR_UNSUPPORTED;
  const size_t need = fgq::gemm_workspace_required(M, N, K);
  if (need > 0) {
    if (!workspace) return FGQ_ERR_NULL;
    if (workspace_bytes < need) return FGQ_ERR_SHAPE;
    if (!aligned(workspace, 256)) return FGQ_ERR_ALIGN;
  }
  return FGQ_OK;
}

fgq_status_t check_grouped(const void* qa, int64_t lda, const void* sa, int64_t sa_sm, int64_t sa_skb,
                           const void* qw, int64_t ldw, int64_t w_es, const void* sw, int64_t sw_snb,
                           int64_t sw_skb, int64_t sw_es, const int32_t* offsets, int64_t E, int64_t total_rows,
                           const void* c, int64_t ldc, int64_t N, int64_t K, bool mode_ok, uintptr_t s_align) {
  if (E < 0 || total_rows < 0 || N < 0 || K < 0) return FGQ_ERR_SHAPE;
  if (!mode_ok) return FGQ_ERR_UNSUPPORTED;
  if (N % 128 != 0 || K % 128 != 0 || K == 0) return FGQ_ERR_UNSUPPORTED;
  if (E > 65536 || total_rows >= ((int64_t)1 << 31) - 65536) return FGQ_ERR_UNSUPPORTED;
  if (E == 0 || total_rows == 0 || N == 0) return FGQ_OK;
  if (!offsets) return FGQ_ERR_NULL;
  fgq_status_t st = check_gemm_common(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, N, K,
                                      s_align);
  if (st != FGQ_OK) return st;
  if (!aligned(offsets, 4)) return FGQ_ERR_ALIGN;
  if (w_es % 16 != 0 || w_es < 0 || sw_es < 0) return FGQ_ERR_STRIDE;
  if (E > 1 && w_es < N * ldw) return FGQ_ERR_STRIDE;
  return FGQ_OK;
}

}  // namespace

extern "C" {

fgq_status_t fgq_quant_act_1x128(const void* x, int64_t ldx, int64_t M, int64_t K, void* q, int64_t ldq,
                                 float* s, int64_t s_sm, int64_t s_skb, void* stream) {
  const fgq_status_t st = check_act_io(x, ldx, M, K, q, ldq, s, s_sm, s_skb);
  if (st != FGQ_OK || M == 0 || K == 0) return st;
  clear_stale_error();
  return from_hip(fgq::launch_quant_act_1x128(static_cast<const uint16_t*>(x), ldx, M, K,
                                              static_cast<uint8_t*>(q), ldq, s, s_sm, s_skb,
                                              as_stream(stream)));
}

fgq_status_t fgq_quant_w_128x128(const void* w, int64_t ldw, int64_t w_bs, int64_t B, int64_t N, int64_t K,
                                 void* q, int64_t ldq, int64_t q_bs, float* s, int64_t s_snb,
                                 int64_t s_skb, int64_t s_bs, void* stream) {
  const fgq_status_t st = check_quant_w(w, ldw, w_bs, B, N, K, q, ldq, q_bs, s, s_snb, s_skb, s_bs, 4);
  if (st != FGQ_OK || B == 0 || N == 0 || K == 0) return st;
  clear_stale_error();
  return from_hip(fgq::launch_quant_w_128x128(static_cast<const uint16_t*>(w), ldw, w_bs, B, N, K,
                                              static_cast<uint8_t*>(q), ldq, q_bs, s, s_snb, s_skb, s_bs,
                                              as_stream(stream)));
}

fgq_status_t fgq_fused_rmsnorm_quant(const void* x, int64_t ldx, const void* gamma, float eps, int64_t M,
                                     int64_t K, void* q, int64_t ldq, float* s, int64_t s_sm,
                                     int64_t s_skb, void* stream) {
  const fgq_status_t st = check_fused(x, ldx, gamma, M, K, q, ldq, s, s_sm, s_skb, 4);
  if (st != FGQ_OK || M == 0 || K == 0) return st;
  clear_stale_error();
  return from_hip(fgq::launch_fused_rmsnorm_quant(static_cast<const uint16_t*>(x), ldx,
                                                  static_cast<const uint16_t*>(gamma), eps, M, K,
                                                  static_cast<uint8_t*>(q), ldq, s, s_sm, s_skb,
                                                  as_stream(stream)));
}

size_t fgq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return fgq::gemm_workspace_bytes(M, N, K);
}

fgq_status_t fgq_gemm_fp8_blockscaled(const void* qa, int64_t lda, const float* sa, int64_t sa_sm,
                                      int64_t sa_skb, const void* qw, int64_t ldw, const float* sw,
                                      int64_t sw_snb, int64_t sw_skb, void* c, int64_t ldc, int64_t M,
                                      int64_t N, int64_t K, int32_t mode, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  const fgq_status_t st = check_gemm(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K,
                                     mode == FGQ_GEMM_EXACT || mode == FGQ_GEMM_FP8_CORE, workspace,
                                     workspace_bytes, 4);
  if (st != FGQ_OK || M == 0 || N == 0) return st;
  clear_stale_error();
  return from_hip(fgq::launch_gemm_fp8_blockscaled(
      static_cast<const uint8_t*>(qa), lda, sa, sa_sm, sa_skb, static_cast<const uint8_t*>(qw), ldw, sw,
      sw_snb, sw_skb, static_cast<uint16_t*>(c), ldc, M, N, K, mode, workspace, workspace_bytes,
      as_stream(stream)));
}

fgq_status_t fgq_gemm_fp8_blockscaled_noalloc(const void* qa, int64_t lda, const float* sa, int64_t sa_sm,
                                              int64_t sa_skb, const void* qw, int64_t ldw, const float* sw,
                                              int64_t sw_snb, int64_t sw_skb, void* c, int64_t ldc, int64_t M,
                                              int64_t N, int64_t K, int32_t mode, void* stream) {
  // the same checks as fgq_gemm_fp8_blockscaled, with the library's scratch
  // in place of a workspace (its address is checked below, not here)
  const size_t room = fgq::noalloc_scratch_bytes();
  if (M > 0 && N > 0 && K > 0 && N % 128 == 0 && K % 128 == 0 && fgq::gemm_workspace_required(M, N, K) > room)
    return FGQ_ERR_SCRATCH;
  const void* const placeholder = reinterpret_cast<const void*>((uintptr_t)256);  // aligned, non-null
  const fgq_status_t st = check_gemm(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K,
                                     mode == FGQ_GEMM_EXACT || mode == FGQ_GEMM_FP8_CORE, placeholder, room, 4);
  if (st != FGQ_OK || M == 0 || N == 0) return st;
  void* ws = nullptr;
  const fgq_status_t sst = from_hip(fgq::noalloc_scratch(&ws));
  if (sst != FGQ_OK) return sst;
  clear_stale_error();
  return from_hip(fgq::launch_gemm_fp8_blockscaled(
      static_cast<const uint8_t*>(qa), lda, sa, sa_sm, sa_skb, static_cast<const uint8_t*>(qw), ldw, sw,
      sw_snb, sw_skb, static_cast<uint16_t*>(c), ldc, M, N, K, mode, ws, room, as_stream(stream)));
}

fgq_status_t fgq_grouped_gemm_fp8_blockscaled(const void* qa, int64_t lda, const float* sa, int64_t sa_sm,
                                              int64_t sa_skb, const void* qw, int64_t ldw, int64_t w_es,
                                              const float* sw, int64_t sw_snb, int64_t sw_skb,
                                              int64_t sw_es, const int32_t* offsets, int64_t E,
                                              int64_t total_rows, void* c, int64_t ldc, int64_t N,
                                              int64_t K, int32_t mode, void* stream) {
  const fgq_status_t st = check_grouped(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es,
                                        offsets, E, total_rows, c, ldc, N, K,
                                        mode == FGQ_GEMM_EXACT || mode == FGQ_GEMM_FP8_CORE, 4);
  if (st != FGQ_OK || E == 0 || total_rows == 0 || N == 0) return st;
  clear_stale_error();
  return from_hip(fgq::launch_grouped_gemm_fp8_blockscaled(
      static_cast<const uint8_t*>(qa), lda, sa, sa_sm, sa_skb, static_cast<const uint8_t*>(qw), ldw, w_es,
      sw, sw_snb, sw_skb, sw_es, offsets, E, total_rows, static_cast<uint16_t*>(c), ldc, N, K, mode,
      as_stream(stream)));
}

fgq_status_t fgq_gemm_bf16a_fp8_blockscaled(const void* a, int64_t lda, const void* qw, int64_t ldw, const float* sw,
                                            int64_t sw_snb, int64_t sw_skb, void* c, int64_t ldc, int64_t M, int64_t N,
                                            int64_t K, int32_t mode, void* qa_out, int64_t ldq, float* sa_out,
                                            int64_t sa_sm, int64_t sa_skb, void* workspace, size_t workspace_bytes,
                                            void* stream) {
  if (M < 0 || N < 0 || K < 0) return FGQ_ERR_SHAPE;
  if (mode != FGQ_GEMM_EXACT && mode != FGQ_GEMM_FP8_CORE) return FGQ_ERR_UNSUPPORTED;
  if (N % 128 != 0 || K % 128 != 0 || K == 0) return FGQ_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return FGQ_OK;
  if (!a || !qw || !sw || !c) return FGQ_ERR_NULL;
  if ((qa_out == nullptr) != (sa_out == nullptr)) return FGQ_ERR_NULL;
  if (!aligned(a, 16) || !aligned(qw, 16) || !aligned(c, 16) || !aligned(sw, 4)) return FGQ_ERR_ALIGN;
  if (lda < K || lda % 8 != 0 || ldw < K || ldw % 16 != 0 || ldc < N || ldc % 8 != 0) return FGQ_ERR_STRIDE;
  if (sw_snb < 0 || sw_skb < 0) return FGQ_ERR_STRIDE;
  // BF16 A: its rows are 2 * lda bytes apart
  if (2 * lda > kMaxOperandLd || ldw > kMaxOperandLd || N / 128 > 65535 || M >= kMaxTiles)
    return FGQ_ERR_UNSUPPORTED;
  if (qa_out) {
    if (!aligned(qa_out, 16) || !aligned(sa_out, 4)) return FGQ_ERR_ALIGN;
    if (ldq < K || ldq % 16 != 0 || sa_sm < 0 || sa_skb < 0) return FGQ_ERR_STRIDE;
  }
  const size_t need = fgq::gemm_workspace_required(M, N, K);
  if (need > 0) {
    if (!workspace) return FGQ_ERR_NULL;
    if (workspace_bytes < need) return FGQ_ERR_SHAPE;
    if (!aligned(workspace, 256)) return FGQ_ERR_ALIGN;
  }
  clear_stale_error();
  return from_hip(fgq::launch_gemm_bf16a_fp8_blockscaled(
      static_cast<const uint16_t*>(a), lda, static_cast<const uint8_t*>(qw), ldw, sw, sw_snb, sw_skb,
      static_cast<uint16_t*>(c), ldc, M, N, K, mode, static_cast<uint8_t*>(qa_out), ldq, sa_out, sa_sm, sa_skb,
      workspace, as_stream(stream)));
}

fgq_status_t fgq_quant_act_1x128_e8m0(const void* x, int64_t ldx, int64_t M, int64_t K, void* q, int64_t ldq,
                                      uint8_t* s, int64_t s_sm, int64_t s_skb, void* stream) {
  const fgq_status_t st = check_act_io(x, ldx, M, K, q, ldq, s, s_sm, s_skb, 1);
  if (st != FGQ_OK || M == 0 || K == 0) return st;
  clear_stale_error();
  return from_hip(fgq::launch_quant_act_1x128_e8m0(static_cast<const uint16_t*>(x), ldx, M, K,
                                                   static_cast<uint8_t*>(q), ldq, s, s_sm, s_skb,
                                                   as_stream(stream)));
}

fgq_status_t fgq_quant_w_128x128_e8m0(const void* w, int64_t ldw, int64_t w_bs, int64_t B, int64_t N, int64_t K,
                                      void* q, int64_t ldq, int64_t q_bs, uint8_t* s, int64_t s_snb,
                                      int64_t s_skb, int64_t s_bs, void* stream) {
  const fgq_status_t st = check_quant_w(w, ldw, w_bs, B, N, K, q, ldq, q_bs, s, s_snb, s_skb, s_bs, 1);
  if (st != FGQ_OK || B == 0 || N == 0 || K == 0) return st;
  clear_stale_error();
  return from_hip(fgq::launch_quant_w_128x128_e8m0(static_cast<const uint16_t*>(w), ldw, w_bs, B, N, K,
                                                   static_cast<uint8_t*>(q), ldq, q_bs, s, s_snb, s_skb, s_bs,
                                                   as_stream(stream)));
}

fgq_status_t fgq_fused_rmsnorm_quant_e8m0(const void* x, int64_t ldx, const void* gamma, float eps, int64_t M,
                                          int64_t K, void* q, int64_t ldq, uint8_t* s, int64_t s_sm,
                                          int64_t s_skb, void* stream) {
  const fgq_status_t st = check_fused(x, ldx, gamma, M, K, q, ldq, s, s_sm, s_skb, 1);
  if (st != FGQ_OK || M == 0 || K == 0) return st;
  clear_stale_error();
  return from_hip(fgq::launch_fused_rmsnorm_quant_e8m0(static_cast<const uint16_t*>(x), ldx,
                                                       static_cast<const uint16_t*>(gamma), eps, M, K,
                                                       static_cast<uint8_t*>(q), ldq, s, s_sm, s_skb,
                                                       as_stream(stream)));
}

fgq_status_t fgq_gemm_fp8_e8m0(const void* qa, int64_t lda, const uint8_t* sa, int64_t sa_sm, int64_t sa_skb,
                               const void* qw, int64_t ldw, const uint8_t* sw, int64_t sw_snb, int64_t sw_skb,
                               void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, int32_t accumulate,
                               void* workspace, size_t workspace_bytes, void* stream) {
  const fgq_status_t st = check_gemm(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K,
                                     accumulate == FGQ_E8M0_PROMOTE || accumulate == FGQ_E8M0_IN_CORE, workspace,
                                     workspace_bytes, 1);
  if (st != FGQ_OK || M == 0 || N == 0) return st;
  clear_stale_error();
  return from_hip(fgq::launch_gemm_fp8_e8m0(static_cast<const uint8_t*>(qa), lda, sa, sa_sm, sa_skb,
                                            static_cast<const uint8_t*>(qw), ldw, sw, sw_snb, sw_skb,
                                            static_cast<uint16_t*>(c), ldc, M, N, K,
                                            accumulate == FGQ_E8M0_IN_CORE ? 1 : 0, workspace, workspace_bytes,
                                            as_stream(stream)));
}

fgq_status_t fgq_grouped_gemm_fp8_e8m0(const void* qa, int64_t lda, const uint8_t* sa, int64_t sa_sm,
                                       int64_t sa_skb, const void* qw, int64_t ldw, int64_t w_es,
                                       const uint8_t* sw, int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
                                       const int32_t* offsets, int64_t E, int64_t total_rows, void* c,
                                       int64_t ldc, int64_t N, int64_t K, int32_t accumulate, void* stream) {
  const fgq_status_t st = check_grouped(qa, lda, sa, sa_sm, sa_skb, qw, ldw, w_es, sw, sw_snb, sw_skb, sw_es,
                                        offsets, E, total_rows, c, ldc, N, K,
                                        accumulate == FGQ_E8M0_PROMOTE || accumulate == FGQ_E8M0_IN_CORE, 1);
  if (st != FGQ_OK || E == 0 || total_rows == 0 || N == 0) return st;
  clear_stale_error();
  return from_hip(fgq::launch_grouped_gemm_fp8_e8m0(
      static_cast<const uint8_t*>(qa), lda, sa, sa_sm, sa_skb, static_cast<const uint8_t*>(qw), ldw, w_es, sw,
      sw_snb, sw_skb, sw_es, offsets, E, total_rows, static_cast<uint16_t*>(c), ldc, N, K,
      accumulate == FGQ_E8M0_IN_CORE ? 1 : 0, as_stream(stream)));
}

const char* fgq_status_string(fgq_status_t status) {
  switch (status) {
    case FGQ_OK: return "ok";
    case FGQ_ERR_NULL: return "a required pointer is NULL";
    case FGQ_ERR_SHAPE: return "negative or inconsistent size";
    case FGQ_ERR_ALIGN: return "pointer not aligned as documented";
    case FGQ_ERR_STRIDE: return "leading dimension or stride too small or misaligned";
    case FGQ_ERR_UNSUPPORTED: return "size not supported (K and N must be multiples of 128)";
    case FGQ_ERR_HIP: return "HIP launch failed (see fgq_last_hip_error)";
    case FGQ_ERR_SCRATCH: return "the product needs more scratch than the no-allocation entry point holds (48 MiB)";
    default: return "unknown status";
  }
}

int32_t fgq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

namespace {

fgq_status_t check_dispatch(const void* x, int64_t ldx, int64_t T, int64_t K, const int32_t* ids, int64_t topk,
                            int64_t E, const void* q, int64_t ldq, const void* s, int64_t s_sm, int64_t s_skb,
                            const int32_t* offsets, const int32_t* row_src, const int32_t* dest,
                            const void* workspace, size_t workspace_bytes, uintptr_t s_align) {
  if (T < 0 || K < 0 || topk < 1 || E < 1) return FGQ_ERR_SHAPE;
  if (K % 128 != 0 || E > 4096 || K / 128 > 65535) return FGQ_ERR_UNSUPPORTED;
  if (T >= kMaxTiles || topk >= kMaxTiles || T * topk >= kMaxTiles) return FGQ_ERR_UNSUPPORTED;
  if (!offsets) return FGQ_ERR_NULL;
  if (!aligned(offsets, 4)) return FGQ_ERR_ALIGN;
  if (T > 0) {
    if (!ids || !row_src || !dest) return FGQ_ERR_NULL;
    if (!aligned(ids, 4) || !aligned(row_src, 4) || !aligned(dest, 4)) return FGQ_ERR_ALIGN;
    const fgq_status_t st = check_act_io(x, ldx, T, K, q, ldq, s, s_sm, s_skb, s_align);
    if (st != FGQ_OK) return st;
    const size_t need = fgq::dispatch_workspace_bytes(T, topk, E, K);
    if (need > 0) {
      if (!workspace) return FGQ_ERR_NULL;
      if (workspace_bytes < need) return FGQ_ERR_SHAPE;
      if (!aligned(workspace, 256)) return FGQ_ERR_ALIGN;
    }
  }
  return FGQ_OK;
}

}  // namespace

extern "C" {

fgq_status_t fgq_quant_dispatch_1x128(const void* x, int64_t ldx, int64_t T, int64_t K, const int32_t* ids,
                                      int64_t topk, int64_t E, void* q, int64_t ldq, float* s, int64_t s_sm,
                                      int64_t s_skb, int32_t* offsets, int32_t* row_src, int32_t* dest,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const fgq_status_t st = check_dispatch(x, ldx, T, K, ids, topk, E, q, ldq, s, s_sm, s_skb, offsets, row_src, dest,
                                         workspace, workspace_bytes, 4);
  if (st != FGQ_OK) return st;
  clear_stale_error();
  return from_hip(fgq::launch_quant_dispatch_1x128(static_cast<const uint16_t*>(x), ldx, T, K, ids, topk, E,
                                                   static_cast<uint8_t*>(q), ldq, s, s_sm, s_skb, offsets,
                                                   row_src, dest, workspace, as_stream(stream)));
}

fgq_status_t fgq_quant_dispatch_1x128_e8m0(const void* x, int64_t ldx, int64_t T, int64_t K, const int32_t* ids,
                                           int64_t topk, int64_t E, void* q, int64_t ldq, uint8_t* s, int64_t s_sm,
                                           int64_t s_skb, int32_t* offsets, int32_t* row_src, int32_t* dest,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  const fgq_status_t st = check_dispatch(x, ldx, T, K, ids, topk, E, q, ldq, s, s_sm, s_skb, offsets, row_src, dest,
                                         workspace, workspace_bytes, 1);
  if (st != FGQ_OK) return st;
  clear_stale_error();
  return from_hip(fgq::launch_quant_dispatch_1x128_e8m0(static_cast<const uint16_t*>(x), ldx, T, K, ids, topk, E,
                                                        static_cast<uint8_t*>(q), ldq, s, s_sm, s_skb, offsets,
                                                        row_src, dest, workspace, as_stream(stream)));
}

size_t fgq_quant_dispatch_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t K) {
  if (T < 0 || topk < 1 || E < 1 || K < 0 || K % 128 != 0) return 0;
  if (T >= kMaxTiles || topk >= kMaxTiles || T * topk >= kMaxTiles || T * (K / 128) >= kMaxTiles) return 0;
  return fgq::dispatch_workspace_bytes(T, topk, E, K);
}

int32_t fgq_abi_version(void) { return FGQ_ABI_VERSION; }

fgq_status_t fgq_debug_encode_e4m3(uint32_t start, int64_t n, void* out, void* stream) {
  if (n < 0 || n > ((int64_t)1 << 32)) return FGQ_ERR_SHAPE;
  if (n == 0) return FGQ_OK;
  if (!out) return FGQ_ERR_NULL;
  clear_stale_error();
  return from_hip(fgq::launch_debug_encode_e4m3(start, n, static_cast<uint8_t*>(out), as_stream(stream)));
}

fgq_status_t fgq_debug_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0) return FGQ_ERR_SHAPE;
  if (bytes == 0) return FGQ_OK;
  if (!src || !dst) return FGQ_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16) || bytes % 16 != 0) return FGQ_ERR_ALIGN;
  clear_stale_error();
  return from_hip(fgq::launch_debug_copy(src, dst, bytes, as_stream(stream)));
}

fgq_status_t fgq_debug_mfma_16x16x128(const void* a, const void* b, const float* cin, float* d, void* stream) {
  if (!a || !b || !cin || !d) return FGQ_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(cin, 4) || !aligned(d, 4)) return FGQ_ERR_ALIGN;
  clear_stale_error();
  return from_hip(fgq::launch_debug_mfma(static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(b), cin, d,
                                         as_stream(stream)));
}

fgq_status_t fgq_debug_mfma_e8m0_16x16x128(const void* a, const void* b, const uint8_t* sa, const uint8_t* sb,
                                           const float* cin, float* d, void* stream) {
  if (!a || !b || !sa || !sb || !cin || !d) return FGQ_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(cin, 4) || !aligned(d, 4)) return FGQ_ERR_ALIGN;
  clear_stale_error();
  return from_hip(fgq::launch_debug_mfma_e8m0(static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(b), sa, sb,
                                              cin, d, as_stream(stream)));
}

fgq_status_t fgq_debug_mfma_loop(int32_t kind, int64_t iters, int64_t waves, uint64_t* out, float* sink,
                                 void* stream) {
  if (kind < 0 || kind > 2) return FGQ_ERR_UNSUPPORTED;
  if (iters < 0 || waves < 0 || waves % 4 != 0 || waves / 4 > 65535) return FGQ_ERR_SHAPE;
  if (waves == 0) return FGQ_OK;
  if (!out || !sink) return FGQ_ERR_NULL;
  if (!aligned(out, 8) || !aligned(sink, 4)) return FGQ_ERR_ALIGN;
  clear_stale_error();
  return from_hip(fgq::launch_debug_mfma_loop(kind, iters, waves, out, sink, as_stream(stream)));
}

}  // extern "C"
