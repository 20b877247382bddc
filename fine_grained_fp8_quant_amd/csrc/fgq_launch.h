// Internal launch entry points behind the C ABI in include/fgq.h.  Arguments
// have already been validated by fgq_api.cpp; each function only enqueues
// work on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgq {

hipError_t launch_quant_act_1x128(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, uint8_t* q,
                                  int64_t ldq, float* s, int64_t s_sm, int64_t s_skb, hipStream_t st);

hipError_t launch_quant_w_128x128(const uint16_t* w, int64_t ldw, int64_t w_bs, int64_t B, int64_t N,
                                  int64_t K, uint8_t* q, int64_t ldq, int64_t q_bs, float* s,
                                  int64_t s_snb, int64_t s_skb, int64_t s_bs, hipStream_t st);

hipError_t launch_fused_rmsnorm_quant(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps,
                                      int64_t M, int64_t K, uint8_t* q, int64_t ldq, float* s,
                                      int64_t s_sm, int64_t s_skb, hipStream_t st);

hipError_t launch_gemm_fp8_blockscaled(const uint8_t* qa, int64_t lda, const float* sa, int64_t sa_sm,
                                       int64_t sa_skb, const uint8_t* qw, int64_t ldw, const float* sw,
                                       int64_t sw_snb, int64_t sw_skb, uint16_t* c, int64_t ldc,
                                       int64_t M, int64_t N, int64_t K, int mode, void* workspace,
                                       size_t workspace_bytes, hipStream_t st);

// The no-allocation variant's device scratch: its size, and this device's
// address of it (resolved once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);

// recommended size (lets large products split their last round) and the
// size the call requires (split-K of small M)
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
size_t gemm_workspace_required(int64_t M, int64_t N, int64_t K);

hipError_t launch_grouped_gemm_fp8_blockscaled(const uint8_t* qa, int64_t lda, const float* sa,
                                               int64_t sa_sm, int64_t sa_skb, const uint8_t* qw,
                                               int64_t ldw, int64_t w_es, const float* sw,
                                               int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
                                               const int32_t* offsets, int64_t E, int64_t total_rows,
                                               uint16_t* c, int64_t ldc, int64_t N, int64_t K, int mode,
                                               hipStream_t st);

hipError_t launch_quant_dispatch_1x128(const uint16_t* x, int64_t ldx, int64_t T, int64_t K,
                                       const int32_t* ids, int64_t topk, int64_t E, uint8_t* q, int64_t ldq,
                                       float* s, int64_t s_sm, int64_t s_skb, int32_t* offsets,
                                       int32_t* row_src, int32_t* dest, void* workspace, hipStream_t st);

size_t dispatch_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t K);

// Power-of-two (E8M0 byte) scale variants of the quantisers and GEMMs.
hipError_t launch_quant_act_1x128_e8m0(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, uint8_t* q,
                                       int64_t ldq, uint8_t* s, int64_t s_sm, int64_t s_skb, hipStream_t st);

hipError_t launch_quant_w_128x128_e8m0(const uint16_t* w, int64_t ldw, int64_t w_bs, int64_t B, int64_t N,
                                       int64_t K, uint8_t* q, int64_t ldq, int64_t q_bs, uint8_t* s,
                                       int64_t s_snb, int64_t s_skb, int64_t s_bs, hipStream_t st);

hipError_t launch_fused_rmsnorm_quant_e8m0(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps,
                                           int64_t M, int64_t K, uint8_t* q, int64_t ldq, uint8_t* s,
                                           int64_t s_sm, int64_t s_skb, hipStream_t st);

hipError_t launch_quant_dispatch_1x128_e8m0(const uint16_t* x, int64_t ldx, int64_t T, int64_t K,
                                            const int32_t* ids, int64_t topk, int64_t E, uint8_t* q, int64_t ldq,
                                            uint8_t* s, int64_t s_sm, int64_t s_skb, int32_t* offsets,
                                            int32_t* row_src, int32_t* dest, void* workspace, hipStream_t st);

hipError_t launch_gemm_fp8_e8m0(const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t sa_sm, int64_t sa_skb,
                                const uint8_t* qw, int64_t ldw, const uint8_t* sw, int64_t sw_snb, int64_t sw_skb,
                                uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, int in_core,
                                void* workspace, size_t workspace_bytes, hipStream_t st);

hipError_t launch_grouped_gemm_fp8_e8m0(const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t sa_sm,
                                        int64_t sa_skb, const uint8_t* qw, int64_t ldw, int64_t w_es,
                                        const uint8_t* sw, int64_t sw_snb, int64_t sw_skb, int64_t sw_es,
                                        const int32_t* offsets, int64_t E, int64_t total_rows, uint16_t* c,
                                        int64_t ldc, int64_t N, int64_t K, int in_core, hipStream_t st);

// BF16 activations quantised inside the GEMM's A-load; optional emission of
// the codes and scales (qa_out == nullptr: none).
hipError_t launch_gemm_bf16a_fp8_blockscaled(const uint16_t* a, int64_t lda, const uint8_t* qw, int64_t ldw,
                                             const float* sw, int64_t sw_snb, int64_t sw_skb, uint16_t* c,
                                             int64_t ldc, int64_t M, int64_t N, int64_t K, int mode,
                                             uint8_t* qa_out, int64_t ldq, float* sa_out, int64_t sa_sm,
                                             int64_t sa_skb, void* workspace, hipStream_t st);

hipError_t launch_debug_encode_e4m3(uint32_t start, int64_t n, uint8_t* out, hipStream_t st);
hipError_t launch_debug_copy(const void* src, void* dst, int64_t bytes, hipStream_t st);
hipError_t launch_debug_mfma(const uint8_t* a, const uint8_t* b, const float* cin, float* d, hipStream_t st);
hipError_t launch_debug_mfma_loop(int kind, int64_t iters, int64_t waves, uint64_t* out, float* sink,
                                  hipStream_t st);
hipError_t launch_debug_mfma_e8m0(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                                 const float* cin, float* d, hipStream_t st);

}  // namespace fgq
