// Internal launchers (host side); the C ABI validates arguments first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

hipError_t launch_act_quant(const void *x, int64_t M, int64_t K, void *q, float *s,
                            hipStream_t stream);
hipError_t launch_weight_quant(const void *w, int64_t N, int64_t K, void *q, float *s,
                               hipStream_t stream);
hipError_t launch_act_quant_static(const void *x, int64_t M, int64_t K, const float *s, void *q,
                                   hipStream_t stream);
hipError_t launch_block_gemm_static(const void *xq, const float *xs, const void *wq,
                                    const float *ws, int64_t M, int64_t N, int64_t K, void *y,
                                    hipStream_t stream);
hipError_t launch_rowwise_quant(const void *x, int64_t R, int64_t K, void *q, float *s,
                                hipStream_t stream);
hipError_t launch_rowwise_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                               int64_t M, int64_t N, int64_t K, void *y, hipStream_t stream);
hipError_t launch_batched_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                               const int32_t *counts, int32_t E, int64_t capacity, int64_t N,
                               int64_t K, void *y, hipStream_t stream);
hipError_t launch_linear_decode(const void *x, const void *wq, const float *ws, int64_t M,
                                int64_t N, int64_t K, void *y, hipStream_t stream);
hipError_t launch_act_quant_e8m0(const void *x, int64_t M, int64_t K, void *q, uint8_t *s,
                                 hipStream_t stream);
// Column slabs per workgroup of the fused decode layer (up to 4 for
// M <= 16, up to 2 above).
int linear_decode_slabs(int64_t M, int64_t N);
hipError_t launch_swiglu_act_quant(const void *gu, int64_t M, int64_t I, void *q, float *s,
                                   hipStream_t stream);
hipError_t launch_swiglu_act_quant_e8m0(const void *gu, int64_t M, int64_t I, void *q,
                                        uint8_t *s, hipStream_t stream);
hipError_t launch_weight_quant_e8m0(const void *w, int64_t N, int64_t K, void *q, uint8_t *s,
                                    hipStream_t stream);
hipError_t launch_block_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                             int64_t M, int64_t N, int64_t K, void *y, hipStream_t stream);
// Split-K over workgroups through a caller workspace (falls back to
// launch_block_gemm when the plan needs none or the workspace is short).
size_t block_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_block_gemm_ws(const void *xq, const float *xs, const void *wq, const float *ws,
                                int64_t M, int64_t N, int64_t K, void *y, void *work,
                                size_t work_bytes, hipStream_t stream);
// Workspace of the K splits over workgroups alone (no stream-K tail).
size_t block_gemm_split_workspace_bytes(int64_t M, int64_t N, int64_t K);
// The same splits through the library's own device scratch (no caller
// workspace, no allocation); the plan's workspace must fit kScratchBytes.
constexpr size_t kScratchBytes = (size_t(16) << 20) + (size_t(64) << 10);
constexpr int kScratchMaxDevices = 64;
hipError_t launch_block_gemm_noalloc(const void *xq, const float *xs, const void *wq,
                                     const float *ws, int64_t M, int64_t N, int64_t K, void *y,
                                     hipStream_t stream);
size_t block_gemm_e8m0_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_block_gemm_e8m0_ws(const void *xq, const uint8_t *xs, const void *wq,
                                     const uint8_t *ws, int64_t M, int64_t N, int64_t K, void *y,
                                     void *work, size_t work_bytes, hipStream_t stream);
hipError_t launch_grouped_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                               const int32_t *offsets, int32_t E, int64_t total_M, int64_t N,
                               int64_t K, void *y, hipStream_t stream);
hipError_t launch_block_gemm_e8m0(const void *xq, const uint8_t *xs, const void *wq,
                                  const uint8_t *ws, int64_t M, int64_t N, int64_t K, void *y,
                                  hipStream_t stream);
hipError_t launch_grouped_gemm_e8m0(const void *xq, const uint8_t *xs, const void *wq,
                                    const uint8_t *ws, const int32_t *offsets, int32_t E,
                                    int64_t total_M, int64_t N, int64_t K, void *y,
                                    hipStream_t stream);

}  // namespace fp8blk
