// C ABI of fp8blk: argument validation (before any HIP runtime call), the
// gfx950 device check, and dispatch to the kernels.  Declared in fp8blk.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "../../include/fp8blk.h"
#include "fp8blk_launch.h"

namespace {

constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxK = int64_t(1) << 24;
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int kMaxDevices = 64;

// 0 = unknown, 1 = gfx950, 2 = other / unusable
std::atomic<int> g_arch_state[kMaxDevices];

bool misaligned(const void *p, uintptr_t align = 16) {
  return (reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0;
}

fp8blk_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return FP8BLK_ERR_DEVICE;
  }
  int st = g_arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return FP8BLK_ERR_DEVICE;
    }
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? FP8BLK_OK : FP8BLK_ERR_DEVICE;
}

fp8blk_status launched(hipError_t e) { return e == hipSuccess ? FP8BLK_OK : FP8BLK_ERR_LAUNCH; }

// Shape rules shared by the entry points: rows in [0, 2^31), K a positive
// multiple of 128 up to 2^24, element counts up to 2^40.
bool bad_rows(int64_t r) { return r < 0 || r > kMaxRows; }
bool bad_k(int64_t K) { return K <= 0 || K > kMaxK || (K % FP8BLK_BLOCK) != 0; }
bool too_big(int64_t rows, int64_t K) { return rows > 0 && K > 0 && rows > kMaxElems / K; }

// Validation of each operation, shared by its variants.  The scale arrays'
// alignment (bytes) depends on the variant: fp32 scale arrays 16, one
// static fp32 scale 4, E8M0 byte arrays 1 (none).
fp8blk_status check_quant(const void *in, int64_t rows, int64_t K, const void *q,
                          const void *scale, uintptr_t scale_align) {
  if (rows > 0 && (!in || !q || !scale)) return FP8BLK_ERR_NULL;
  if (bad_rows(rows) || bad_k(K) || too_big(rows, K)) return FP8BLK_ERR_SHAPE;
  if (rows > 0 && (misaligned(in) || misaligned(q) || misaligned(scale, scale_align)))
    return FP8BLK_ERR_ALIGN;
  return check_device();
}

// `work`: a workspace that the call will use (checked for 16-byte alignment
// with the other pointers), or NULL.
fp8blk_status check_gemm(const void *x_q, const void *x_scale, const void *w_q,
                         const void *w_scale, int64_t M, int64_t N, int64_t K, const void *y,
                         uintptr_t xs_align, uintptr_t ws_align, const void *work_buf = nullptr) {
  const bool work = M > 0 && N > 0;
  if (work && (!x_q || !x_scale || !w_q || !w_scale || !y)) return FP8BLK_ERR_NULL;
  if (bad_rows(M) || bad_rows(N) || bad_k(K) || too_big(M, K) || too_big(N, K) ||
      too_big(M, N))
    return FP8BLK_ERR_SHAPE;
  if (work && ((M + 127) / 128) * ((N + 127) / 128) > kMaxRows) return FP8BLK_ERR_SHAPE;
  if (work && (misaligned(x_q) || misaligned(w_q) || misaligned(y) ||
               misaligned(x_scale, xs_align) || misaligned(w_scale, ws_align) ||
               (work_buf && misaligned(work_buf))))
    return FP8BLK_ERR_ALIGN;
  return check_device();
}

fp8blk_status check_grouped(const void *x_q, const void *x_scale, const void *w_q,
                            const void *w_scale, const int32_t *offsets, int32_t E,
                            int64_t total_M, int64_t N, int64_t K, const void *y,
                            uintptr_t scale_align) {
  const bool work = E > 0 && total_M > 0 && N > 0;
  if (work && (!x_q || !x_scale || !w_q || !w_scale || !offsets || !y)) return FP8BLK_ERR_NULL;
  if (E < 0 || bad_rows(total_M) || bad_rows(N) || bad_k(K) || too_big(total_M, K) ||
      too_big(total_M, N) || (E > 0 && too_big(int64_t(E) * N, K)) || too_big(int64_t(E), N))
    return FP8BLK_ERR_SHAPE;
  if (work && ((total_M + 127) / 128 + E) * ((N + 127) / 128) > kMaxRows) return FP8BLK_ERR_SHAPE;
  if (work && (misaligned(x_q) || misaligned(w_q) || misaligned(y) ||
               misaligned(x_scale, scale_align) || misaligned(w_scale, scale_align)))
    return FP8BLK_ERR_ALIGN;
  return check_device();
}

fp8blk_status check_swiglu(const void *gate_up_bf16, int64_t M, int64_t I, const void *x_q,
                           const void *x_scale, uintptr_t scale_align) {
  if (M > 0 && (!gate_up_bf16 || !x_q || !x_scale)) return FP8BLK_ERR_NULL;
  if (bad_rows(M) || bad_k(I) || too_big(M, 2 * I) || M * (I / FP8BLK_BLOCK) > kMaxRows)
    return FP8BLK_ERR_SHAPE;
  if (M > 0 && (misaligned(gate_up_bf16) || misaligned(x_q) || misaligned(x_scale, scale_align)))
    return FP8BLK_ERR_ALIGN;
  return check_device();
}

}  // namespace

extern "C" {

const char *fp8blk_status_string(int s) {
  switch (s) {
    case FP8BLK_OK: return "FP8BLK_OK";
    case FP8BLK_ERR_NULL: return "FP8BLK_ERR_NULL: a required pointer is NULL";
    case FP8BLK_ERR_SHAPE: return "FP8BLK_ERR_SHAPE: bad size (negative, K not a positive multiple of 128, or over the limits)";
    case FP8BLK_ERR_ALIGN: return "FP8BLK_ERR_ALIGN: a base pointer is not 16-byte aligned";
    case FP8BLK_ERR_DEVICE: return "FP8BLK_ERR_DEVICE: no usable device, or the current device is not gfx950";
    case FP8BLK_ERR_LAUNCH: return "FP8BLK_ERR_LAUNCH: kernel launch failed";
    case FP8BLK_ERR_SCRATCH: return "FP8BLK_ERR_SCRATCH: the call needs more device scratch than the library holds (FP8BLK_SCRATCH_BYTES)";
    default: return "FP8BLK_ERR_UNKNOWN";
  }
}

int fp8blk_abi_version(void) { return FP8BLK_ABI_VERSION; }

fp8blk_status fp8_weight_block_quant(const void *w_bf16, int64_t N, int64_t K, void *w_q,
                                     float *w_scale, void *stream) {
  if (fp8blk_status c = check_quant(w_bf16, N, K, w_q, w_scale, 16)) return c;
  if (N == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_weight_quant(w_bf16, N, K, w_q, w_scale,
                                              static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_act_quant_group(const void *x_bf16, int64_t M, int64_t K, void *x_q,
                                  float *x_scale, void *stream) {
  if (fp8blk_status c = check_quant(x_bf16, M, K, x_q, x_scale, 16)) return c;
  if (M == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_act_quant(x_bf16, M, K, x_q, x_scale,
                                           static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_block_gemm(const void *x_q, const float *x_scale, const void *w_q,
                             const float *w_scale, int64_t M, int64_t N, int64_t K, void *y_bf16,
                             void *stream) {
  if (fp8blk_status c = check_gemm(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16, 16, 16)) return c;
  if (M == 0 || N == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_block_gemm(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16,
                                            static_cast<hipStream_t>(stream)));
}

size_t fp8_block_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (bad_rows(M) || bad_rows(N) || bad_k(K) || too_big(M, K) || too_big(N, K) || too_big(M, N))
    return 0;
  return fp8blk::block_gemm_workspace_bytes(M, N, K);
}

fp8blk_status fp8_block_gemm_ws(const void *x_q, const float *x_scale, const void *w_q,
                                const float *w_scale, int64_t M, int64_t N, int64_t K,
                                void *y_bf16, void *workspace, size_t workspace_bytes,
                                void *stream) {
  // whether the workspace will be used (known before validation so that its
  // alignment is checked with the other pointers; check_gemm still rejects
  // bad sizes before anything runs)
  const size_t need = fp8blk::block_gemm_workspace_bytes(M, N, K);
  const bool use = need > 0 && workspace != nullptr && workspace_bytes >= need;
  if (fp8blk_status c = check_gemm(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16, 16, 16,
                                   use ? workspace : nullptr))
    return c;
  if (M == 0 || N == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_block_gemm_ws(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16,
                                               use ? workspace : nullptr, use ? workspace_bytes : 0,
                                               static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_grouped_block_gemm(const void *x_q, const float *x_scale, const void *w_q,
                                     const float *w_scale, const int32_t *expert_offsets,
                                     int32_t E, int64_t total_M, int64_t N, int64_t K,
                                     void *y_bf16, void *stream) {
  if (fp8blk_status c = check_grouped(x_q, x_scale, w_q, w_scale, expert_offsets, E, total_M, N,
                                      K, y_bf16, 16))
    return c;
  if (E == 0 || total_M == 0 || N == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_grouped_gemm(x_q, x_scale, w_q, w_scale, expert_offsets, E,
                                              total_M, N, K, y_bf16,
                                              static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_act_quant_static(const void *x_bf16, int64_t M, int64_t K,
                                   const float *x_scale, void *x_q, void *stream) {
  if (fp8blk_status c = check_quant(x_bf16, M, K, x_q, x_scale, 4)) return c;
  if (M == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_act_quant_static(x_bf16, M, K, x_scale, x_q,
                                                  static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_block_gemm_static(const void *x_q, const float *x_scale, const void *w_q,
                                    const float *w_scale, int64_t M, int64_t N, int64_t K,
                                    void *y_bf16, void *stream) {
  if (fp8blk_status c = check_gemm(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16, 4, 16)) return c;
  if (M == 0 || N == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_block_gemm_static(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16,
                                                   static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_block_gemm_noalloc(const void *x_q, const float *x_scale, const void *w_q,
                                     const float *w_scale, int64_t M, int64_t N, int64_t K,
                                     void *y_bf16, void *stream) {
  static_assert(fp8blk::kScratchBytes == FP8BLK_SCRATCH_BYTES, "scratch size out of step");
  if (fp8blk_status c = check_gemm(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16, 16, 16)) return c;
  if (M == 0 || N == 0) return FP8BLK_OK;
  if (fp8blk::block_gemm_split_workspace_bytes(M, N, K) > fp8blk::kScratchBytes)
    return FP8BLK_ERR_SCRATCH;
  return launched(fp8blk::launch_block_gemm_noalloc(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16,
                                                    static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_linear(const void *x_bf16, int64_t M, int64_t N, int64_t K, const void *w_q,
                         const float *w_scale, void *x_q_ws, float *x_scale_ws, void *y_bf16,
                         void *stream) {
  // The fused decode kernel re-quantizes x in every workgroup (each reads
  // all of x in bf16 from L2), once per K block for all the workgroup's
  // 16-column slabs.  With workspaces at hand it runs only where it beats
  // the two kernels: at M <= 16 for small weights (the second launch costs
  // more) and for K <= 8192 when the launcher packs two or more slabs per
  // workgroup; at M = 17-32 for weights of at most 2^24 elements; never
  // past M = 32.  Measured, weights streamed from HBM (fused against two
  // kernels), M = 16: 4096x4096 10.1 us / 19.4; 14336x4096 (4 slabs) 15.9 /
  // 19.5; 24576x1536 (2 slabs) 16.5 / 19.5; 4096x14336 (1 slab) 26.7 /
  // 21.1; 7168x16384 (2 slabs) 38.4 / 33.5; 18432x7168 (1 slab) 66.4 /
  // 47.2.  M = 17-32: 4096x4096 13.4-14.4 / 19.3-19.6; 1024x4096 11.4-12.6
  // / 19.1; 1536x7168 17.6-20.2 / 18.9-19.0; 14336x4096 27-31 / 23-24.
  // M = 33-64: 4096x4096 24.2-25.1 / 19.6-19.7; 1024x4096 21.1-23.1 /
  // 19.2-19.3; 1536x7168 35.7-39.1 / 19.3-25.7.
  constexpr int64_t kFusedMaxM = 64;
  constexpr int64_t kFusedMaxWeight = int64_t(1) << 25;     // N * K elements, M <= 16
  constexpr int64_t kFusedMaxWeight32 = int64_t(1) << 24;   // N * K elements, M <= 32
  constexpr int64_t kFusedSlabsMaxK = 8192;
  const bool work = M > 0 && N > 0;
  const bool have_ws = x_q_ws != nullptr && x_scale_ws != nullptr;
  // (N * K only for sizes within the limits, which keep it below 2^55;
  // others are refused below)
  const bool sized = !bad_rows(N) && !bad_k(K);
  const bool fused =
      M <= kFusedMaxM &&
      (!have_ws || !sized ||
       (M <= 16 && (N * K <= kFusedMaxWeight ||
                    (K <= kFusedSlabsMaxK && fp8blk::linear_decode_slabs(M, N) >= 2))) ||
       (M <= 32 && N * K <= kFusedMaxWeight32));
  if (work && (!x_bf16 || !w_q || !w_scale || !y_bf16 || (!fused && (!x_q_ws || !x_scale_ws))))
    return FP8BLK_ERR_NULL;
  if (bad_rows(M) || bad_rows(N) || bad_k(K) || too_big(M, K) || too_big(N, K) || too_big(M, N))
    return FP8BLK_ERR_SHAPE;
  if (work && ((M + 127) / 128) * ((N + 127) / 128) > kMaxRows) return FP8BLK_ERR_SHAPE;
  if (work && (misaligned(x_bf16) || misaligned(w_q) || misaligned(w_scale) ||
               misaligned(y_bf16) || (!fused && (misaligned(x_q_ws) || misaligned(x_scale_ws)))))
    return FP8BLK_ERR_ALIGN;
  if (fp8blk_status d = check_device()) return d;
  if (!work) return FP8BLK_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (fused) return launched(fp8blk::launch_linear_decode(x_bf16, w_q, w_scale, M, N, K, y_bf16, st));
  if (fp8blk_status e = launched(fp8blk::launch_act_quant(x_bf16, M, K, x_q_ws, x_scale_ws, st)))
    return e;
  return launched(fp8blk::launch_block_gemm(x_q_ws, x_scale_ws, w_q, w_scale, M, N, K, y_bf16, st));
}

fp8blk_status fp8_batched_block_gemm(const void *x_q, const float *x_scale, const void *w_q,
                                     const float *w_scale, const int32_t *expert_counts,
                                     int32_t E, int64_t capacity, int64_t N, int64_t K,
                                     void *y_bf16, void *stream) {
  const bool work = E > 0 && capacity > 0 && N > 0;
  if (work && (!x_q || !x_scale || !w_q || !w_scale || !expert_counts || !y_bf16))
    return FP8BLK_ERR_NULL;
  if (E < 0 || capacity < 0 || bad_rows(N) || bad_k(K) || (E > 0 && capacity > kMaxRows / E))
    return FP8BLK_ERR_SHAPE;
  const int64_t total = int64_t(E) * capacity;
  if (too_big(total, K) || too_big(total, N) || (E > 0 && too_big(int64_t(E) * N, K)) ||
      too_big(int64_t(E), N))
    return FP8BLK_ERR_SHAPE;
  if (work && int64_t(E) * ((capacity + 127) / 128) * ((N + 127) / 128) > kMaxRows)
    return FP8BLK_ERR_SHAPE;
  if (work && (misaligned(x_q) || misaligned(x_scale) || misaligned(w_q) || misaligned(w_scale) ||
               misaligned(y_bf16) || misaligned(expert_counts, 4)))
    return FP8BLK_ERR_ALIGN;
  if (fp8blk_status d = check_device()) return d;
  if (!work) return FP8BLK_OK;
  return launched(fp8blk::launch_batched_gemm(x_q, x_scale, w_q, w_scale, expert_counts, E,
                                              capacity, N, K, y_bf16,
                                              static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_rowwise_quant(const void *in_bf16, int64_t R, int64_t K, void *q,
                                float *scale, void *stream) {
  if (fp8blk_status c = check_quant(in_bf16, R, K, q, scale, 16)) return c;
  if (R == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_rowwise_quant(in_bf16, R, K, q, scale,
                                               static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_rowwise_gemm(const void *x_q, const float *x_scale, const void *w_q,
                               const float *w_scale, int64_t M, int64_t N, int64_t K,
                               void *y_bf16, void *stream) {
  if (fp8blk_status c = check_gemm(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16, 16, 16)) return c;
  if (M == 0 || N == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_rowwise_gemm(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16,
                                              static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_swiglu_act_quant(const void *gate_up_bf16, int64_t M, int64_t I, void *x_q,
                                   float *x_scale, void *stream) {
  if (fp8blk_status c = check_swiglu(gate_up_bf16, M, I, x_q, x_scale, 16)) return c;
  if (M == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_swiglu_act_quant(gate_up_bf16, M, I, x_q, x_scale,
                                                  static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_swiglu_act_quant_ue8m0(const void *gate_up_bf16, int64_t M, int64_t I,
                                         void *x_q, uint8_t *x_scale, void *stream) {
  if (fp8blk_status c = check_swiglu(gate_up_bf16, M, I, x_q, x_scale, 1)) return c;
  if (M == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_swiglu_act_quant_e8m0(gate_up_bf16, M, I, x_q, x_scale,
                                                       static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_weight_block_quant_ue8m0(const void *w_bf16, int64_t N, int64_t K, void *w_q,
                                           uint8_t *w_scale, void *stream) {
  if (fp8blk_status c = check_quant(w_bf16, N, K, w_q, w_scale, 1)) return c;
  if (N == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_weight_quant_e8m0(w_bf16, N, K, w_q, w_scale,
                                                   static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_act_quant_group_ue8m0(const void *x_bf16, int64_t M, int64_t K, void *x_q,
                                        uint8_t *x_scale, void *stream) {
  if (fp8blk_status c = check_quant(x_bf16, M, K, x_q, x_scale, 1)) return c;
  if (M == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_act_quant_e8m0(x_bf16, M, K, x_q, x_scale,
                                                static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_block_gemm_ue8m0(const void *x_q, const uint8_t *x_scale, const void *w_q,
                                   const uint8_t *w_scale, int64_t M, int64_t N, int64_t K,
                                   void *y_bf16, void *stream) {
  if (fp8blk_status c = check_gemm(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16, 1, 1)) return c;
  if (M == 0 || N == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_block_gemm_e8m0(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16,
                                                 static_cast<hipStream_t>(stream)));
}

size_t fp8_block_gemm_ue8m0_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (bad_rows(M) || bad_rows(N) || bad_k(K) || too_big(M, K) || too_big(N, K) || too_big(M, N))
    return 0;
  return fp8blk::block_gemm_e8m0_workspace_bytes(M, N, K);
}

fp8blk_status fp8_block_gemm_ue8m0_ws(const void *x_q, const uint8_t *x_scale, const void *w_q,
                                      const uint8_t *w_scale, int64_t M, int64_t N, int64_t K,
                                      void *y_bf16, void *workspace, size_t workspace_bytes,
                                      void *stream) {
  // as fp8_block_gemm_ws
  const size_t need = fp8blk::block_gemm_e8m0_workspace_bytes(M, N, K);
  const bool use = need > 0 && workspace != nullptr && workspace_bytes >= need;
  if (fp8blk_status c = check_gemm(x_q, x_scale, w_q, w_scale, M, N, K, y_bf16, 1, 1,
                                   use ? workspace : nullptr))
    return c;
  if (M == 0 || N == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_block_gemm_e8m0_ws(
      x_q, x_scale, w_q, w_scale, M, N, K, y_bf16, use ? workspace : nullptr,
      use ? workspace_bytes : 0, static_cast<hipStream_t>(stream)));
}

fp8blk_status fp8_grouped_block_gemm_ue8m0(const void *x_q, const uint8_t *x_scale,
                                           const void *w_q, const uint8_t *w_scale,
                                           const int32_t *expert_offsets, int32_t E,
                                           int64_t total_M, int64_t N, int64_t K, void *y_bf16,
                                           void *stream) {
  if (fp8blk_status c = check_grouped(x_q, x_scale, w_q, w_scale, expert_offsets, E, total_M, N,
                                      K, y_bf16, 1))
    return c;
  if (E == 0 || total_M == 0 || N == 0) return FP8BLK_OK;
  return launched(fp8blk::launch_grouped_gemm_e8m0(x_q, x_scale, w_q, w_scale, expert_offsets, E,
                                                   total_M, N, K, y_bf16,
                                                   static_cast<hipStream_t>(stream)));
}

}  // extern "C"
