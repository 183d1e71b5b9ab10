// Practical ceilings of the fp8 matrix cores on gfx950, for measurement only
// (libfp8ceil.so; not part of the fp8blk C ABI and never called by it).
//
// Both kernels keep every operand in registers -- no global, LDS or scalar
// memory traffic inside the timed loop -- so their rate is what the matrix
// cores sustain at the clock the chip actually holds under this load:
//
//   kPromote = false: back-to-back v_mfma_f32_16x16x128_f8f6f4 accumulating
//     into 32 independent 16x16 fp32 fragments per wave (128 accumulators
//     per lane, the wave tile of the 256x256 GEMM tile).
//   kPromote = true: the inner loop of the fp32-scale block GEMM without its
//     memory side -- each MFMA starts from zero (one 128-wide K block) and
//     its result is added into the accumulators with one fp32 FMA per output
//     and a per-row scale, one fragment behind the MFMA stream.
//
// 512 threads per workgroup (two waves per SIMD, as the GEMM runs).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <bool kPromote>
__global__ __launch_bounds__(512) void mfma_ceiling_kernel(float *__restrict__ out, int iters) {
  const int t = threadIdx.x;
  v8i a, b[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = 0x38383838 ^ (t * 7 + i);
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int i = 0; i < 8; ++i) b[n][i] = 0x30303030 ^ (t * 3 + i + 8 * n);
  v4f acc[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  float s = 1.0f + (float)t * 1e-7f;

  for (int it = 0; it < iters; ++it) {
    a[0] ^= it;
    if constexpr (!kPromote) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        // an opaque use so the compiler cannot merge equal MFMAs
        asm volatile("" : "+v"(a));
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[n], acc[m][n], 0, 0, 0,
                                                                       0, 0, 0);
      }
    } else {
      v4f prev[4];
      float sc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        asm volatile("" : "+v"(a));
        v4f cur[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          cur[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a, b[n], v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if (m > 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[m - 1][n][r] = fmaf(prev[n][r], sc[r], acc[m - 1][n][r]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        sc[0] = s * 1.5f; sc[1] = s * 0.5f; sc[2] = s * 0.25f; sc[3] = s * 2.0f;
#pragma unroll
        for (int n = 0; n < 4; ++n) prev[n] = cur[n];
      }
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[7][n][r] = fmaf(prev[n][r], sc[r], acc[7][n][r]);
      s *= 1.0000001f;
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) sum += acc[m][n][r];
  out[(int64_t)blockIdx.x * 512 + t] = sum;
}

}  // namespace

// Launch `blocks` workgroups of 512 threads, each wave running `iters` loop
// iterations of 32 MFMAs (65536 FLOP each).  `out` holds blocks * 512
// floats (device).  promote selects the kernel.  Returns the hipError_t of
// the launch (0 on success); -1 for bad arguments.
extern "C" __attribute__((visibility("default"))) int fp8ceil_mfma(int promote, float *out,
                                                                   int blocks, int iters,
                                                                   void *stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0) return -1;
  if (promote)
    hipLaunchKernelGGL(mfma_ceiling_kernel<true>, dim3(blocks), dim3(512), 0,
                       (hipStream_t)stream, out, iters);
  else
    hipLaunchKernelGGL(mfma_ceiling_kernel<false>, dim3(blocks), dim3(512), 0,
                       (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}
