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
// kRandom = false keeps the operand registers nearly constant (one word of A
// changes per iteration), which is the least switching activity the matrix
// cores can see.  kRandom = true gives them the switching of a GEMM on real
// data without adding any instruction to the loop: four A and four B
// fragments hold independent random bits and the loop walks them as the GEMM
// walks its fragments (row m uses A[m mod 4], column n uses B[n]), so about
// half the operand bits flip between consecutive MFMAs.  Bit 6 of every fp8
// byte (the top exponent bit of E4M3) is clear, so every operand is a finite
// value below 2 in magnitude: no NaN, no overflow.
//
// 512 threads per workgroup (two waves per SIMD, as the GEMM runs).  With a
// non-null clk, thread 0 of each workgroup records the shader-clock
// (s_memtime) and the constant-rate wall-clock (s_memrealtime) ticks its
// loop took, so the host can read the engine clock the chip held.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kExpTopClear = (int)0xBFBFBFBFu;

__device__ __forceinline__ uint32_t xorshift32(uint32_t x) {
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  return x;
}

template <bool kPromote, bool kRandom>
__global__ __launch_bounds__(512) void mfma_ceiling_kernel(float *__restrict__ out,
                                                           unsigned long long *__restrict__ clk,
                                                           int iters) {
  constexpr int NA = kRandom ? 4 : 1;
  const int t = threadIdx.x;
  v8i a[NA], b[4];
  if constexpr (kRandom) {
    uint32_t x = 0x9E3779B9u ^ (uint32_t)(t * 0x85EBCA6Bu) ^ (uint32_t)(blockIdx.x * 0xC2B2AE35u);
#pragma unroll
    for (int j = 0; j < NA; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x = xorshift32(x);
        a[j][i] = (int)x & kExpTopClear;
      }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x = xorshift32(x);
        b[n][i] = (int)x & kExpTopClear;
      }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[0][i] = 0x38383838 ^ (t * 7 + i);
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 8; ++i) b[n][i] = 0x30303030 ^ (t * 3 + i + 8 * n);
  }
  v4f acc[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  float s = 1.0f + (float)t * 1e-7f;

  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if constexpr (!kRandom) a[0][0] ^= it;
    if constexpr (!kPromote) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        v8i &am = a[m % NA];
        // an opaque use so the compiler cannot merge equal MFMAs
        asm volatile("" : "+v"(am));
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(am, b[n], acc[m][n], 0, 0, 0,
                                                                       0, 0, 0);
      }
    } else {
      v4f prev[4];
      float sc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        v8i &am = a[m % NA];
        asm volatile("" : "+v"(am));
        v4f cur[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          cur[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              am, b[n], v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
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
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) sum += acc[m][n][r];
  out[(int64_t)blockIdx.x * 512 + t] = sum;
  if (clk != nullptr && t == 0) {
    clk[2 * (int64_t)blockIdx.x] = t1 - t0;
    clk[2 * (int64_t)blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

// Launch `blocks` workgroups of 512 threads, each wave running `iters` loop
// iterations of 32 MFMAs (65536 FLOP each).  mode bit 0 adds the fp32
// promotion, bit 1 gives the matrix cores random operand bits (see above).
// `out` holds blocks * 512 floats (device).  `clk` is null or holds
// 2 * blocks unsigned 64-bit words (device): per workgroup the shader-clock
// ticks, then the wall-clock ticks, of its loop.  Returns the hipError_t of
// the launch (0 on success); -1 for bad arguments.
extern "C" __attribute__((visibility("default"))) int fp8ceil_mfma(int mode, float *out,
                                                                   unsigned long long *clk,
                                                                   int blocks, int iters,
                                                                   void *stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0 || mode < 0 || mode > 3) return -1;
  const hipStream_t st = (hipStream_t)stream;
  switch (mode) {
    case 0: hipLaunchKernelGGL((mfma_ceiling_kernel<false, false>), dim3(blocks), dim3(512), 0, st, out, clk, iters); break;
    case 1: hipLaunchKernelGGL((mfma_ceiling_kernel<true, false>), dim3(blocks), dim3(512), 0, st, out, clk, iters); break;
    case 2: hipLaunchKernelGGL((mfma_ceiling_kernel<false, true>), dim3(blocks), dim3(512), 0, st, out, clk, iters); break;
    default: hipLaunchKernelGGL((mfma_ceiling_kernel<true, true>), dim3(blocks), dim3(512), 0, st, out, clk, iters); break;
  }
  return (int)hipGetLastError();
}

// The rate of the wall clock s_memrealtime reads, in kHz, for the current
// device; -1 on error.
extern "C" __attribute__((visibility("default"))) int fp8ceil_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1;
  return khz;
}
