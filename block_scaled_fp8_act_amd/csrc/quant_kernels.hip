// Activation (per token, per 128-channel group) and weight (per 128x128
// block) quantizers to E4M3, with fp32 scales or with power-of-two scales
// stored as E8M0 bytes ("UE8M0 scale format"), for gfx950.
//
// Both apply one element map to a set of bf16 values sharing a scale
// ("Fine-grained FP8" page of the transformers docs, introduction: weights
// per 2D block (128, 128); activations per token per group matching the
// weight block along the input channel; "DeepGEMM fast path": dynamic
// activation scales):  s = fl32(amax/448),  q = E4M3_RNE(fl32(x/s)).
//
// Both kernels are HBM-bound (3 bytes moved per element, plus 4 bytes per
// set), so the layout is chosen for fully coalesced 16-byte loads and the
// VALU work per element is kept small: the per-set division and reciprocal
// are paid once per set, and each element costs one multiply, two FMAs and
// half a packed conversion.
//
// E8M0 scales: the set's exponent e is the smallest integer >= -127 with
// amax <= 448 * 2^e (the scale rounded up to a power of two, so no quotient
// leaves E4M3's range), the stored byte is e + 127 and q = E4M3_RNE(x * 2^-e),
// an exact product: one multiply and half a packed conversion per element.
#include "fp8blk_device.h"
#include "fp8blk_launch.h"

namespace fp8blk {

// ---------------------------------------------------------------------------
// Activation quantizer.
//
// The input is viewed as a flat sequence of 128-element groups (row-major
// [M,K] with K % 128 == 0 makes group g = columns [128*(g % KB), +128) of row
// g / KB, and its scale lives at x_scale[g]).  A "tile" is 16 consecutive
// groups = 4 KB of bf16: load i (0..3) of lane l reads 16 bytes at
// tile*4096 + i*1024 + l*16, so every load instruction is one contiguous
// 1 KB run and each group is one DPP row of 16 lanes (8 values per lane).
// A wave handles two tiles per iteration (eight 16-byte loads in flight per
// lane).
//
// Fast path: when no group of the wave's tiles has 0 < amax < 2^-50 (always, in
// practice), s comes from div448, the power-of-two rescale is skipped
// (k = 0) and each element costs one multiply and two FMAs plus half a
// packed conversion.  Otherwise the wave takes the general element map of
// make_qparams / quotient.  Both agree with the IEEE definition on every
// (x, amax) bf16 pair.
constexpr int kActThreads = 256;
constexpr int kActWaves = kActThreads / 64;
constexpr int kGroupsPerTile = 16;
constexpr int kTilesPerIter = 2;
constexpr float kTinyAmax = 0x1p-50f;


__global__ __launch_bounds__(kActThreads) void act_quant_kernel(
    const uint4 *__restrict__ x, uint2 *__restrict__ q, float *__restrict__ scale,
    int64_t n_groups) {
  constexpr int L = 4 * kTilesPerIter;  // loads per lane per iteration
  const int lane = threadIdx.x & 63;
  const int64_t n_tiles = (n_groups + kGroupsPerTile - 1) / kGroupsPerTile;
  const int64_t stride = (int64_t)gridDim.x * kActWaves * kTilesPerIter;
  for (int64_t tile0 = ((int64_t)blockIdx.x * kActWaves + (threadIdx.x >> 6)) * kTilesPerIter;
       tile0 < n_tiles; tile0 += stride) {
    uint4 v[L];
    bool ok[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int64_t g = tile0 * kGroupsPerTile + i * 4 + (lane >> 4);
      ok[i] = g < n_groups;
      v[i] = ok[i] ? x[tile0 * 256 + i * 64 + lane] : make_uint4(0, 0, 0, 0);
    }
    float amax[L];
    bool tiny = false;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      float f[8];
      unpack8(v[i], f);
      amax[i] = row16_max(absmax8(f));
      tiny |= ok[i] && amax[i] > 0.0f && amax[i] < kTinyAmax;
    }
    if (__builtin_amdgcn_ballot_w64(tiny) == 0) {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        float f[8];
        unpack8(v[i], f);
        const float s = div448(amax[i]);
        const float sp = s == 0.0f ? 1.0f : s;   // all-zero group: codes are +-0
        const float y = 1.0f / sp;
        float t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = quotient(f[j], sp, y);
        uint2 out;
        out.x = pack4_e4m3(t[0], t[1], t[2], t[3]);
        out.y = pack4_e4m3(t[4], t[5], t[6], t[7]);
        if (ok[i]) {
          q[tile0 * 256 + i * 64 + lane] = out;
          if ((lane & 15) == 0) scale[tile0 * kGroupsPerTile + i * 4 + (lane >> 4)] = s;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        float f[8];
        unpack8(v[i], f);
        const QParams p = make_qparams(amax[i]);
        float t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = quotient(ldexpf(f[j], p.k), p.sp, p.y);
        uint2 out;
        out.x = pack4_e4m3(t[0], t[1], t[2], t[3]);
        out.y = pack4_e4m3(t[4], t[5], t[6], t[7]);
        if (ok[i]) {
          q[tile0 * 256 + i * 64 + lane] = out;
          if ((lane & 15) == 0) scale[tile0 * kGroupsPerTile + i * 4 + (lane >> 4)] = p.s;
        }
      }
    }
  }
}

// Power-of-two variant: same tiles and loads; one byte per group.
__global__ __launch_bounds__(kActThreads) void act_quant_e8m0_kernel(
    const uint4 *__restrict__ x, uint2 *__restrict__ q, uint8_t *__restrict__ scale,
    int64_t n_groups) {
  constexpr int L = 4 * kTilesPerIter;
  const int lane = threadIdx.x & 63;
  const int64_t n_tiles = (n_groups + kGroupsPerTile - 1) / kGroupsPerTile;
  const int64_t stride = (int64_t)gridDim.x * kActWaves * kTilesPerIter;
  for (int64_t tile0 = ((int64_t)blockIdx.x * kActWaves + (threadIdx.x >> 6)) * kTilesPerIter;
       tile0 < n_tiles; tile0 += stride) {
    uint4 v[L];
    bool ok[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int64_t g = tile0 * kGroupsPerTile + i * 4 + (lane >> 4);
      ok[i] = g < n_groups;
      v[i] = ok[i] ? x[tile0 * 256 + i * 64 + lane] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
      float f[8];
      unpack8(v[i], f);
      const int e = e8m0_exponent(row16_max(absmax8(f)));
      const float r = e8m0_inv_scale(e);
      uint2 out;
      out.x = pack4_e4m3(f[0] * r, f[1] * r, f[2] * r, f[3] * r);
      out.y = pack4_e4m3(f[4] * r, f[5] * r, f[6] * r, f[7] * r);
      if (ok[i]) {
        q[tile0 * 256 + i * 64 + lane] = out;
        if ((lane & 15) == 0)
          scale[tile0 * kGroupsPerTile + i * 4 + (lane >> 4)] = (uint8_t)(e + 127);
      }
    }
  }
}

// Static variant: one caller-supplied scale for the whole tensor (device
// memory, read once per thread), q = E4M3_RNE(sat(fl32(x / s))).  The
// quotient is the IEEE division (the compiler's correctly rounded sequence;
// an arbitrary calibrated s has no precomputed reciprocal that is exact for
// every x), then clamped to +-448 -- here inputs can exceed the calibrated
// range, and the conversion without its clamp bit returns NaN from 464.
// Each thread converts 16 consecutive elements per iteration (two 16-byte
// loads, one 16-byte store).
constexpr int kStaticThreads = 256;

__device__ __forceinline__ float sat448(float t) { return fminf(fmaxf(t, -448.0f), 448.0f); }

__global__ __launch_bounds__(kStaticThreads) void act_quant_static_kernel(
    const uint4 *__restrict__ x, uint4 *__restrict__ q, const float *__restrict__ scale,
    int64_t n16) {
  const float s = *scale;
  const int64_t stride = (int64_t)gridDim.x * kStaticThreads;
  for (int64_t i = (int64_t)blockIdx.x * kStaticThreads + threadIdx.x; i < n16; i += stride) {
    const uint4 v0 = x[2 * i], v1 = x[2 * i + 1];
    float f[16];
    unpack8(v0, f);
    unpack8(v1, f + 8);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = pack4_e4m3(sat448(f[4 * j] / s), sat448(f[4 * j + 1] / s), sat448(f[4 * j + 2] / s),
                        sat448(f[4 * j + 3] / s));
    q[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---------------------------------------------------------------------------
// Row-wise quantizer (one scale per row: weights' output rows, or tokens):
// one workgroup per row, an amax pass and a quantize pass over the row (the
// second pass re-reads the row from L2 for the usual K), with the element map
// of make_qparams / quotient.
constexpr int kRowThreads = 256;

__global__ __launch_bounds__(kRowThreads) void rowwise_quant_kernel(
    const uint16_t *__restrict__ x, int64_t K, uint8_t *__restrict__ q, float *__restrict__ scale) {
  __shared__ float wave_max[kRowThreads / 64];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const uint4 *xr = reinterpret_cast<const uint4 *>(x + row * K);
  const int64_t n8 = K / 8;
  float m = 0.0f;
  for (int64_t i = t; i < n8; i += kRowThreads) {
    float f[8];
    unpack8(xr[i], f);
    m = fmaxf(m, absmax8(f));
  }
  m = row16_max(m);
  m = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0)),
                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16))),
            fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32)),
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48))));
  if (lane == 0) wave_max[t >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  const QParams p = make_qparams(amax);
  uint2 *qr = reinterpret_cast<uint2 *>(q + row * K);
  for (int64_t i = t; i < n8; i += kRowThreads) {
    float f[8];
    unpack8(xr[i], f);
    float tq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) tq[j] = quotient(ldexpf(f[j], p.k), p.sp, p.y);
    uint2 out;
    out.x = pack4_e4m3(tq[0], tq[1], tq[2], tq[3]);
    out.y = pack4_e4m3(tq[4], tq[5], tq[6], tq[7]);
    qr[i] = out;
  }
  if (t == 0) scale[row] = p.s;
}

// ---------------------------------------------------------------------------
// Weight quantizer: one workgroup per 128x128 block.  Thread t reads, for
// i = 0..7, the 16 bytes at row i*16 + t/16, columns (t%16)*8 .. +8 of the
// block, so each wave covers four full 256-byte rows per load.  Rows past N
// (a short last block row) are skipped and do not enter the amax.
constexpr int kWqThreads = 256;

// E8M0 selects power-of-two scales (one byte each) over fp32 scales.
template <bool E8M0>
__global__ __launch_bounds__(kWqThreads) void weight_quant_kernel(
    const uint16_t *__restrict__ w, uint8_t *__restrict__ q, void *__restrict__ scale,
    int64_t N, int64_t K) {
  __shared__ float wave_max[kWqThreads / 64];
  const int64_t KB = K / kBlock;
  const int64_t kb = blockIdx.x % KB;
  const int64_t nb = blockIdx.x / KB;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int col = (t & 15) * 8;
  uint4 v[8];
  bool ok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = nb * kBlock + i * 16 + (t >> 4);
    ok[i] = row < N;
    v[i] = ok[i] ? *reinterpret_cast<const uint4 *>(w + row * K + kb * kBlock + col)
                 : make_uint4(0, 0, 0, 0);
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(v[i].x)), fabsf(bf16_hi(v[i].x))),
                       fmaxf(fabsf(bf16_lo(v[i].y)), fabsf(bf16_hi(v[i].y)))));
    m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(v[i].z)), fabsf(bf16_hi(v[i].z))),
                       fmaxf(fabsf(bf16_lo(v[i].w)), fabsf(bf16_hi(v[i].w)))));
  }
  m = row16_max(m);
  m = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0)),
                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16))),
            fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32)),
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48))));
  if (lane == 0) wave_max[t >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  QParams p;
  int e = 0;
  float r = 1.0f;
  if constexpr (E8M0) {
    e = e8m0_exponent(amax);
    r = e8m0_inv_scale(e);
  } else {
    p = make_qparams(amax);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = nb * kBlock + i * 16 + (t >> 4);
    float f[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                  bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
    float tq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (E8M0) tq[j] = f[j] * r;
      else tq[j] = quotient(ldexpf(f[j], p.k), p.sp, p.y);
    }
    uint2 out;
    out.x = pack4_e4m3(tq[0], tq[1], tq[2], tq[3]);
    out.y = pack4_e4m3(tq[4], tq[5], tq[6], tq[7]);
    if (ok[i]) *reinterpret_cast<uint2 *>(q + row * K + kb * kBlock + col) = out;
  }
  if (t == 0) {
    if constexpr (E8M0) static_cast<uint8_t *>(scale)[nb * KB + kb] = (uint8_t)(e + 127);
    else static_cast<float *>(scale)[nb * KB + kb] = p.s;
  }
}

// ---------------------------------------------------------------------------
static unsigned act_quant_blocks(int64_t n_groups) {
  const int64_t n_tiles = (n_groups + kGroupsPerTile - 1) / kGroupsPerTile;
  const int64_t per_block = (int64_t)kActWaves * kTilesPerIter;
  int64_t blocks = (n_tiles + per_block - 1) / per_block;
  const int64_t cap = 256 * 8;  // grid-stride beyond 8 workgroups per CU
  return (unsigned)(blocks > cap ? cap : blocks);
}

hipError_t launch_act_quant(const void *x, int64_t M, int64_t K, void *q, float *s,
                            hipStream_t stream) {
  const int64_t n_groups = M * (K / kBlock);
  hipLaunchKernelGGL(act_quant_kernel, dim3(act_quant_blocks(n_groups)), dim3(kActThreads), 0,
                     stream, static_cast<const uint4 *>(x), static_cast<uint2 *>(q), s, n_groups);
  return hipGetLastError();
}

hipError_t launch_act_quant_e8m0(const void *x, int64_t M, int64_t K, void *q, uint8_t *s,
                                 hipStream_t stream) {
  const int64_t n_groups = M * (K / kBlock);
  hipLaunchKernelGGL(act_quant_e8m0_kernel, dim3(act_quant_blocks(n_groups)), dim3(kActThreads),
                     0, stream, static_cast<const uint4 *>(x), static_cast<uint2 *>(q), s,
                     n_groups);
  return hipGetLastError();
}

hipError_t launch_act_quant_static(const void *x, int64_t M, int64_t K, const float *s, void *q,
                                   hipStream_t stream) {
  const int64_t n16 = M * K / 16;  // K % 128 == 0
  int64_t blocks = (n16 + kStaticThreads - 1) / kStaticThreads;
  if (blocks > 256 * 8) blocks = 256 * 8;
  hipLaunchKernelGGL(act_quant_static_kernel, dim3((unsigned)blocks), dim3(kStaticThreads), 0,
                     stream, static_cast<const uint4 *>(x), static_cast<uint4 *>(q), s, n16);
  return hipGetLastError();
}

hipError_t launch_rowwise_quant(const void *x, int64_t R, int64_t K, void *q, float *s,
                                hipStream_t stream) {
  hipLaunchKernelGGL(rowwise_quant_kernel, dim3((unsigned)R), dim3(kRowThreads), 0, stream,
                     static_cast<const uint16_t *>(x), K, static_cast<uint8_t *>(q), s);
  return hipGetLastError();
}

hipError_t launch_weight_quant(const void *w, int64_t N, int64_t K, void *q, float *s,
                               hipStream_t stream) {
  const int64_t NB = (N + kBlock - 1) / kBlock;
  const int64_t KB = K / kBlock;
  hipLaunchKernelGGL(weight_quant_kernel<false>, dim3((unsigned)(NB * KB)), dim3(kWqThreads), 0,
                     stream, static_cast<const uint16_t *>(w), static_cast<uint8_t *>(q),
                     static_cast<void *>(s), N, K);
  return hipGetLastError();
}

hipError_t launch_weight_quant_e8m0(const void *w, int64_t N, int64_t K, void *q, uint8_t *s,
                                    hipStream_t stream) {
  const int64_t NB = (N + kBlock - 1) / kBlock;
  const int64_t KB = K / kBlock;
  hipLaunchKernelGGL(weight_quant_kernel<true>, dim3((unsigned)(NB * KB)), dim3(kWqThreads), 0,
                     stream, static_cast<const uint16_t *>(w), static_cast<uint8_t *>(q),
                     static_cast<void *>(s), N, K);
  return hipGetLastError();
}

}  // namespace fp8blk
