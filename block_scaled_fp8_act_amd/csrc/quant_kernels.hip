// Activation (per token, per 128-channel group) and weight (per 128x128
// block) quantizers to E4M3 with fp32 scales, for gfx950.
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
// are paid once per set, and each element costs one multiply, two FMAs, a
// clamp and half a packed conversion.
#include "fp8blk_device.h"
#include "fp8blk_launch.h"

namespace fp8blk {

// ---------------------------------------------------------------------------
// Activation quantizer.
//
// The input is viewed as a flat sequence of 128-element groups (row-major
// [M,K] with K % 128 == 0 makes group g = columns [128*(g % KB), +128) of row
// g / KB, and its scale lives at x_scale[g]).  A wave handles a "tile" of 16
// consecutive groups = 4 KB of bf16: load i (0..3) of lane l reads 16 bytes
// at tile*4096 + i*1024 + l*16, so every load instruction is one contiguous
// 1 KB run and each group is one DPP row of 16 lanes (8 values per lane).
constexpr int kActThreads = 256;
constexpr int kActWaves = kActThreads / 64;
constexpr int kGroupsPerTile = 16;

__global__ __launch_bounds__(kActThreads) void act_quant_kernel(
    const uint4 *__restrict__ x, uint2 *__restrict__ q, float *__restrict__ scale,
    int64_t n_groups) {
  const int lane = threadIdx.x & 63;
  const int64_t n_tiles = (n_groups + kGroupsPerTile - 1) / kGroupsPerTile;
  const int64_t stride = (int64_t)gridDim.x * kActWaves;
  for (int64_t tile = (int64_t)blockIdx.x * kActWaves + (threadIdx.x >> 6); tile < n_tiles;
       tile += stride) {
    uint4 v[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t g = tile * kGroupsPerTile + i * 4 + (lane >> 4);
      ok[i] = g < n_groups;
      v[i] = ok[i] ? x[tile * 256 + i * 64 + lane] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float f[8];
      f[0] = bf16_lo(v[i].x); f[1] = bf16_hi(v[i].x);
      f[2] = bf16_lo(v[i].y); f[3] = bf16_hi(v[i].y);
      f[4] = bf16_lo(v[i].z); f[5] = bf16_hi(v[i].z);
      f[6] = bf16_lo(v[i].w); f[7] = bf16_hi(v[i].w);
      float m = fmaxf(fmaxf(fabsf(f[0]), fabsf(f[1])), fmaxf(fabsf(f[2]), fabsf(f[3])));
      m = fmaxf(m, fmaxf(fmaxf(fabsf(f[4]), fabsf(f[5])), fmaxf(fabsf(f[6]), fabsf(f[7]))));
      const float amax = row16_max(m);
      const QParams p = make_qparams(amax);
      float t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = quotient(ldexpf(f[j], p.k), p.sp, p.y);
      uint2 out;
      out.x = pack4_e4m3(t[0], t[1], t[2], t[3]);
      out.y = pack4_e4m3(t[4], t[5], t[6], t[7]);
      if (ok[i]) {
        q[tile * 256 + i * 64 + lane] = out;
        if ((lane & 15) == 0) scale[tile * kGroupsPerTile + i * 4 + (lane >> 4)] = p.s;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Weight quantizer: one workgroup per 128x128 block.  Thread t reads, for
// i = 0..7, the 16 bytes at row i*16 + t/16, columns (t%16)*8 .. +8 of the
// block, so each wave covers four full 256-byte rows per load.  Rows past N
// (a short last block row) are skipped and do not enter the amax.
constexpr int kWqThreads = 256;

__global__ __launch_bounds__(kWqThreads) void weight_quant_kernel(
    const uint16_t *__restrict__ w, uint8_t *__restrict__ q, float *__restrict__ scale,
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
  const QParams p = make_qparams(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = nb * kBlock + i * 16 + (t >> 4);
    float f[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                  bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
    float tq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) tq[j] = quotient(ldexpf(f[j], p.k), p.sp, p.y);
    uint2 out;
    out.x = pack4_e4m3(tq[0], tq[1], tq[2], tq[3]);
    out.y = pack4_e4m3(tq[4], tq[5], tq[6], tq[7]);
    if (ok[i]) *reinterpret_cast<uint2 *>(q + row * K + kb * kBlock + col) = out;
  }
  if (t == 0) scale[nb * KB + kb] = p.s;
}

// ---------------------------------------------------------------------------
hipError_t launch_act_quant(const void *x, int64_t M, int64_t K, void *q, float *s,
                            hipStream_t stream) {
  const int64_t n_groups = M * (K / kBlock);
  const int64_t n_tiles = (n_groups + kGroupsPerTile - 1) / kGroupsPerTile;
  int64_t blocks = (n_tiles + kActWaves - 1) / kActWaves;
  const int64_t cap = 256 * 16;  // grid-stride beyond 16 workgroups per CU
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(act_quant_kernel, dim3((unsigned)blocks), dim3(kActThreads), 0, stream,
                     static_cast<const uint4 *>(x), static_cast<uint2 *>(q), s, n_groups);
  return hipGetLastError();
}

hipError_t launch_weight_quant(const void *w, int64_t N, int64_t K, void *q, float *s,
                               hipStream_t stream) {
  const int64_t NB = (N + kBlock - 1) / kBlock;
  const int64_t KB = K / kBlock;
  hipLaunchKernelGGL(weight_quant_kernel, dim3((unsigned)(NB * KB)), dim3(kWqThreads), 0,
                     stream, static_cast<const uint16_t *>(w), static_cast<uint8_t *>(q), s, N, K);
  return hipGetLastError();
}

}  // namespace fp8blk
