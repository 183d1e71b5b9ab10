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
// A wave handles one tile per iteration (four 16-byte loads in flight per
// lane) and the grid holds up to 32 workgroups per CU: more, shorter-lived
// waves measured 2-11 % faster than two tiles per wave and 8 workgroups
// per CU (4096x4096: 12.0 -> 10.7 us from HBM).
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
constexpr int kTilesPerIter = 1;
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
      v[i] = ok[i] ? ld_stream(x + tile0 * 256 + i * 64 + lane) : make_uint4(0, 0, 0, 0);
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
      v[i] = ok[i] ? ld_stream(x + tile0 * 256 + i * 64 + lane) : make_uint4(0, 0, 0, 0);
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
    const uint4 v0 = ld_stream(x + 2 * i), v1 = ld_stream(x + 2 * i + 1);
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
// one workgroup per row, an amax pass and a quantize pass over the row, with
// the element map of make_qparams / quotient.  Rows of up to 32768 values
// stay in registers between the passes; longer rows are re-read.
constexpr int kRowThreads = 256;

// C > 0: rows of at most C * 8 * kRowThreads values, held in registers
// between the amax and the quantization (one pass over HBM); C = 0: any
// length, the row re-read (from L2 for the usual K) for the second pass.
template <int C>
__global__ __launch_bounds__(kRowThreads) void rowwise_quant_kernel(
    const uint16_t *__restrict__ x, int64_t K, uint8_t *__restrict__ q, float *__restrict__ scale) {
  __shared__ float wave_max[kRowThreads / 64];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const uint4 *xr = reinterpret_cast<const uint4 *>(x + row * K);
  const int64_t n8 = K / 8;
  float m = 0.0f;
  uint4 v[C > 0 ? C : 1];
  if constexpr (C > 0) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int64_t i = t + (int64_t)c * kRowThreads;
      v[c] = i < n8 ? ld_stream(xr + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float f[8];
      unpack8(v[c], f);
      m = fmaxf(m, absmax8(f));
    }
  } else {
    for (int64_t i = t; i < n8; i += kRowThreads) {
      float f[8];
      unpack8(xr[i], f);
      m = fmaxf(m, absmax8(f));
    }
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
  auto quant8 = [&](const uint4 &w) {
    float f[8];
    unpack8(w, f);
    float tq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) tq[j] = quotient(ldexpf(f[j], p.k), p.sp, p.y);
    uint2 out;
    out.x = pack4_e4m3(tq[0], tq[1], tq[2], tq[3]);
    out.y = pack4_e4m3(tq[4], tq[5], tq[6], tq[7]);
    return out;
  };
  if constexpr (C > 0) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int64_t i = t + (int64_t)c * kRowThreads;
      if (i < n8) qr[i] = quant8(v[c]);
    }
  } else {
    for (int64_t i = t; i < n8; i += kRowThreads) qr[i] = quant8(xr[i]);
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
    v[i] = ok[i] ? ld_stream(reinterpret_cast<const uint4 *>(w + row * K + kb * kBlock + col))
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
// ---------------------------------------------------------------------------
// SwiGLU ahead of the activation quantizer: the quantized input of a
// mixture-of-experts down projection, straight from the gate/up projection's
// bf16 output.  A token's gate/up row holds the gate g in columns [0, I) and
// the up value u in [I, 2I); h = bf16_RNE(SiLU(g) * u) with SiLU(g) =
// g / (1 + e^-g) is defined by its binary64 evaluation (IEEE division, the
// math library's exp), whose bf16 rounding is that of the exact value except
// within ~2^-52 of a rounding midpoint; an fp32 evaluation is used wherever
// its rounding is certified to be the same (swiglu_h32).  h [M, I] is then
// quantized per token per 128-group with the element map of make_qparams /
// quotient (bit-identical to act_quant_kernel).  h never goes to memory: 4 bytes read and 1 + 4/128
// written per element of h, against 4 + 2 and 2 + 1 + 4/128 for a SwiGLU
// kernel followed by the quantizer.
//
// Tiles as in act_quant_kernel but of 8 groups, over h's groups (group G =
// row G / (I/128), 128-column block G % (I/128)), one tile per wave per
// iteration: load i of lane l holds 8 gate values of group 8*tile + 4i + l/16
// and, I columns further, the matching 8 up values.  The small tile keeps
// registers low (45) for occupancy: the kernel is about as much ALU work as
// memory traffic.

// binary64 -> the nearest bf16 value (ties to even), as an exact fp32.  At or
// above 2^-126 the significand is rounded to 8 bits on the bit pattern (a
// carry into the exponent field is the correct result; past bf16's largest
// value the conversion to fp32 overflows to infinity); below, the quantum is
// 2^-133 and the value is rounded by scaling.
__device__ __forceinline__ float bf16_round_f64(double h) {
  const uint64_t b = (uint64_t)__double_as_longlong(h);
  if (((b >> 52) & 0x7ff) >= 1023 - 126) {
    const uint64_t r = (b + 0xFFFFFFFFFFFull + ((b >> 45) & 1)) & ~0x1FFFFFFFFFFFull;
    return (float)__longlong_as_double((long long)r);
  }
  return (float)(rint(h * 0x1p133) * 0x1p-133);
}

// Kept out of line: it runs for about one element in 2000, and inlined at
// every element it would hold its constants in registers throughout.
__device__ __attribute__((noinline)) float swiglu_h64(float g, float u) {
  const double gd = g;
  return bf16_round_f64(gd / (1.0 + exp(-gd)) * (double)u);
}

// e^x for x <= 80 in fp32 from the hardware base-2 exponential: x * log2(e)
// is formed as th + tl with log2(e) split into an fp32 head and tail and the
// head product's rounding error recovered exactly by an FMA, so th is an
// fp32 value and |tl| < 2^-16; then e^x = 2^th * 2^tl with 2^tl = 1 + tl ln 2
// to within 2^-33.  Relative error: v_exp_f32's (1 ulp) plus one rounding,
// below 3 * 2^-24.  Results below 2^-126 may be flushed, and x is clamped
// at -150 so that nothing overflows (callers only add such results to 1).
__device__ __forceinline__ float exp_small(float x) {
  constexpr float kL2eHi = 1.44269502162933349609375f;  // fp32(log2 e)
  constexpr float kL2eLo = 1.925963033500011e-08f;      // log2 e - kL2eHi
  x = fmaxf(x, -150.0f);
  const float th = x * kL2eHi;
  const float tl = fmaf(x, kL2eHi, -th) + x * kL2eLo;
  const float e0 = __builtin_amdgcn_exp2f(th);
  return fmaf(e0, tl * 0.693147180559945309f, e0);
}

// Fast path: the same expression in fp32 (exp_small, the hardware
// reciprocal, within 1 ulp).  Relative to the exact value its error is
// below 8 * 2^-24, i.e. at most 8 fp32 ulps of the result, provided nothing
// over- or underflows: g >= -80 (e^-g finite), |g| >= 2^-100 (SiLU(g)
// normal) and 2^-120 <= |h| < 2^126.  If moreover the result lies more than
// 16 fp32 ulps from a bf16 rounding midpoint (its low 16 bits differ from
// 0x8000 by more than 16), the exact value, the binary64 evaluation and this
// result all round to the same bf16 value, which is returned with ok = true;
// otherwise ok = false and the caller takes swiglu_h64 (about 1 element in
// 2000).
__device__ __forceinline__ float swiglu_h32(float g, float u, bool &ok) {
  const float e = exp_small(-g);
  const float hf = g * __builtin_amdgcn_rcpf(1.0f + e) * u;
  const uint32_t b = __float_as_uint(hf);
  const uint32_t mag = b & 0x7fffffffu;
  const int dist = (int)(b & 0xffffu) - 0x8000;
  // g = 0 or u = 0 (with e^-g finite): hf is the exact signed zero that
  // the binary64 evaluation gives too
  ok = g >= -80.0f && (g == 0.0f || u == 0.0f ||
                       (fabsf(g) >= 0x1p-100f && mag >= 0x03800000u && mag < 0x7e800000u &&
                        (dist > 16 || dist < -16)));
  return __uint_as_float((b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u);
}

constexpr int kSwigluGpt = 8;  // groups per tile of swiglu_quant_kernel (4 per load)

// E8M0: power-of-two scales as in act_quant_e8m0_kernel (scale = bytes).
template <bool E8M0>
__global__ __launch_bounds__(kActThreads) void swiglu_quant_kernel(
    const uint16_t *__restrict__ gu, uint32_t gpr, uint2 *__restrict__ q,
    void *__restrict__ scale, uint32_t n_groups) {
  constexpr int kGpt = kSwigluGpt;
  constexpr int L = kGpt / 4;  // 16-byte gate and up loads per lane per tile
  const int lane = threadIdx.x & 63;
  const int64_t I = (int64_t)gpr * kBlock;
  const uint32_t n_tiles = (n_groups + kGpt - 1) / kGpt;
  const uint32_t stride = gridDim.x * kActWaves;
  for (uint32_t tile = blockIdx.x * kActWaves + (threadIdx.x >> 6); tile < n_tiles;
       tile += stride) {
    uint4 vg[L], vu[L];
    bool ok[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const uint32_t G = tile * kGpt + i * 4 + (lane >> 4);
      ok[i] = G < n_groups;
      const uint32_t Gc = ok[i] ? G : 0;
      const uint32_t m = Gc / gpr, j = Gc - m * gpr;
      const uint4 *p =
          reinterpret_cast<const uint4 *>(gu + (int64_t)m * 2 * I + (int64_t)j * kBlock) +
          (lane & 15);
      vg[i] = ok[i] ? ld_stream(p) : make_uint4(0, 0, 0, 0);
      vu[i] = ok[i] ? ld_stream(p + I / 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
      float g[8], u[8], h[8];
      unpack8(vg[i], g);
      unpack8(vu[i], u);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bool ok32;
        h[j] = swiglu_h32(g[j], u[j], ok32);
        if (!ok32) h[j] = swiglu_h64(g[j], u[j]);
      }
      const float amax = row16_max(absmax8(h));
      if constexpr (E8M0) {
        const int e = e8m0_exponent(amax);
        const float r = e8m0_inv_scale(e);
        uint2 out;
        out.x = pack4_e4m3(h[0] * r, h[1] * r, h[2] * r, h[3] * r);
        out.y = pack4_e4m3(h[4] * r, h[5] * r, h[6] * r, h[7] * r);
        if (ok[i]) {
          const uint32_t G = tile * kGpt + i * 4 + (lane >> 4);
          q[(int64_t)G * 16 + (lane & 15)] = out;
          if ((lane & 15) == 0) static_cast<uint8_t *>(scale)[G] = (uint8_t)(e + 127);
        }
        continue;
      }
      float t[8], sc;
      if (__builtin_amdgcn_ballot_w64(amax > 0.0f && amax < kTinyAmax) == 0) {
        // as act_quant_kernel's fast path: no power-of-two rescale
        sc = div448(amax);
        const float sp = sc == 0.0f ? 1.0f : sc;
        const float y = 1.0f / sp;
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = quotient(h[j], sp, y);
      } else {
        const QParams p = make_qparams(amax);
        sc = p.s;
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = quotient(ldexpf(h[j], p.k), p.sp, p.y);
      }
      uint2 out;
      out.x = pack4_e4m3(t[0], t[1], t[2], t[3]);
      out.y = pack4_e4m3(t[4], t[5], t[6], t[7]);
      if (ok[i]) {
        const uint32_t G = tile * kGpt + i * 4 + (lane >> 4);
        q[(int64_t)G * 16 + (lane & 15)] = out;
        if ((lane & 15) == 0) static_cast<float *>(scale)[G] = sc;
      }
    }
  }
}

static unsigned act_quant_blocks(int64_t n_groups) {
  const int64_t n_tiles = (n_groups + kGroupsPerTile - 1) / kGroupsPerTile;
  const int64_t per_block = (int64_t)kActWaves * kTilesPerIter;
  int64_t blocks = (n_tiles + per_block - 1) / per_block;
  const int64_t cap = 256 * 32;  // grid-stride beyond 32 workgroups per CU
  return (unsigned)(blocks > cap ? cap : blocks);
}

hipError_t launch_act_quant(const void *x, int64_t M, int64_t K, void *q, float *s,
                            hipStream_t stream) {
  const int64_t n_groups = M * (K / kBlock);
  hipLaunchKernelGGL(act_quant_kernel, dim3(act_quant_blocks(n_groups)), dim3(kActThreads), 0,
                     stream, static_cast<const uint4 *>(x), static_cast<uint2 *>(q), s, n_groups);
  return hipGetLastError();
}

template <bool E8M0>
static hipError_t launch_swiglu(const void *gu, int64_t M, int64_t I, void *q, void *s,
                                hipStream_t stream) {
  const int64_t n_groups = M * (I / kBlock);  // < 2^31 (checked by the caller)
  const int64_t n_tiles = (n_groups + kSwigluGpt - 1) / kSwigluGpt;
  int64_t blocks = (n_tiles + kActWaves - 1) / kActWaves;
  if (blocks > 256 * 32) blocks = 256 * 32;  // up to 32 workgroups per CU
  hipLaunchKernelGGL(swiglu_quant_kernel<E8M0>, dim3((unsigned)blocks), dim3(kActThreads), 0,
                     stream, static_cast<const uint16_t *>(gu), (uint32_t)(I / kBlock),
                     static_cast<uint2 *>(q), s, (uint32_t)n_groups);
  return hipGetLastError();
}

hipError_t launch_swiglu_act_quant(const void *gu, int64_t M, int64_t I, void *q, float *s,
                                   hipStream_t stream) {
  return launch_swiglu<false>(gu, M, I, q, s, stream);
}

hipError_t launch_swiglu_act_quant_e8m0(const void *gu, int64_t M, int64_t I, void *q,
                                        uint8_t *s, hipStream_t stream) {
  return launch_swiglu<true>(gu, M, I, q, s, stream);
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
  if (blocks > 256 * 32) blocks = 256 * 32;  // up to 32 workgroups per CU
  hipLaunchKernelGGL(act_quant_static_kernel, dim3((unsigned)blocks), dim3(kStaticThreads), 0,
                     stream, static_cast<const uint4 *>(x), static_cast<uint4 *>(q), s, n16);
  return hipGetLastError();
}

hipError_t launch_rowwise_quant(const void *x, int64_t R, int64_t K, void *q, float *s,
                                hipStream_t stream) {
  const int64_t chunks = (K / 8 + kRowThreads - 1) / kRowThreads;  // 16-byte loads per thread
  const auto *xp = static_cast<const uint16_t *>(x);
  auto *qp = static_cast<uint8_t *>(q);
  if (chunks <= 2)
    hipLaunchKernelGGL(rowwise_quant_kernel<2>, dim3((unsigned)R), dim3(kRowThreads), 0, stream,
                       xp, K, qp, s);
  else if (chunks <= 4)
    hipLaunchKernelGGL(rowwise_quant_kernel<4>, dim3((unsigned)R), dim3(kRowThreads), 0, stream,
                       xp, K, qp, s);
  else if (chunks <= 8)
    hipLaunchKernelGGL(rowwise_quant_kernel<8>, dim3((unsigned)R), dim3(kRowThreads), 0, stream,
                       xp, K, qp, s);
  else if (chunks <= 16)
    hipLaunchKernelGGL(rowwise_quant_kernel<16>, dim3((unsigned)R), dim3(kRowThreads), 0, stream,
                       xp, K, qp, s);
  else
    hipLaunchKernelGGL(rowwise_quant_kernel<0>, dim3((unsigned)R), dim3(kRowThreads), 0, stream,
                       xp, K, qp, s);
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
