// Device helpers shared by the fp8blk kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

constexpr int kBlock = 128;  // weight block edge and activation group width

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// bf16 halves of a packed dword -> fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Eight bf16 (one 16-byte load) -> fp32, and their largest magnitude.
__device__ __forceinline__ void unpack8(const uint4 &v, float *f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// 16-byte load of input that is read exactly once (the quantizers' bf16
// input): non-temporal, so the stream does not displace cached data.
// Measured on 4096x14336 bf16 from HBM: 32.7 -> 29.4 us for the activation
// quantizer (5.44 -> 6.07 TB/s).
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ float absmax8(const float *f) {
  return fmaxf(fmaxf(fmaxf(fabsf(f[0]), fabsf(f[1])), fmaxf(fabsf(f[2]), fabsf(f[3]))),
               fmaxf(fmaxf(fabsf(f[4]), fabsf(f[5])), fmaxf(fabsf(f[6]), fabsf(f[7]))));
}

// DPP lane permutes inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over the 16 lanes of a DPP row (values are >= 0); every lane gets it.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_f<0x128>(v));  // row_ror:8
  return v;
}

// Quantization parameters of one block or group.
//   s  = fl32(amax / 448)           (IEEE division, denormals kept)
//   sp = s * 2^k, y = fl32(1 / sp)  with k > 0 only for tiny s (< 2^-64),
//        so that sp, y and the residual below stay far from underflow.
// The quotient fl32(x / s) is then x' * y corrected once with an exact FMA
// residual (Markstein's correction with a correctly rounded reciprocal),
// x' = x * 2^k.  For every bf16 x with |x| <= amax this equals the IEEE
// quotient wherever the quotient can round to a nonzero E4M3 code, and
// gives the same signed-zero code elsewhere (checked over all
// 1,065,402,238 (x, amax) bf16 pairs).  An all-zero set gets s = 0 and
// sp = y = 1, which maps +-0 to +-0.
struct QParams {
  float s, sp, y;
  int k;
};

__device__ __forceinline__ QParams make_qparams(float amax) {
  QParams p;
  p.s = amax / 448.0f;
  p.k = 0;
  if (p.s == 0.0f) {
    p.sp = 1.0f;
    p.y = 1.0f;
  } else {
    if (p.s < 0x1p-64f) {
      int e;
      (void)frexpf(p.s, &e);
      p.k = 1 - e;
    }
    p.sp = ldexpf(p.s, p.k);
    p.y = 1.0f / p.sp;
  }
  return p;
}

// fl32(x / s) for x' = x * 2^k already formed.
__device__ __forceinline__ float quotient(float xp, float sp, float y) {
  const float q0 = xp * y;
  const float nr = fmaf(q0, sp, -xp);  // exact: q0*sp - x'
  return fmaf(-nr, y, q0);
}

// fl32(amax / 448) for amax >= 2^-100: the product with R = fl32(1/448)
// corrected once with an exact FMA residual (Markstein's correction with a
// correctly rounded reciprocal); equal to the IEEE quotient for every bf16
// amax >= 2^-100 (checked over all of them).  Smaller amax take the IEEE
// division (make_qparams).
__device__ __forceinline__ float div448(float amax) {
  constexpr float R = 0x1.24924ap-9f;  // fl32(1/448)
  const float q0 = amax * R;
  const float r = fmaf(-q0, 448.0f, amax);
  return fmaf(r, R, q0);
}

// Four fp32 -> four E4M3 codes packed little-endian into one dword, with
// the hardware conversion (round to nearest even, OCP E4M3FN on gfx950).
// Without its clamp bit the conversion returns NaN from |t| >= 464 and
// rounds (448, 464) to 448; the quantizers' quotients never exceed 448.88
// (|x| <= amax and s = fl32(amax / 448)), so no saturation step is needed:
// the E4M3 saturation at +-448 is exactly what RNE gives on that range.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Power-of-two (E8M0) scales: the exponent e of a set is the smallest
// integer >= -127 with amax <= 448 * 2^e, taken from amax's bits exactly.
// With amax = (1 + f) * 2^E (f from the fraction field) and 448 = 1.75 * 2^8,
// e = E - 8 when 1 + f <= 1.75 and E - 7 otherwise; amax below 2^-126
// (zero or subnormal) gives e <= -134, held at -127.  For finite amax
// e <= 120, so the scale byte e + 127 is never the NaN byte 0xFF.
__device__ __forceinline__ int e8m0_exponent(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int be = (int)(u >> 23);
  if (be == 0) return -127;
  const int e = be - 135 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : e;
}

// 2^-e as fp32 for e in [-127, 120] (biased exponent 127 - e in [7, 254]).
// x * e8m0_inv_scale(e) is exact for every bf16 x whose quotient is above
// fp32's normal range floor; below it the quotient's E4M3 code is a signed
// zero either way.
__device__ __forceinline__ float e8m0_inv_scale(int e) {
  return __uint_as_float((uint32_t)(127 - e) << 23);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

}  // namespace fp8blk
