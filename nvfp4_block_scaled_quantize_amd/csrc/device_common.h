// device_common.h -- gfx950 device helpers shared by the NVFP4 kernels.
//
// Numerics: every function here performs binary32 operations with one
// rounding each (the library is compiled with -ffp-contract=off and denormals
// kept); fma appears only where written.  The hardware conversions used were
// checked on gfx950 for their rounding:
//   v_cvt_pk_fp8_f32          : OCP E4M3FN, round-half-even, no saturation
//                               (so the input is clamped to 448 first)
//   v_cvt_f32_fp8             : exact E4M3FN decode
//   v_cvt_scalef32_pk_fp4_f32 : E2M1 round-half-even, saturating at 6, sign
//                               kept; the scale operand contributes only its
//                               exponent, so it is always passed 1.0 here
//   v_cvt_scalef32_pk_f16_fp4 : exact E2M1 -> f16 times 2^exponent(scale)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- inputs
// bf16 is the upper half of a binary32; fp16 converts exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float fp16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float fp16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

template <int DT>
__device__ __forceinline__ void unpack2(uint32_t w, float& a, float& b) {
  if constexpr (DT == 0) { a = bf16_lo(w); b = bf16_hi(w); }
  else { a = fp16_lo(w); b = fp16_hi(w); }
}
template <int DT>
__device__ __forceinline__ float unpack1(uint16_t h) {
  if constexpr (DT == 0) return __uint_as_float((uint32_t)h << 16);
  else return (float)__builtin_bit_cast(_Float16, h);
}

// ---------------------------------------------------------------- exp
// exp(x) as a fixed binary32 evaluation (Cody-Waite reduction with ln 2 split
// into two binary32 parts, degree-7 Taylor polynomial by Horner with fma,
// exact scaling by 2^n).  Constants: binary32 roundings of log2(e), ln 2,
// ln 2 minus its binary32 rounding, and 1/k! for k = 0..7.
__device__ __forceinline__ float exp_f32(float x) {
  const float kL2E = __uint_as_float(0x3FB8AA3Bu);
  const float kLn2Hi = __uint_as_float(0x3F317218u);
  const float kLn2Lo = __uint_as_float(0xB102E308u);
  const float kC2 = __uint_as_float(0x3F000000u);   // 1/2
  const float kC3 = __uint_as_float(0x3E2AAAABu);   // 1/6
  const float kC4 = __uint_as_float(0x3D2AAAABu);   // 1/24
  const float kC5 = __uint_as_float(0x3C088889u);   // 1/120
  const float kC6 = __uint_as_float(0x3AB60B61u);   // 1/720
  const float kC7 = __uint_as_float(0x39500D01u);   // 1/5040
  if (x > 88.75f) return __builtin_inff();
  if (x < -87.0f) return 0.0f;
  float n = __builtin_rintf(x * kL2E);
  float r = __builtin_fmaf(-n, kLn2Hi, x);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float p = kC7;
  p = __builtin_fmaf(p, r, kC6);
  p = __builtin_fmaf(p, r, kC5);
  p = __builtin_fmaf(p, r, kC4);
  p = __builtin_fmaf(p, r, kC3);
  p = __builtin_fmaf(p, r, kC2);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, (int)n);
}

// silu(g) = g / (1 + exp(-g)) with an exactly rounded division.
__device__ __forceinline__ float silu_f32(float g) {
  float e = exp_f32(-g);
  float s = 1.0f + e;
  return g / s;
}

// SwiGLU output silu(g) * u.
__device__ __forceinline__ float swiglu_f32(float g, float u) { return silu_f32(g) * u; }

__device__ __forceinline__ float relu2_f32(float x) {
  float r = (x > 0.0f) ? x : 0.0f;
  return r * r;
}

__device__ __forceinline__ float sigmoid_f32(float l) {
  float e = exp_f32(-l);
  float d = 1.0f + e;
  return 1.0f / d;
}

// x / 6 correctly rounded.  The product with RN(1/6) is within one ulp of the
// quotient, and one fma correction step (Markstein) then rounds correctly; this
// equals the exact quotient for every x in [2^-125, FLT_MAX] (checked for all
// binary32 values by a host test).  Smaller x (subnormal quotients) and
// non-finite x divide.
__device__ __forceinline__ float div6_f32(float x) {
  const float r = __uint_as_float(0x3E2AAAABu);   // RN(1/6)
  float q = x * r;
  const float e = __builtin_fmaf(-q, 6.0f, x);
  q = __builtin_fmaf(e, r, q);
  if (!(x >= 0x1p-125f && x <= 3.40282346638528859812e+38f)) {
    asm volatile("");   // keeps this rare path a branch (not evaluated for every lane)
    q = x / 6.0f;
  }
  return q;
}

// ---------------------------------------------------------------- scales
// Global scale pair of a group from its amax.
__device__ __forceinline__ void global_scales(float amax, float& g_enc, float& g_dec) {
  float ge = 2688.0f / amax;
  if (!__builtin_isfinite(ge)) ge = 3.40282346638528859812e+38f;
  g_enc = ge;
  g_dec = 1.0f / ge;
}

// E4M3 block scale byte from a block amax; returns the byte and the combined
// scale c and its encode factor.
__device__ __forceinline__ uint32_t block_scale(float amax_b, float g_enc, float g_dec, float& c,
                                                float& enc) {
  float sf_f = div6_f32(amax_b) * g_enc;
  float sat = __builtin_fminf(sf_f, 448.0f);
  uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat, 0.0f, 0, false);
  float sfd = __builtin_amdgcn_cvt_f32_fp8((int)pk, 0);
  c = sfd * g_dec;
  enc = (c == 0.0f) ? 0.0f : 1.0f / c;
  return pk & 0xFFu;
}

// Eight values -> eight E2M1 codes in one dword (element 0 in bits 3..0).
// A zero element always gets a zero code with its own sign; this needs care
// only when enc overflowed to +inf (combined scale below 2^-128), where the
// product 0 * inf is NaN -- that rare block is encoded directly: non-zero
// elements saturate to magnitude code 7.
__device__ __forceinline__ uint32_t pack8_e2m1(const float* v, float enc) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0] * enc, v[1] * enc, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2] * enc, v[3] * enc, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4] * enc, v[5] * enc, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6] * enc, v[7] * enc, 1.0f, 3);
  if (enc == __builtin_inff()) {
    w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = __float_as_uint(v[i]);
      const uint32_t code = ((b >> 31) << 3) | ((b << 1) != 0u ? 7u : 0u);
      w |= code << (4 * i);
    }
  }
  return w;
}

// ---------------------------------------------------------------- barriers
// Workgroup barrier that waits only for this wave's LDS operations.
// __syncthreads() also waits for every outstanding global load (vmcnt(0)),
// which would drain the loads a streaming kernel keeps in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Lane exchange inside rows of 16 lanes through DPP (no LDS round trip).
// CTRL: 0xB1 = quad_perm [1,0,3,2] (lane ^ 1), 0x4E = quad_perm [2,3,0,1]
// (lane ^ 2), 0x141 = row_half_mirror, 0x140 = row_mirror.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over each row of 16 lanes; every lane of the row receives it.
__device__ __forceinline__ float row16_max(float v) {
  v = __builtin_fmaxf(v, dpp_f32<0xB1>(v));
  v = __builtin_fmaxf(v, dpp_f32<0x4E>(v));
  v = __builtin_fmaxf(v, dpp_f32<0x141>(v));
  return __builtin_fmaxf(v, dpp_f32<0x140>(v));
}

// Max over the 64 lanes of a wave, returned as a wave-uniform value.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = row16_max(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return __builtin_fmaxf(__builtin_fmaxf(r0, r1), __builtin_fmaxf(r2, r3));
}

}  // namespace nvfp4
