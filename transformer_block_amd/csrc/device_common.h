// Device-side helpers shared by the gfx950 kernels of libptb.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace ptb {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(u16 b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ u16 f2bf(float f) {
  return __builtin_bit_cast(u16, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}

// The same in one v_cvt_pk_bf16_f32 (both halves rounded to nearest even).
__device__ __forceinline__ uint32_t pack2bf_pk(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, b2));
}

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// D = A(32x16) * B(16x32) + C, bf16 in, fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32];
// it holds D[8*j + 4*(l/32) + i][l%32] in element 4*j + i.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// The same product with fp16 operands (v_mfma_f32_32x32x16_f16, same lane
// layout and rate).  Fragments travel as 16-bit words in bf16x8 containers.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma32x32x16_f16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// fp32 -> fp16, round to nearest even, saturated to the largest finite fp16
// (65504) so that an out-of-range value never becomes an infinity.
constexpr float kF16Max = 65504.0f;
__device__ __forceinline__ uint32_t pack2h(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  lo = __builtin_amdgcn_fmed3f(lo, -kF16Max, kF16Max);
  hi = __builtin_amdgcn_fmed3f(hi, -kF16Max, kF16Max);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, h2));
}
__device__ __forceinline__ float lo_h(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float hi_h(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8 cat8(uint4 lo, uint4 hi) {
  return (i32x8){static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
                 static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
                 static_cast<int>(hi.z), static_cast<int>(hi.w)};
}

// D = A(32x64) * B(64x32) + C with 8-bit float operands (FA, FB: 0 E4M3,
// 1 E5M2), fp32 accumulate (v_mfma_f32_32x32x64_f8f6f4, no block scales).
// Lane l supplies 32 bytes of row l%32 of A and of column l%32 of B, the same
// k-values for both; D is laid out as in mfma32x32x16.
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma32x32x64_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// The same with block scales: E8M0 codes (2^(e - 127)) in byte OS of sa and
// sb.  Lane l holds row l%32 at k [16 (l/32), +16) in bytes 0-15 and at
// k [32 + 16 (l/32), +16) in bytes 16-31, so the 32-wide block b of row i
// (k [32 b, 32 b + 32)) is bytes 16 b .. 16 b + 15 of lanes i and i + 32; its
// scale comes from lane i + 32 b.  The same for B's columns.
template <int FA, int FB, int OSA, int OSB>
__device__ __forceinline__ f32x16 mfma32x32x64_f8_mx(i32x8 a, i32x8 b, f32x16 c, uint32_t sa,
                                                     uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, OSA,
                                                         static_cast<int>(sa), OSB,
                                                         static_cast<int>(sb));
}
// The scaled MFMA with A's scale in byte i of sa and B's in byte j of sb
// (i, j < 4; both selects immediates after unrolling).
template <int FA, int FB, int I>
__device__ __forceinline__ f32x16 mx_step4_i(int j, i32x8 a, i32x8 b, f32x16 c, uint32_t sa,
                                             uint32_t sb) {
  if (j == 0) return mfma32x32x64_f8_mx<FA, FB, I, 0>(a, b, c, sa, sb);
  if (j == 1) return mfma32x32x64_f8_mx<FA, FB, I, 1>(a, b, c, sa, sb);
  if (j == 2) return mfma32x32x64_f8_mx<FA, FB, I, 2>(a, b, c, sa, sb);
  return mfma32x32x64_f8_mx<FA, FB, I, 3>(a, b, c, sa, sb);
}
template <int FA, int FB>
__device__ __forceinline__ f32x16 mx_step4(int i, int j, i32x8 a, i32x8 b, f32x16 c, uint32_t sa,
                                           uint32_t sb) {
  if (i == 0) return mx_step4_i<FA, FB, 0>(j, a, b, c, sa, sb);
  if (i == 1) return mx_step4_i<FA, FB, 1>(j, a, b, c, sa, sb);
  if (i == 2) return mx_step4_i<FA, FB, 2>(j, a, b, c, sa, sb);
  return mx_step4_i<FA, FB, 3>(j, a, b, c, sa, sb);
}

// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds of a keyed bijection of a 128-bit
// counter.  Each round takes the 64-bit products of counter words 0 and 2
// with the two round multipliers and forms
//   (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0));
// the key words advance by the two Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(M0, c.x), lo0 = M0 * c.x;
    const uint32_t hi1 = __umulhi(M1, c.z), lo1 = M1 * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    k0 += W0;
    k1 += W1;
  }
  return c;
}

// v[0..15] = the values of elements e0 .. e0 + 15 (e0 a multiple of 4) after
// dropout.
__device__ __forceinline__ void dropout16(const Dropout& d, uint32_t e0, float* v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w = philox4x32_10(make_uint4((e0 >> 2) + q, d.stream, 0u, 0u), d.k0, d.k1);
    v[4 * q + 0] = w.x >= d.t ? v[4 * q + 0] * d.scale : 0.0f;
    v[4 * q + 1] = w.y >= d.t ? v[4 * q + 1] * d.scale : 0.0f;
    v[4 * q + 2] = w.z >= d.t ? v[4 * q + 2] * d.scale : 0.0f;
    v[4 * q + 3] = w.w >= d.t ? v[4 * q + 3] * d.scale : 0.0f;
  }
}

// Largest finite value of the 8-bit formats: E4M3 448, E5M2 57344.
__device__ __forceinline__ constexpr float fp8_max(int fmt) { return fmt ? 57344.0f : 448.0f; }

// Current scaling: s = FMAX / amax (1 for an all-zero tensor); the GEMM
// undoes it with 1 / s.  One fp32 division each, the same on both sides.
__device__ __forceinline__ float fp8_scale(float amax, float fmax) {
  return amax > 0.0f ? fmax / amax : 1.0f;
}
__device__ __forceinline__ float inv_scale(float amax, float fmax) {
  return 1.0f / fp8_scale(amax, fmax);
}

// erf(x) by the rational approximation of Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (|error| <= 1.5e-7 for all x):
//   erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//   t = 1 / (1 + p x), x >= 0, and erf(-x) = -erf(x).
// erf_as_e takes e = exp(-x^2) from the caller (GeLU's derivative shares it
// with the normal density).  Inline straight-line code: a library call here
// would force every live accumulator of the GEMM epilogue to be saved around
// it.
__device__ __forceinline__ float erf_as_e(float x, float e) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  float poly = 1.061405429f;
  poly = poly * t - 1.453152027f;
  poly = poly * t + 1.421413741f;
  poly = poly * t - 0.284496736f;
  poly = poly * t + 0.254829592f;
  poly *= t;
  return copysignf(1.0f - poly * e, x);
}
__device__ __forceinline__ float erf_as(float x) { return erf_as_e(x, __expf(-x * x)); }

// Exact GeLU u * Phi(u) and its derivative Phi(u) + u * phi(u), with
// Phi(u) = (1 + erf(u / sqrt 2)) / 2 and phi(u) = exp(-u^2 / 2) / sqrt(2 pi).
__device__ __forceinline__ float gelu_f(float u) {
  return 0.5f * u * (1.0f + erf_as(u * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_grad_f(float u) {
  const float e = __expf(-0.5f * u * u);  // exp(-x^2) at x = u / sqrt 2
  const float cdf = 0.5f * (1.0f + erf_as_e(u * 0.70710678118654752f, e));
  return cdf + u * (0.39894228040143268f * e);
}

// SiLU u * sigmoid(u) and its derivative s + u s (1 - s), s = sigmoid(u)
// (SwiGLU's gate, MegaScale reading notes, section 1.3).
__device__ __forceinline__ float sigmoid_f(float u) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-u));
}
__device__ __forceinline__ float silu_f(float u) { return u * sigmoid_f(u); }
__device__ __forceinline__ float silu_grad_f(float u) {
  const float sg = sigmoid_f(u);
  return sg + u * sg * (1.0f - sg);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace ptb
