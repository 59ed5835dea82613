// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWaves = 4;          // waves of a 256-thread workgroup
constexpr int kBlockTokens = 64;   // tokens per permutation wave (one lane per token)
constexpr int kGroupTokens = 16;   // tokens per routing group (one histogram / probability-sum row)
constexpr int kMaxE = 64;
constexpr int kMaxK = 8;

__device__ __forceinline__ float bf16_to_f32(u16 b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<u16>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<u16>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): words 0-2 of the block for counter
// (c0, c1, 0, 0) and key (k0, k1).
__device__ __forceinline__ void philox_words012(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1, uint32_t& w0,
                                                uint32_t& w1, uint32_t& w2) {
  uint32_t x0 = c0, x1 = c1, x2 = 0u, x3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, x0), lo0 = 0xD2511F53u * x0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, x2), lo1 = 0xCD9E8D57u * x2;
    const uint32_t n0 = hi1 ^ x1 ^ k0;
    const uint32_t n2 = hi0 ^ x3 ^ k1;
    x0 = n0;
    x1 = lo1;
    x2 = n2;
    x3 = lo0;
  }
  w0 = x0;
  w1 = x1;
  w2 = x2;
}

__device__ __forceinline__ void philox_words01(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1, uint32_t& w0,
                                               uint32_t& w1) {
  uint32_t w2;
  philox_words012(c0, c1, k0, k1, w0, w1, w2);
}

__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1) {
  uint32_t w0, w1;
  philox_words01(c0, c1, k0, k1, w0, w1);
  return w0;
}

// Priority of slot (token t, expert e) for random capacity dropping: word 2 of the block above.
__device__ __forceinline__ uint32_t drop_priority(uint32_t t, uint32_t e, uint32_t k0, uint32_t k1) {
  uint32_t w0, w1, w2;
  philox_words012(t, e, k0, k1, w0, w1, w2);
  return w2;
}

// Gumbel(0,1) noise for (token t, expert e): u = (w0 + 1/2) 2^-32 in float64, strictly inside
// (0,1); g = -log(-log u) in float64, rounded once to float32.
__device__ __forceinline__ float gumbel_noise(uint32_t t, uint32_t e, uint32_t k0, uint32_t k1) {
  const uint32_t w0 = philox_word0(t, e, k0, k1);
  const double u = (static_cast<double>(w0) + 0.5) * 0x1p-32;
  return static_cast<float>(-log(-log(u)));
}

// Gaussian noise std * n for (token t, expert e): u1, u2 from words 0 and 1 as above,
// n = sqrt(-2 ln u1) cos(2 pi u2) (Box-Muller) in float64, rounded once to float32.
__device__ __forceinline__ float gaussian_noise(uint32_t t, uint32_t e, uint32_t k0, uint32_t k1, float std) {
  uint32_t w0, w1;
  philox_words01(t, e, k0, k1, w0, w1);
  const double u1 = (static_cast<double>(w0) + 0.5) * 0x1p-32;
  const double u2 = (static_cast<double>(w1) + 0.5) * 0x1p-32;
  const double n = sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925287 * u2);
  return static_cast<float>(static_cast<double>(std) * n);
}

// SiLU(v) = v sigmoid(v) = v / (1 + e^-v), float32 with the library exponential.
__device__ __forceinline__ float silu_exact(float v) { return v / (1.0f + expf(-v)); }

// SiLU for results rounded to bf16: v * rcp(1 + 2^(-v log2 e)) with the hardware exp2 and
// reciprocal (a few float32 ulps). SiLU(+inf) = +inf; a -inf input gives NaN.
__device__ __forceinline__ float silu_bf16_path(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
}

__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752440f));
}

// GeLU(v) = v Phi(v) with the normal tail h = Phi(-|v|) = (1 - erf(|v| / sqrt 2)) / 2 from
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26: for x >= 0,
// 1 - erf(x) = t (a1 + a2 t + ... + a5 t^4) e^(-x^2), t = 1 / (1 + p x), |error| <= 1.5e-7.
// Here x = |v| / sqrt 2, the coefficients are halved and e^(-x^2) = 2^(-v^2 / (2 ln 2)); then
// GeLU(v) = max(v, 0) - |v| h for both signs (no cancellation for v < 0). The error is at most
// 0.75e-7 |v| plus float32 rounding (3.3e-7 absolute over [-12, 12]), and the relative error
// stays below half a bf16 step (2^-9) for v >= -5; used only where the result is rounded to
// bf16. |v| is capped at FLT_MAX in the last product so that GeLU(+inf) = +inf.
__device__ __forceinline__ float gelu_bf16_path(float v) {
  const float a = fabsf(v);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164189f, a, 1.0f));     // p / sqrt 2
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 0.5307027f, -0.72657603f), 0.7107069f), -0.14224836f), 0.1274148f);
  const float h = poly * __builtin_amdgcn_exp2f((v * v) * -0.7213475f);   // -1 / (2 ln 2)
  return fmaf(-fminf(a, 3.4028235e38f), h, fmaxf(v, 0.0f));
}

// Derivatives for the backward pass, float32 with the library erf and exponential:
// GeLU'(v) = Phi(v) + v phi(v), phi(v) = e^(-v^2 / 2) / sqrt(2 pi); SiLU'(v) = s (1 + v (1 - s)),
// s = sigmoid(v).
__device__ __forceinline__ float gelu_grad_exact(float v) {
  return 0.5f * (1.0f + erff(v * 0.70710678118654752440f)) + v * 0.39894228040143267794f * expf(-0.5f * v * v);
}

__device__ __forceinline__ float silu_grad_exact(float v) {
  const float s = 1.0f / (1.0f + expf(-v));
  return s * (1.0f + v * (1.0f - s));
}

// The same derivatives for results rounded to bf16, from the hardware exp2 and reciprocal.
// GeLU': Phi(v) from the tail h = Phi(-|v|) of gelu_bf16_path (A&S 7.1.26, |error| <= 0.75e-7)
// and phi(v) = e^(-v^2/2) / sqrt(2 pi) from the same exponential; the v phi(v) term uses |v|
// capped at 1e30 so that infinite inputs give 0 or 1. SiLU': s (1 + v (1 - s)) with
// s = rcp(1 + 2^(-v log2 e)), v clamped to [-1e4, 1e4] (beyond it the value is 0 or 1).
__device__ __forceinline__ float gelu_grad_bf16_path(float v) {
  const float a = fabsf(v);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164189f, a, 1.0f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 0.5307027f, -0.72657603f), 0.7107069f), -0.14224836f), 0.1274148f);
  const float g = __builtin_amdgcn_exp2f((v * v) * -0.7213475f);        // e^(-v^2 / 2)
  const float h = poly * g;
  const float phi_big = v >= 0.0f ? 1.0f - h : h;
  return fmaf(copysignf(fminf(a, 1e30f), v) * 0.39894228040143267794f, g, phi_big);
}

__device__ __forceinline__ float silu_grad_bf16_path(float v) {
  const float vc = fminf(fmaxf(v, -1e4f), 1e4f);
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(vc * -1.4426950408889634f));
  return s * fmaf(vc, 1.0f - s, 1.0f);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace moe
