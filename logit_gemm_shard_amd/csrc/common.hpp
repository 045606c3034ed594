// Shared device helpers for the gfx950 (CDNA4) kernels: types, vector
// loads / stores, and the GeLU / GeLU' and Swish / Swish' forms used by the
// GEMM epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lgs {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Act : int { ACT_ERF = 0, ACT_TANH = 1 };

// GeLU(u) = u * Phi(u), Phi the standard normal CDF: the nonlinearity the
// pages put between the column-parallel and the row-parallel GEMM ("Cutting
// a Model Into Pieces", "Megatron-LM: cutting inside the layer").  ACT_TANH
// is the published tanh approximation of the same function.
//
// Phi comes from erf by Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26: for z >= 0, with t = 1 / (1 + p z),
//   erf(z) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2) + e(z),
//   |e(z)| <= 1.5e-7,
// which is branch-free (one exp, one reciprocal) and shares exp(-u^2/2) with
// the density phi(u) needed by GeLU'.  Both values come out of one call.
struct GeluVals {
  float y;   // GeLU(u)
  float dy;  // GeLU'(u)
};

__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);  // v_exp_f32 computes 2^x
}

__device__ __forceinline__ GeluVals gelu_both(float u, int act) {
  if (act == ACT_ERF) {
    const float z = fabsf(u) * 0.70710678118654752f;  // |u| / sqrt(2)
    const float e = fast_exp(-z * z);                  // exp(-u^2/2)
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
    float p = fmaf(t, 1.061405429f, -1.453152027f);
    p = fmaf(t, p, 1.421413741f);
    p = fmaf(t, p, -0.284496736f);
    p = fmaf(t, p, 0.254829592f);
    const float tail = 0.5f * (p * t) * e;             // 1 - Phi(|u|)
    const float phi = u >= 0.f ? 1.0f - tail : tail;   // Phi(u)
    return {u * phi, fmaf(u * 0.39894228040143268f, e, phi)};
  }
  // tanh(a) = 1 - 2 / (1 + exp(2a)), finite at both ends (exp -> 0 or inf)
  const float a = 0.79788456080286536f * fmaf(0.044715f * u, u * u, u);
  const float th = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + fast_exp(2.0f * a));
  const float da = 0.79788456080286536f * fmaf(0.134145f * u, u, 1.0f);
  return {0.5f * u * (1.0f + th), fmaf(0.5f * u * (1.0f - th * th), da, 0.5f * (1.0f + th))};
}

// Swish(g) = g * sigmoid(g), the gate nonlinearity of the SwiGLU MLP block
// (the mohashari.github.io page on tensor parallelism for 70B models,
// section "The MLP Block"), and its slope
// sigmoid(g) (1 + g (1 - sigmoid(g))).  sigmoid = 1 / (1 + exp(-g)) stays
// finite at both ends: exp(-g) overflows to inf for g << 0 (sigmoid -> 0)
// and underflows to 0 for g >> 0 (sigmoid -> 1).
__device__ __forceinline__ float sigmoid_fast(float g) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp(-g));
}

struct SwishVals {
  float y;   // Swish(g)
  float dy;  // Swish'(g)
};

__device__ __forceinline__ SwishVals swish_both(float g) {
  const float sg = sigmoid_fast(g);
  return {g * sg, sg * fmaf(g, 1.0f - sg, 1.0f)};
}

// W consecutive values at p (W = 4 or 8); bf16 uses one vector access,
// fp32 scalar accesses (the fp32 path only guarantees 4-byte alignment).
template <int W>
__device__ __forceinline__ void store_vec(bf16* p, const float* v) {
  if constexpr (W == 8) {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
    *reinterpret_cast<bf16x8*>(p) = o;
  } else {
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (bf16)v[i];
    *reinterpret_cast<bf16x4*>(p) = o;
  }
}
template <int W>
__device__ __forceinline__ void store_vec(float* p, const float* v) {
#pragma unroll
  for (int i = 0; i < W; ++i) p[i] = v[i];
}
template <int W>
__device__ __forceinline__ void load_vec(const bf16* p, float* v) {
  if constexpr (W == 8) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)x[i];
  } else {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (float)x[i];
  }
}
template <int W>
__device__ __forceinline__ void load_vec(const float* p, float* v) {
#pragma unroll
  for (int i = 0; i < W; ++i) v[i] = p[i];
}

}  // namespace lgs
