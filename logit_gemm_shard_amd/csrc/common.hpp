// Shared device helpers for the gfx950 (CDNA4) kernels: types, vector
// loads / stores, and the GeLU / GeLU' and Swish / Swish' forms used by the
// GEMM epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "debug.hpp"

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
// the density phi(u) needed by GeLU'.
//
// The epilogues evaluate it per element on the vector ALU, at 4 cycles per
// 64-lane instruction, so the forms below are arranged for few instructions:
// z = |u| / sqrt(2) is folded into p, the factor 1/2 of Phi = (1 + erf) / 2
// into the a_k (halving is exact in binary, so the tail is unchanged), and
// GeLU(u) = max(u, 0) - |u| (1 - Phi(|u|)) needs no select.  A non-finite u
// gives a non-finite result.
struct GeluVals {
  float y;   // GeLU(u)
  float dy;  // GeLU'(u)
};

__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);  // v_exp_f32 computes 2^x
}

// 1 - Phi(|u|) and exp(-u^2 / 2).
struct PhiTail {
  float tail, e;
};
__device__ __forceinline__ PhiTail phi_tail(float u) {
  const float t = __builtin_amdgcn_rcpf(fmaf(fabsf(u), 0.23164188826636040f, 1.0f));  // p / sqrt(2)
  const float e = __builtin_amdgcn_exp2f(u * u * -0.72134752044448170f);  // 2^(-u^2 log2(e) / 2)
  float q = fmaf(t, 0.5307027145f, -0.7265760135f);  // a5 / 2, a4 / 2
  q = fmaf(t, q, 0.7107068705f);
  q = fmaf(t, q, -0.142248368f);
  q = fmaf(t, q, 0.127414796f);
  return {(q * t) * e, e};
}

// tanh form: with a = sqrt(2/pi) (u + 0.044715 u^3) and r = 1 / (1 + exp(2a)),
// (1 + tanh a) / 2 = 1 - r, so GeLU(u) = u (1 - r) and
// GeLU'(u) = (1 - r) (1 + 2 u r a'(u)), a'(u) = sqrt(2/pi) (1 + 0.134145 u^2).
// exp(2a) overflows to inf for u >> 0 (r = 0) and underflows to 0 for u << 0 (r = 1).
__device__ __forceinline__ float tanh_exp2a(float u, float uu) {
  return __builtin_amdgcn_exp2f(u * fmaf(uu, 0.10294323958002350f, 2.3022081981443250f));  // 2 a log2(e)
}
__device__ __forceinline__ float tanh_r(float u, float uu) {
  return __builtin_amdgcn_rcpf(1.0f + tanh_exp2a(u, uu));
}

// max(u, 0) as one integer max on the bit pattern (negative floats, -0
// included, are negative integers); fmaxf would first quiet u in IEEE mode,
// one more instruction.
__device__ __forceinline__ float pos_part(float u) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, u), 0));
}

__device__ __forceinline__ float gelu_erf(float u) {
  return fmaf(-fabsf(u), phi_tail(u).tail, pos_part(u));
}

__device__ __forceinline__ GeluVals gelu_erf_both(float u) {
  const PhiTail q = phi_tail(u);
  const float phi = u >= 0.f ? 1.0f - q.tail : q.tail;  // Phi(u)
  return {fmaf(-fabsf(u), q.tail, pos_part(u)), fmaf(u * 0.39894228040143270f, q.e, phi)};
}

__device__ __forceinline__ float gelu_tanh(float u) {
  return fmaf(-u, tanh_r(u, u * u), u);
}

// For u < 0, 1 - r = exp(2a) r avoids the cancellation of 1 - r with r near
// 1, which GeLU' multiplies by |2 u a'(u)| (about 30 at u = -5).
__device__ __forceinline__ GeluVals gelu_tanh_both(float u) {
  const float uu = u * u;
  const float e2a = tanh_exp2a(u, uu);
  const float r = __builtin_amdgcn_rcpf(1.0f + e2a);
  const float omr = u >= 0.f ? 1.0f - r : e2a * r;
  const float da2 = fmaf(uu, 0.21406444881780073f, 1.5957691216057308f);  // 2 a'(u)
  return {u * omr, omr * fmaf(u * r, da2, 1.0f)};
}

// Elementwise over W values; the form is chosen once per call (act is
// uniform), so the W evaluations interleave.
template <int W>
__device__ __forceinline__ void gelu_vec(const float* u, float* y, int act) {
  if (act == ACT_ERF) {
#pragma unroll
    for (int i = 0; i < W; ++i) y[i] = gelu_erf(u[i]);
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) y[i] = gelu_tanh(u[i]);
  }
}

template <int W>
__device__ __forceinline__ void gelu_both_vec(const float* u, float* y, float* dy, int act) {
  if (act == ACT_ERF) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const GeluVals g = gelu_erf_both(u[i]);
      y[i] = g.y;
      dy[i] = g.dy;
    }
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const GeluVals g = gelu_tanh_both(u[i]);
      y[i] = g.y;
      dy[i] = g.dy;
    }
  }
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
// bf16 -> fp32 of W packed values: a bf16 is the high half of its fp32, so
// the even element of each 32-bit pair is one shift and the odd one one mask
// (the generic conversion spends two shifts on the odd one).
template <int W, class V>
__device__ __forceinline__ void unpack_bf16(const V& x, float* v) {
  static_assert(sizeof(V) == 2 * W && W % 2 == 0, "packed bf16 vector");
  uint32_t w[W / 2];
  __builtin_memcpy(w, &x, sizeof(w));
#pragma unroll
  for (int i = 0; i < W / 2; ++i) {
    v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}
template <int W>
__device__ __forceinline__ void load_vec(const bf16* p, float* v) {
  if constexpr (W == 8)
    unpack_bf16<8>(*reinterpret_cast<const bf16x8*>(p), v);
  else
    unpack_bf16<4>(*reinterpret_cast<const bf16x4*>(p), v);
}
template <int W>
__device__ __forceinline__ void load_vec(const float* p, float* v) {
#pragma unroll
  for (int i = 0; i < W; ++i) v[i] = p[i];
}

}  // namespace lgs
