// Shared device helpers for the gfx950 (CDNA4) kernels: types, bf16
// packing and the GeLU / GeLU' forms used by the GEMM epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lgs {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Act : int { ACT_ERF = 0, ACT_TANH = 1 };

// GeLU(u) = u * Phi(u), Phi the standard normal CDF; the nonlinearity the
// pages put between the column-parallel and the row-parallel GEMM ("Cutting
// a Model Into Pieces", "Megatron-LM: cutting inside the layer").
// ACT_TANH is the published tanh approximation of the same function.
// erff / tanhf / __expf are ROCm's device math library functions.
__device__ __forceinline__ float gelu_f(float u, int act) {
  if (act == ACT_ERF) return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f));
  const float a = 0.79788456080286536f * (u + 0.044715f * u * u * u);
  return 0.5f * u * (1.0f + tanhf(a));
}

// d GeLU / du.  Exact form: Phi(u) + u * phi(u), phi(u) = exp(-u^2/2)/sqrt(2 pi).
__device__ __forceinline__ float gelu_grad_f(float u, int act) {
  if (act == ACT_ERF)
    return 0.5f * (1.0f + erff(u * 0.70710678118654752f)) +
           u * __expf(-0.5f * u * u) * 0.39894228040143268f;
  const float a = 0.79788456080286536f * (u + 0.044715f * u * u * u);
  const float s = tanhf(a);
  return 0.5f * (1.0f + s) +
         0.5f * u * (1.0f - s * s) * 0.79788456080286536f * (1.0f + 0.134145f * u * u);
}

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

// Store four consecutive values (round-to-nearest-even for bf16).
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
  bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *reinterpret_cast<bf16x4*>(p) = o;
}
__device__ __forceinline__ void store4(float* p, f32x4 v) {
  p[0] = v[0]; p[1] = v[1]; p[2] = v[2]; p[3] = v[3];
}
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
__device__ __forceinline__ f32x4 load4(const float* p) {
  return f32x4{p[0], p[1], p[2], p[3]};
}

}  // namespace lgs
