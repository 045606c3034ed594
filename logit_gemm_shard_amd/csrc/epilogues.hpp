// GEMM epilogues.  Each works on "quads": four consecutive output columns
// n..n+3 of one row m, the unit both GEMM kernels hand out.  Columns come in
// whole quads because every N the library accepts is a multiple of 8.
#pragma once

#include "common.hpp"

namespace lgs {

// C = acc
template <typename T>
struct EpiStore {
  static constexpr bool kWholeTile = false;
  T* C;
  int64_t ldc;
  int M, N;
  __device__ __forceinline__ void quad(int m, int n, f32x4 v) const {
    if (m < M && n < N) store4(C + (int64_t)m * ldc + n, v);
  }
};

// Column-parallel exit: U = acc (optional, saved for the backward pass) and
// Y = GeLU(U), the input of the row-parallel GEMM.
template <typename T>
struct EpiGeluFwd {
  static constexpr bool kWholeTile = false;
  T* U;  // may be null
  int64_t ldu;
  T* Y;
  int64_t ldy;
  int M, N, act;
  __device__ __forceinline__ void quad(int m, int n, f32x4 v) const {
    if (m >= M || n >= N) return;
    if (U) store4(U + (int64_t)m * ldu + n, v);
    f32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = gelu_f(v[i], act);
    store4(Y + (int64_t)m * ldy + n, y);
  }
};

// Backward through the nonlinearity: acc = dY = dZ B_i^T; reads the saved
// pre-activation U, writes dU = dY * GeLU'(U) and the recomputed Y = GeLU(U).
template <typename T>
struct EpiGeluBwd {
  static constexpr bool kWholeTile = false;
  const T* U;
  int64_t ldu;
  T* dU;
  int64_t lddu;
  T* Y;
  int64_t ldy;
  int M, N, act;
  __device__ __forceinline__ void quad(int m, int n, f32x4 dy) const {
    if (m >= M || n >= N) return;
    const f32x4 u = load4(U + (int64_t)m * ldu + n);
    f32x4 du, y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      du[i] = dy[i] * gelu_grad_f(u[i], act);
      y[i] = gelu_f(u[i], act);
    }
    store4(dU + (int64_t)m * lddu + n, du);
    store4(Y + (int64_t)m * ldy + n, y);
  }
};

}  // namespace lgs
