// GEMM epilogues.  Each receives W consecutive output columns n..n+W-1 of
// one row m: apply8 from the bf16 MFMA kernel (with the chunk's 8 input
// values when the epilogue has an input, kLoads), apply<4> from the fp32
// kernel.  Columns come in whole groups because every N routed here is a
// multiple of 8.
#pragma once

#include "common.hpp"
#include "gemm_bf16.hpp"

namespace lgs {

// C = acc
template <typename T>
struct EpiStore {
  static constexpr bool kDirect = false, kLoads = false;
  T* C;
  int64_t ldc;
  int M, N;
  __device__ __forceinline__ bf16x8 load8(int, int) const { return bf16x8{}; }
  __device__ __forceinline__ void apply8(int m, int n, const float* v, bf16x8) const {
    apply<8>(m, n, v);
  }
  template <int W>
  __device__ __forceinline__ void apply(int m, int n, const float* v) const {
    if (m < M && n < N) store_vec<W>(C + (int64_t)m * ldc + n, v);
  }
};

// Column-parallel exit: U = acc (optional, saved for the backward pass) and
// Y = GeLU(U), the input of the row-parallel GEMM.
template <typename T>
struct EpiGeluFwd {
  static constexpr bool kDirect = false, kLoads = false;
  T* U;  // may be null
  int64_t ldu;
  T* Y;
  int64_t ldy;
  int M, N, act;
  __device__ __forceinline__ bf16x8 load8(int, int) const { return bf16x8{}; }
  __device__ __forceinline__ void apply8(int m, int n, const float* v, bf16x8) const {
    apply<8>(m, n, v);
  }
  template <int W>
  __device__ __forceinline__ void apply(int m, int n, const float* v) const {
    if (m >= M || n >= N) return;
    if (U) store_vec<W>(U + (int64_t)m * ldu + n, v);
    float y[W];
#pragma unroll
    for (int i = 0; i < W; ++i) y[i] = gelu_both(v[i], act).y;
    store_vec<W>(Y + (int64_t)m * ldy + n, y);
  }
};

// Backward through the nonlinearity: acc = dY = dZ B_i^T; reads the saved
// pre-activation U, writes dU = dY * GeLU'(U) and the recomputed Y = GeLU(U).
template <typename T>
struct EpiGeluBwd {
  static constexpr bool kDirect = false, kLoads = true;
  const T* U;
  int64_t ldu;
  T* dU;
  int64_t lddu;
  T* Y;
  int64_t ldy;
  int M, N, act;
  // bf16 path: the chunk's 8 values of U (zeros outside the matrix).
  __device__ __forceinline__ bf16x8 load8(int m, int n) const {
    if (m >= M || n >= N) return bf16x8{};
    return *reinterpret_cast<const bf16x8*>(U + (int64_t)m * ldu + n);
  }
  __device__ __forceinline__ void apply8(int m, int n, const float* dy, bf16x8 u8) const {
    float u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = (float)u8[i];
    finish<8>(m, n, dy, u);
  }
  template <int W>
  __device__ __forceinline__ void apply(int m, int n, const float* dy) const {
    if (m >= M || n >= N) return;
    float u[W];
    load_vec<W>(U + (int64_t)m * ldu + n, u);
    finish<W>(m, n, dy, u);
  }
  template <int W>
  __device__ __forceinline__ void finish(int m, int n, const float* dy, const float* u) const {
    if (m >= M || n >= N) return;
    float du[W], y[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const GeluVals g = gelu_both(u[i], act);
      du[i] = dy[i] * g.dy;
      y[i] = g.y;
    }
    store_vec<W>(dU + (int64_t)m * lddu + n, du);
    store_vec<W>(Y + (int64_t)m * ldy + n, y);
  }
};

}  // namespace lgs
