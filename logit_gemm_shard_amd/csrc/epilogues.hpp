// GEMM epilogues.  Each receives W consecutive output columns n..n+W-1 of
// one row m (W = 8 from the bf16 MFMA kernel, 4 from the fp32 kernel).
// Columns come in whole groups because every N routed here is a multiple
// of 8.
#pragma once

#include "common.hpp"
#include "gemm_bf16.hpp"

namespace lgs {

// C = acc
template <typename T>
struct EpiStore {
  static constexpr bool kDirect = false;
  T* C;
  int64_t ldc;
  int M, N;
  template <int WN, int LD>
  __device__ __forceinline__ void slice(const float* st, int m0, int nb, int lane) const {
    elementwise_slice<WN, LD>(*this, st, m0, nb, lane);
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
  static constexpr bool kDirect = false;
  T* U;  // may be null
  int64_t ldu;
  T* Y;
  int64_t ldy;
  int M, N, act;
  template <int WN, int LD>
  __device__ __forceinline__ void slice(const float* st, int m0, int nb, int lane) const {
    elementwise_slice<WN, LD>(*this, st, m0, nb, lane);
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
  static constexpr bool kDirect = false;
  const T* U;
  int64_t ldu;
  T* dU;
  int64_t lddu;
  T* Y;
  int64_t ldy;
  int M, N, act;
  template <int WN, int LD>
  __device__ __forceinline__ void slice(const float* st, int m0, int nb, int lane) const {
    elementwise_slice<WN, LD>(*this, st, m0, nb, lane);
  }
  template <int W>
  __device__ __forceinline__ void apply(int m, int n, const float* dy) const {
    if (m >= M || n >= N) return;
    float u[W], du[W], y[W];
    load_vec<W>(U + (int64_t)m * ldu + n, u);
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
