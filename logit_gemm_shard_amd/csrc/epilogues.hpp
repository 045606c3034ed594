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
  void debug_spans(int) const { LGS_NEED(C, debug::mat_bytes(M, ldc, N, sizeof(T)), "EpiStore C"); }
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
  void debug_spans(int) const {
    if (U) LGS_NEED(U, debug::mat_bytes(M, ldu, N, sizeof(T)), "EpiGeluFwd U");
    LGS_NEED(Y, debug::mat_bytes(M, ldy, N, sizeof(T)), "EpiGeluFwd Y");
  }
  __device__ __forceinline__ bf16x8 load8(int, int) const { return bf16x8{}; }
  __device__ __forceinline__ void apply8(int m, int n, const float* v, bf16x8) const {
    apply<8>(m, n, v);
  }
  template <int W>
  __device__ __forceinline__ void apply(int m, int n, const float* v) const {
    if (m >= M || n >= N) return;
    if (U) store_vec<W>(U + (int64_t)m * ldu + n, v);
    float y[W];
    gelu_vec<W>(v, y, act);
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
  void debug_spans(int) const {
    LGS_NEED(U, debug::mat_bytes(M, ldu, N, sizeof(T)), "EpiGeluBwd U");
    LGS_NEED(dU, debug::mat_bytes(M, lddu, N, sizeof(T)), "EpiGeluBwd dU");
    LGS_NEED(Y, debug::mat_bytes(M, ldy, N, sizeof(T)), "EpiGeluBwd Y");
  }
  // bf16 path: the chunk's 8 values of U (zeros outside the matrix).
  __device__ __forceinline__ bf16x8 load8(int m, int n) const {
    if (m >= M || n >= N) return bf16x8{};
    return *reinterpret_cast<const bf16x8*>(U + (int64_t)m * ldu + n);
  }
  __device__ __forceinline__ void apply8(int m, int n, const float* dy, bf16x8 u8) const {
    float u[8];
    unpack_bf16<8>(u8, u);
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
    gelu_both_vec<W>(u, y, du, act);
#pragma unroll
    for (int i = 0; i < W; ++i) du[i] *= dy[i];
    store_vec<W>(dU + (int64_t)m * lddu + n, du);
    store_vec<W>(Y + (int64_t)m * ldy + n, y);
  }
};

// ---------------------------------------------------------------- SwiGLU
//
// The mohashari.github.io page on tensor parallelism for fine-tuning 70B
// models with Megatron-LM, section "The MLP Block": rank i holds the
// column blocks W_gate,i and W_up,i side by side as one [h, 2f] matrix and
// computes Y_i = Swish(X W_gate,i) * (X W_up,i).  Pre-activations and their
// gradients use the same side-by-side layout: G at columns [0, f), U at
// [f, 2f) of one [M, 2f] matrix.

// Store of a paired product: output column n of the interleaved product
// (32-column groups alternating between the two blocks) goes to column
// (n / 64) 32 + n % 32 of the first block of C, or of the second block,
// `half` columns to the right.
template <typename T>
struct EpiPairStore {
  static constexpr bool kDirect = false, kLoads = false;
  T* C;  // may be null (nothing kept)
  int64_t ldc;
  int M, half;
  void debug_spans(int) const {
    if (C) LGS_NEED(C, debug::mat_bytes(M, ldc, 2 * (int64_t)half, sizeof(T)), "EpiPairStore [G | U]");
  }
  __device__ __forceinline__ bf16x8 load8(int, int) const { return bf16x8{}; }
  __device__ __forceinline__ void apply8(int m, int n, const float* v, bf16x8) const {
    const int col = ((n >> 6) << 5) + (n & 31);
    if (m < M && col < half) store_vec<8>(C + (int64_t)m * ldc + col + ((n >> 5) & 1) * half, v);
  }
};

// Column-parallel exit of the gated block: the GEMM X [W_gate,i | W_up,i]
// runs as a paired product, so each wave holds G (tiles 2q) and U (tiles
// 2q+1) of the same columns and forms Y = Swish(G) * U in registers.  G and U
// are kept for the backward pass when pairs.C is set.
struct EpiSwigluFwd {
  static constexpr bool kDirect = false, kLoads = false, kPaired = true;
  EpiPairStore<bf16> pairs;
  EpiStore<bf16> out;
  int half;
  void debug_spans(int bn) const {
    pairs.debug_spans(bn);
    out.debug_spans(bn);
  }
  __device__ __forceinline__ bool keeps_pairs() const { return pairs.C != nullptr; }
  template <int TM, int TN>
  __device__ __forceinline__ void combine(const f32x16 (&acc)[TM][TN], f32x16 (&y)[TM][TN / 2]) const {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < TN / 2; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) y[i][q][r] = swish_both(acc[i][2 * q][r]).y * acc[i][2 * q + 1][r];
  }
};

// Backward through the gate: acc = dY = dZ W_down,i^T; reads the saved G and
// U, writes dG = dY * U * Swish'(G) and dU = dY * Swish(G) side by side, and
// the recomputed Y = Swish(G) * U.
struct GateUp8 {
  bf16x8 g, u;
};

struct EpiSwigluBwd {
  static constexpr bool kDirect = false, kLoads = true;
  static constexpr int kMaxRows = 16;  // two prefetched input chunks per output chunk
  const bf16* GU;  // G at [m, n], U at [m, half + n]
  int64_t ldgu;
  bf16* dGU;       // dG at [m, n], dU at [m, half + n]
  int64_t lddgu;
  bf16* Y;
  int64_t ldy;
  int M, half;
  void debug_spans(int) const {
    LGS_NEED(GU, debug::mat_bytes(M, ldgu, 2 * (int64_t)half, 2), "EpiSwigluBwd [G | U]");
    LGS_NEED(dGU, debug::mat_bytes(M, lddgu, 2 * (int64_t)half, 2), "EpiSwigluBwd [dG | dU]");
    LGS_NEED(Y, debug::mat_bytes(M, ldy, half, 2), "EpiSwigluBwd Y");
  }
  __device__ __forceinline__ GateUp8 load8(int m, int n) const {
    if (m >= M || n >= half) return GateUp8{};
    const bf16* p = GU + (int64_t)m * ldgu + n;
    return {*reinterpret_cast<const bf16x8*>(p), *reinterpret_cast<const bf16x8*>(p + half)};
  }
  __device__ __forceinline__ void apply8(int m, int n, const float* dy, GateUp8 in) const {
    if (m >= M || n >= half) return;
    float dg[8], du[8], y[8], gv[8], uv[8];
    unpack_bf16<8>(in.g, gv);
    unpack_bf16<8>(in.u, uv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float g = gv[i], u = uv[i];
      const SwishVals sw = swish_both(g);
      dg[i] = dy[i] * u * sw.dy;
      du[i] = dy[i] * sw.y;
      y[i] = sw.y * u;
    }
    bf16* q = dGU + (int64_t)m * lddgu + n;
    store_vec<8>(q, dg);
    store_vec<8>(q + half, du);
    store_vec<8>(Y + (int64_t)m * ldy + n, y);
  }
};

}  // namespace lgs
