// fp32 GEMM for the fp32 workloads (small, launch-bound shapes): a plain
// LDS-tiled vector-ALU kernel.  Output tile 32x32, K tile 64, 256 threads each
// owning one row's four consecutive columns.  The next K tile's operands are
// loaded into registers while the current one is multiplied out of LDS, so
// each K tile costs about one memory latency.  Operands may be K-contiguous
// or M/N-contiguous; elements are read with scalar loads (no alignment beyond
// 4 bytes needed), consecutive threads walking the contiguous dimension.
#pragma once

#include "common.hpp"

namespace lgs {

template <bool AK, bool BK, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ B, int64_t ldb,
                                                       int M, int N, int K, Epi epi) {
  constexpr int T = 32, KS = 64, PER = T * KS / 256;  // elements of each operand per thread
  __shared__ float As[KS][T + 1];  // [k][m]
  __shared__ float Bs[KS][T + 4];  // [k][n]
  const int tid = threadIdx.x, tx = tid & 7, ty = tid >> 3;
  const int tiles_n = (N + T - 1) / T;
  const int m0 = (blockIdx.x / tiles_n) * T, n0 = (blockIdx.x % tiles_n) * T;
  float ra[PER], rb[PER];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + 256 * q;
      {
        const int k = AK ? (e % KS) : (e / T), r = AK ? (e / KS) : (e % T);
        const int gm = m0 + r, gk = k0 + k;
        ra[q] = (gm < M && gk < K) ? (AK ? A[(int64_t)gm * lda + gk] : A[(int64_t)gk * lda + gm]) : 0.f;
      }
      {
        const int k = BK ? (e % KS) : (e / T), r = BK ? (e / KS) : (e % T);
        const int gn = n0 + r, gk = k0 + k;
        rb[q] = (gn < N && gk < K) ? (BK ? B[(int64_t)gn * ldb + gk] : B[(int64_t)gk * ldb + gn]) : 0.f;
      }
    }
  };
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  fetch(0);
  for (int k0 = 0; k0 < K; k0 += KS) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + 256 * q;
      As[AK ? (e % KS) : (e / T)][AK ? (e / KS) : (e % T)] = ra[q];
      Bs[BK ? (e % KS) : (e / T)][BK ? (e / KS) : (e % T)] = rb[q];
    }
    __syncthreads();
    if (k0 + KS < K) fetch(k0 + KS);  // in flight during the multiply below
#pragma unroll 16
    for (int k = 0; k < KS; ++k) {
      const float a = As[k][ty];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(a, Bs[k][tx * 4 + j], acc[j]);
    }
    __syncthreads();
  }
  epi.template apply<4>(m0 + ty, n0 + tx * 4, acc);
}

template <bool AK, bool BK, class Epi>
inline hipError_t launch_gemm_f32(const float* A, int64_t lda, const float* B, int64_t ldb, int M,
                                  int N, int K, const Epi& epi, hipStream_t stream) {
  const int tiles = ((M + 31) / 32) * ((N + 31) / 32);
  hipLaunchKernelGGL((gemm_f32_kernel<AK, BK, Epi>), dim3(tiles), dim3(256), 0, stream, A, lda, B,
                     ldb, M, N, K, epi);
  return hipGetLastError();
}

}  // namespace lgs
