// fp32 GEMM for the fp32 workloads (small, launch-bound shapes): a plain
// LDS-tiled vector-ALU kernel, 64x64 output tile, K step 16, 256 threads each
// owning a 4x4 block (four quads of four consecutive columns).  Operands may
// be K-contiguous or M/N-contiguous; every element is read once per tile with
// scalar loads, so no alignment beyond 4 bytes is required.  Each thread
// hands its rows to the epilogue four columns at a time.
#pragma once

#include "common.hpp"

namespace lgs {

template <bool AK, bool BK, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ B, int64_t ldb,
                                                       int M, int N, int K, Epi epi) {
  constexpr int T = 64, KS = 16;
  __shared__ float As[KS][T + 4];  // [k][m]
  __shared__ float Bs[KS][T + 4];  // [k][n]
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tiles_n = (N + T - 1) / T;
  const int m0 = (blockIdx.x / tiles_n) * T, n0 = (blockIdx.x % tiles_n) * T;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += KS) {
#pragma unroll
    for (int e = tid; e < T * KS; e += 256) {
      // K-contiguous: consecutive threads walk k; otherwise they walk m / n
      const int k = AK ? (e % KS) : (e / T), r = AK ? (e / KS) : (e % T);
      const int gm = m0 + r, gk = k0 + k;
      As[k][r] = (gm < M && gk < K) ? (AK ? A[(int64_t)gm * lda + gk] : A[(int64_t)gk * lda + gm]) : 0.f;
    }
#pragma unroll
    for (int e = tid; e < T * KS; e += 256) {
      const int k = BK ? (e % KS) : (e / T), r = BK ? (e / KS) : (e % T);
      const int gn = n0 + r, gk = k0 + k;
      Bs[k][r] = (gn < N && gk < K) ? (BK ? B[(int64_t)gn * ldb + gk] : B[(int64_t)gk * ldb + gn]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) epi.template apply<4>(m0 + ty * 4 + i, n0 + tx * 4, acc[i]);
}

template <bool AK, bool BK, class Epi>
inline hipError_t launch_gemm_f32(const float* A, int64_t lda, const float* B, int64_t ldb, int M,
                                  int N, int K, const Epi& epi, hipStream_t stream) {
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  hipLaunchKernelGGL((gemm_f32_kernel<AK, BK, Epi>), dim3(tiles), dim3(256), 0, stream, A, lda, B,
                     ldb, M, N, K, epi);
  return hipGetLastError();
}

}  // namespace lgs
