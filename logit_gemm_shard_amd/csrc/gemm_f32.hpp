// fp32 GEMM for the fp32 workloads (small, launch-bound shapes): a plain
// LDS-tiled vector-ALU kernel.  Output tile 32 x 32, K tile 64, 256 threads
// each owning one row's four consecutive columns.  The next K tile's operands
// are loaded into registers while the current one is multiplied out of LDS,
// so each K tile costs about one memory latency.  Operands may be
// K-contiguous or M/N-contiguous; elements are read with scalar loads (no
// alignment beyond 4 bytes needed), consecutive threads walking the
// contiguous dimension.
//
// A thread's serial work is 4 K FMAs, so a problem with few output tiles is
// bound by that chain, not by the chip.  Those problems use the split form
// below: 16 x 16 tiles whose K range is divided among the block's waves
// (each with its own LDS tiles), the waves' partial sums added in LDS in
// wave order at the end.
#pragma once

#include "common.hpp"

namespace lgs {

template <bool AK, bool BK, class Epi, int T>  // T = 32 (T * T / 4 threads)
__global__ __launch_bounds__(T * T / 4) void gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                             const float* __restrict__ B, int64_t ldb,
                                                             int M, int N, int K, Epi epi) {
  constexpr int NT = T * T / 4, KS = 64, PER = T * KS / NT;  // threads; elements of each operand per thread
  constexpr int CG = T / 4;                                   // four-column groups per row
  __shared__ float As[KS][T + 1];  // [k][m]
  __shared__ float Bs[KS][T + 4];  // [k][n]
  const int tid = threadIdx.x, tx = tid % CG, ty = tid / CG;
  const int tiles_n = (N + T - 1) / T;
  const int m0 = (blockIdx.x / tiles_n) * T, n0 = (blockIdx.x % tiles_n) * T;
  float ra[PER], rb[PER];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + NT * q;
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
      const int e = tid + NT * q;
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

// Split form: block = kWaves waves on one 16 x 16 output tile; wave w takes
// K tiles w, w + kWaves, ... (every wave runs the same number of steps; tiles
// past K load zeros).  Thread (w, l) owns row l / 4, columns 4 (l % 4) .. +3
// of wave w's partial.
constexpr int kSplitWaves = 8;
template <bool AK, bool BK, class Epi>
__global__ __launch_bounds__(64 * kSplitWaves) void gemm_f32_split_kernel(const float* __restrict__ A,
                                                                          int64_t lda,
                                                                          const float* __restrict__ B,
                                                                          int64_t ldb, int M, int N, int K,
                                                                          Epi epi) {
  constexpr int T = 16, KS = 64, PER = T * KS / 64;  // elements of each operand per lane per K tile
  __shared__ float As[kSplitWaves][KS][T + 1];  // [wave][k][m]
  __shared__ float Bs[kSplitWaves][KS][T + 4];  // [wave][k][n]
  __shared__ float part[kSplitWaves][T][T + 4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tx = lane & 3, ty = lane >> 2;
  const int tiles_n = (N + T - 1) / T;
  const int m0 = (blockIdx.x / tiles_n) * T, n0 = (blockIdx.x % tiles_n) * T;
  const int nk = (K + KS - 1) / KS, steps = (nk + kSplitWaves - 1) / kSplitWaves;
  float ra[PER], rb[PER];
  auto fetch = [&](int kt) {
    const int k0 = kt * KS;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = lane + 64 * q;
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
  fetch(w);
  for (int st = 0; st < steps; ++st) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = lane + 64 * q;
      As[w][AK ? (e % KS) : (e / T)][AK ? (e / KS) : (e % T)] = ra[q];
      Bs[w][BK ? (e % KS) : (e / T)][BK ? (e / KS) : (e % T)] = rb[q];
    }
    __syncthreads();
    if (st + 1 < steps) fetch(w + kSplitWaves * (st + 1));  // in flight during the multiply below
#pragma unroll 16
    for (int k = 0; k < KS; ++k) {
      const float a = As[w][k][ty];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(a, Bs[w][k][tx * 4 + j], acc[j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) part[w][ty][tx * 4 + j] = acc[j];
  __syncthreads();
  if (w == 0) {
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    for (int v = 0; v < kSplitWaves; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) sum[j] += part[v][ty][tx * 4 + j];
    epi.template apply<4>(m0 + ty, n0 + tx * 4, sum);
  }
}

// 32 x 32 tiles when they fill the compute units, else the split form.
template <bool AK, bool BK, class Epi>
inline hipError_t launch_gemm_f32(const float* A, int64_t lda, const float* B, int64_t ldb, int M,
                                  int N, int K, const Epi& epi, hipStream_t stream) {
  const int tiles32 = ((M + 31) / 32) * ((N + 31) / 32);
  LGS_CHECK(M > 0 && N > 0 && K > 0);
  LGS_NEED(A, AK ? debug::mat_bytes(M, lda, K, 4) : debug::mat_bytes(K, lda, M, 4), "fp32 GEMM operand A");
  LGS_NEED(B, BK ? debug::mat_bytes(N, ldb, K, 4) : debug::mat_bytes(K, ldb, N, 4), "fp32 GEMM operand B");
  epi.debug_spans(0);
  if (tiles32 >= 256) {
    LGS_LAUNCH((gemm_f32_kernel<AK, BK, Epi, 32>), dim3(tiles32), dim3(256), 0, stream, A, lda, B, ldb, M, N, K,
               epi);
  } else {
    const int tiles16 = ((M + 15) / 16) * ((N + 15) / 16);
    LGS_LAUNCH((gemm_f32_split_kernel<AK, BK, Epi>), dim3(tiles16), dim3(64 * kSplitWaves), 0, stream, A, lda,
               B, ldb, M, N, K, epi);
  }
  return LGS_LAUNCH_STATUS();
}

}  // namespace lgs
