// The sequence-parallel region after the row-parallel exit, in one pass.
//
// "Mathematical Foundations of Megatron-LM ..." (llms.blog), "Sequence
// Parallelism", "Splitting All-Reduce into Reduce-Scatter and All-Gather":
// the row-parallel GEMM's partials are reduce-scattered along the sequence,
// and LayerNorm, the residual addition and dropout then run locally on the
// rank's (s/t, b, h) chunk before the all-gather that feeds the next
// column-parallel GEMM.  Per token row of rank r's chunk:
//
//   z  = sum_i part_i[row]      fp32, ascending i (the reduce-scatter's sum)
//   d  = keep ? z * keep_scale : 0      (dropout with a given keep mask;
//        z where no mask is given)
//   hs = residual[row] + d      the residual stream, written in bf16
//   y  = (hs - mean) / sqrt(var + eps) * gamma + beta   written in bf16
//
// with the mean and the biased variance of the row's fp32 hs over h.  One
// pass over HBM: the t partial rows, the residual row and the mask are read
// once, hs and y written once; the row stays in registers between the two
// reductions.
//
// One block of 256 threads per row; thread j owns the 16-byte chunks j,
// j + 256, ... (at most kMaxChunks of them: h <= 16384).  The block's sums
// combine the four waves' shuffle-reduced totals in wave order, so the result
// does not depend on timing.
#include "common.hpp"
#include "internal.hpp"

namespace lgs {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
constexpr int kThreads = 256;
constexpr int kMaxChunks = 8;
constexpr int kRankBatch = 8;  // partials whose loads are issued together

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Sum over the block, the same value in every thread.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();  // the previous use of red has been read
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__global__ __launch_bounds__(kThreads) void rs_layernorm_kernel(
    const bf16* __restrict__ parts, int64_t stride, int t, const bf16* __restrict__ residual,
    const uint8_t* __restrict__ keep, float keep_scale, const bf16* __restrict__ gamma,
    const bf16* __restrict__ beta, float eps, int h, bf16* __restrict__ hs, bf16* __restrict__ y) {
  __shared__ float red[kThreads / 64];
  const int64_t row0 = (int64_t)blockIdx.x * h;
  const int nch = h / 8;
  float v[kMaxChunks][8];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int k = threadIdx.x + kThreads * c;
    if (k >= nch) break;
    const int64_t off = row0 + 8 * k;
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < t; i0 += kRankBatch) {
      u32x4 q[kRankBatch];
#pragma unroll
      for (int j = 0; j < kRankBatch; ++j)
        if (i0 + j < t) q[j] = ld16(parts + (int64_t)(i0 + j) * stride + off);
#pragma unroll
      for (int j = 0; j < kRankBatch; ++j)
        if (i0 + j < t) {
          const bf16x8 x = __builtin_bit_cast(bf16x8, q[j]);
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] += (float)x[e];
        }
    }
    if (keep) {
      const u32x2 m = *reinterpret_cast<const u32x2*>(keep + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = ((m[e >> 2] >> (8 * (e & 3))) & 0xffu) ? a[e] * keep_scale : 0.f;
    }
    const bf16x8 r = __builtin_bit_cast(bf16x8, ld16(residual + off));
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] += (float)r[e];
      o[e] = (bf16)a[e];
      v[c][e] = a[e];
      sum += a[e];
    }
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, o), reinterpret_cast<u32x4*>(hs + off));
  }
  const float mean = block_sum(sum, red) / (float)h;
  float sq = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (threadIdx.x + kThreads * c >= nch) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float dlt = v[c][e] - mean;
      sq += dlt * dlt;
    }
  }
  const float rstd = 1.f / sqrtf(block_sum(sq, red) / (float)h + eps);
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int k = threadIdx.x + kThreads * c;
    if (k >= nch) break;
    const bf16x8 g = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(gamma + 8 * k));
    const bf16x8 bb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(beta + 8 * k));
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)((v[c][e] - mean) * rstd * (float)g[e] + (float)bb[e]);
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, o), reinterpret_cast<u32x4*>(y + row0 + 8 * k));
  }
}

}  // namespace

int rs_layernorm_max_h() { return kMaxChunks * kThreads * 8; }

hipError_t rs_layernorm(int t, int rows, int h, int rank, const void* parts, int64_t stride,
                        const void* residual, const uint8_t* keep, float keep_scale, const void* gamma,
                        const void* beta, float eps, void* hs, void* y, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  LGS_CHECK(h % 8 == 0 && h <= rs_layernorm_max_h() && t >= 1);
  const int64_t chunk = (int64_t)rows * h;
  const bf16* base = (const bf16*)parts + (int64_t)rank * chunk;  // rank's rows of every partial
  LGS_NEED(base, (size_t)((t - 1) * stride + chunk) * 2, "partials (rank's rows)");
  LGS_NEED(residual, (size_t)chunk * 2, "residual chunk");
  if (keep) LGS_NEED(keep, (size_t)chunk, "keep mask");
  LGS_NEED(gamma, (size_t)h * 2, "gamma");
  LGS_NEED(beta, (size_t)h * 2, "beta");
  LGS_NEED(hs, (size_t)chunk * 2, "residual stream out");
  LGS_NEED(y, (size_t)chunk * 2, "LayerNorm out");
  LGS_LAUNCH(rs_layernorm_kernel, dim3(rows), dim3(kThreads), 0, s, base, stride, t, (const bf16*)residual,
             keep, keep_scale, (const bf16*)gamma, (const bf16*)beta, eps, h, (bf16*)hs, (bf16*)y);
  return LGS_LAUNCH_STATUS();
}

}  // namespace lgs
