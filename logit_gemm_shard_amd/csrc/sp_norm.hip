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

// Backward of the region, on rank r's rows: LayerNorm's statistics are
// recomputed from the stored hs (bf16); per row
//   xhat = (hs - mean) * rstd,  dxhat = dy * gamma
//   dx   = (dxhat - mean_h(dxhat) - xhat * mean_h(dxhat * xhat)) * rstd
//   g    = dx + dhs              the gradient of hs and of the residual input
//   dz   = keep ? g * keep_scale : 0  (g without a mask)
// and each block adds dy * xhat and dy over its rows into its own fp32 column
// partials (dgamma, dbeta), which col_sum_kernel then adds in block order.
// Block sums of two values at a time (the two means of a row).
__device__ __forceinline__ void block_sum2(float& a, float& b, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_xor(a, off);
    b += __shfl_xor(b, off);
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = a;
    red[4 + (threadIdx.x >> 6)] = b;
  }
  __syncthreads();
  a = ((red[0] + red[1]) + red[2]) + red[3];
  b = ((red[4] + red[5]) + red[6]) + red[7];
}

__device__ __forceinline__ void load8(const bf16* p, float (&v)[8]) {
  const bf16x8 x = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
}

template <int KC>  // 16-byte chunks per thread: h <= KC * 2048
__global__ __launch_bounds__(kThreads) void layernorm_bwd_kernel(
    const bf16* __restrict__ hs, const bf16* __restrict__ dy, const bf16* __restrict__ dhs,
    const uint8_t* __restrict__ keep, float keep_scale, const bf16* __restrict__ gamma, float eps, int rows,
    int rpb, int h, bf16* __restrict__ g, bf16* __restrict__ dz, float* __restrict__ part) {
  __shared__ float red[8];
  const int nch = h / 8;
  float cg[KC][8], cb[KC][8];
#pragma unroll
  for (int c = 0; c < KC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) cg[c][e] = cb[c][e] = 0.f;
  const int r0 = blockIdx.x * rpb, r1 = min(rows, r0 + rpb);
  for (int row = r0; row < r1; ++row) {
    const int64_t base = (int64_t)row * h;
    float x[KC][8], d[KC][8];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int k = threadIdx.x + kThreads * c;
      if (k >= nch) break;
      load8(hs + base + 8 * k, x[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s1 += x[c][e];
    }
    block_sum2(s1, s2, red);
    const float mean = s1 / (float)h;
    float sq = 0.f, unused = 0.f;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (threadIdx.x + kThreads * c >= nch) break;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[c][e] -= mean;
        sq += x[c][e] * x[c][e];
      }
    }
    block_sum2(sq, unused, red);
    const float rstd = 1.f / sqrtf(sq / (float)h + eps);
    float m1 = 0.f, m2 = 0.f;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int k = threadIdx.x + kThreads * c;
      if (k >= nch) break;
      float gm[8];
      load8(dy + base + 8 * k, d[c]);
      load8(gamma + 8 * k, gm);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[c][e] *= rstd;  // xhat
        cg[c][e] += d[c][e] * x[c][e];
        cb[c][e] += d[c][e];
        d[c][e] *= gm[e];  // dxhat
        m1 += d[c][e];
        m2 += d[c][e] * x[c][e];
      }
    }
    block_sum2(m1, m2, red);
    m1 /= (float)h;
    m2 /= (float)h;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int k = threadIdx.x + kThreads * c;
      if (k >= nch) break;
      float up[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (dhs) load8(dhs + base + 8 * k, up);
      uint64_t m = ~0ull;
      if (keep) m = *reinterpret_cast<const uint64_t*>(keep + base + 8 * k);
      bf16x8 og, oz;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gv = (d[c][e] - m1 - x[c][e] * m2) * rstd + up[e];
        og[e] = (bf16)gv;
        oz[e] = (bf16)(keep ? (((m >> (8 * e)) & 0xffu) ? gv * keep_scale : 0.f) : gv);
      }
      *reinterpret_cast<u32x4*>(g + base + 8 * k) = __builtin_bit_cast(u32x4, og);
      *reinterpret_cast<u32x4*>(dz + base + 8 * k) = __builtin_bit_cast(u32x4, oz);
    }
  }
  float* pg = part + (int64_t)blockIdx.x * 2 * h;
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const int k = threadIdx.x + kThreads * c;
    if (k >= nch) break;
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      *reinterpret_cast<f32x4*>(pg + 8 * k + e) = f32x4{cg[c][e], cg[c][e + 1], cg[c][e + 2], cg[c][e + 3]};
      *reinterpret_cast<f32x4*>(pg + h + 8 * k + e) = f32x4{cb[c][e], cb[c][e + 1], cb[c][e + 2], cb[c][e + 3]};
    }
  }
}

// dgamma[j] and dbeta[j]: the blocks' column partials added in block order.
__global__ __launch_bounds__(256) void col_sum_kernel(const float* __restrict__ part, int nblk, int h,
                                                     float* __restrict__ dgamma, float* __restrict__ dbeta) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= 2 * h) return;
  float acc = 0.f;
  for (int q = 0; q < nblk; ++q) acc += part[(int64_t)q * 2 * h + j];
  if (j < h)
    dgamma[j] = acc;
  else
    dbeta[j - h] = acc;
}

// Rows per block of the backward: at most 256 blocks, so the column partials
// stay small.
int bwd_rows_per_block(int rows) { return (rows + 255) / 256; }

}  // namespace

int rs_layernorm_max_h() { return kMaxChunks * kThreads * 8; }

size_t layernorm_bwd_scratch_bytes(int rows, int h) {
  if (rows == 0) return 0;
  const int rpb = bwd_rows_per_block(rows), nblk = (rows + rpb - 1) / rpb;
  return (size_t)nblk * 2 * h * sizeof(float);
}

hipError_t layernorm_bwd(int rows, int h, const void* hs, const void* dy, const void* dhs, const uint8_t* keep,
                         float keep_scale, const void* gamma, float eps, void* g, void* dz, float* dgamma,
                         float* dbeta, void* scratch, hipStream_t s) {
  LGS_CHECK(h % 8 == 0 && h <= rs_layernorm_max_h());
  LGS_NEED(gamma, (size_t)h * 2, "gamma");
  LGS_NEED(dgamma, (size_t)h * 4, "dgamma");
  LGS_NEED(dbeta, (size_t)h * 4, "dbeta");
  if (rows == 0) {  // no rows: the rank's partial sums are zero
    LGS_LAUNCH(col_sum_kernel, dim3((2 * h + 255) / 256), dim3(256), 0, s, (const float*)nullptr, 0, h, dgamma, dbeta);
    return LGS_LAUNCH_STATUS();
  }
  const int rpb = bwd_rows_per_block(rows), nblk = (rows + rpb - 1) / rpb;
  const size_t chunk = (size_t)rows * h;
  LGS_NEED(hs, chunk * 2, "hs");
  LGS_NEED(dy, chunk * 2, "dy");
  if (dhs) LGS_NEED(dhs, chunk * 2, "dhs");
  if (keep) LGS_NEED(keep, chunk, "keep mask");
  LGS_NEED(g, chunk * 2, "g");
  LGS_NEED(dz, chunk * 2, "dz");
  LGS_NEED(scratch, layernorm_bwd_scratch_bytes(rows, h), "column partials");
  const int kc = (h / 8 + kThreads - 1) / kThreads;
  auto launch = [&](auto kc_c) {
    constexpr int KC = decltype(kc_c)::value;
    LGS_LAUNCH(layernorm_bwd_kernel<KC>, dim3(nblk), dim3(kThreads), 0, s, (const bf16*)hs, (const bf16*)dy,
               (const bf16*)dhs, keep, keep_scale, (const bf16*)gamma, eps, rows, rpb, h, (bf16*)g, (bf16*)dz,
               (float*)scratch);
  };
  if (kc <= 1)
    launch(std::integral_constant<int, 1>{});
  else if (kc <= 2)
    launch(std::integral_constant<int, 2>{});
  else if (kc <= 4)
    launch(std::integral_constant<int, 4>{});
  else
    launch(std::integral_constant<int, 8>{});
  LGS_LAUNCH(col_sum_kernel, dim3((2 * h + 255) / 256), dim3(256), 0, s, (const float*)scratch, nblk, h, dgamma,
             dbeta);
  return LGS_LAUNCH_STATUS();
}

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
