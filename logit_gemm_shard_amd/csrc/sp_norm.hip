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
// Each block takes a run of rows, RB at a time: every load of a batch (hs,
// dy, dhs, mask) is issued before its block sums (2 RB values reduced
// together), so the rows' memory latencies overlap.  The block adds dy * xhat and dy over its
// rows into its own fp32 column partials (dgamma, dbeta); col_sum_kernel then
// adds the blocks' partials in block order.

// Block sums of N values at once, the same in every thread; wave order.
template <int N>
__device__ __forceinline__ void block_sums(float (&v)[N], float* red) {
#pragma unroll
  for (int q = 0; q < N; ++q)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v[q] += __shfl_xor(v[q], off);
  __syncthreads();  // the previous use of red has been read
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int q = 0; q < N; ++q) red[(threadIdx.x >> 6) * N + q] = v[q];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = ((red[q] + red[N + q]) + red[2 * N + q]) + red[3 * N + q];
}

__device__ __forceinline__ void load8(const bf16* p, float (&v)[8]) {
  const bf16x8 x = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
}

template <int KC, int RB>  // KC 16-byte chunks per thread (h <= KC * 2048), RB rows per batch
__global__ __launch_bounds__(kThreads) void layernorm_bwd_kernel(
    const bf16* __restrict__ hs, const bf16* __restrict__ dy, const bf16* __restrict__ dhs,
    const uint8_t* __restrict__ keep, float keep_scale, const bf16* __restrict__ gamma, float eps, int rows,
    int rpb, int h, bf16* __restrict__ g, bf16* __restrict__ dz, float* __restrict__ part) {
  __shared__ float red[4 * 2 * RB];
  const int nch = h / 8;
  float cg[KC][8], cb[KC][8], gm[KC][8];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const int k = threadIdx.x + kThreads * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) cg[c][e] = cb[c][e] = gm[c][e] = 0.f;
    if (k < nch) load8(gamma + 8 * k, gm[c]);
  }
  const int r0 = blockIdx.x * rpb, r1 = min(rows, r0 + rpb);
  for (int rb = r0; rb < r1; rb += RB) {
    float x[RB][KC][8], d[RB][KC][8];
    u32x4 up[RB][KC];
    uint64_t mk[RB][KC];
    float s[2 * RB];
    // every load of the batch: hs, dy, dhs and the mask (rows past r1 read
    // as zeros and are not stored)
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int64_t base = (int64_t)(rb + q) * h;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int k = threadIdx.x + kThreads * c;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[q][c][e] = d[q][c][e] = 0.f;
        up[q][c] = u32x4{0u, 0u, 0u, 0u};
        mk[q][c] = ~0ull;
        if (rb + q < r1 && k < nch) {
          load8(hs + base + 8 * k, x[q][c]);
          load8(dy + base + 8 * k, d[q][c]);
          if (dhs) up[q][c] = *reinterpret_cast<const u32x4*>(dhs + base + 8 * k);
          if (keep) mk[q][c] = *reinterpret_cast<const uint64_t*>(keep + base + 8 * k);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      s[q] = s[RB + q] = 0.f;
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) s[q] += x[q][c][e];
    }
    block_sums<2 * RB>(s, red);  // s[q]: the row sums
    float rstd[RB];
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const float mean = s[q] / (float)h;
      s[q] = s[RB + q] = 0.f;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if (threadIdx.x + kThreads * c >= nch) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[q][c][e] -= mean;
          s[q] += x[q][c][e] * x[q][c][e];
        }
      }
    }
    block_sums<2 * RB>(s, red);  // s[q]: the squared deviations
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      rstd[q] = 1.f / sqrtf(s[q] / (float)h + eps);
      s[q] = s[RB + q] = 0.f;
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[q][c][e] *= rstd[q];  // xhat (zero past the row or past h)
          cg[c][e] += d[q][c][e] * x[q][c][e];
          cb[c][e] += d[q][c][e];
          d[q][c][e] *= gm[c][e];  // dxhat
          s[q] += d[q][c][e];
          s[RB + q] += d[q][c][e] * x[q][c][e];
        }
    }
    block_sums<2 * RB>(s, red);  // the two means' numerators
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      if (rb + q >= r1) break;
      const int64_t base = (int64_t)(rb + q) * h;
      const float m1 = s[q] / (float)h, m2 = s[RB + q] / (float)h;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int k = threadIdx.x + kThreads * c;
        if (k >= nch) continue;
        const bf16x8 u8 = __builtin_bit_cast(bf16x8, up[q][c]);
        const uint64_t m = mk[q][c];
        bf16x8 og, oz;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gv = (d[q][c][e] - m1 - x[q][c][e] * m2) * rstd[q] + (float)u8[e];
          og[e] = (bf16)gv;
          oz[e] = (bf16)(keep ? (((m >> (8 * e)) & 0xffu) ? gv * keep_scale : 0.f) : gv);
        }
        *reinterpret_cast<u32x4*>(g + base + 8 * k) = __builtin_bit_cast(u32x4, og);
        *reinterpret_cast<u32x4*>(dz + base + 8 * k) = __builtin_bit_cast(u32x4, oz);
      }
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

// dgamma[j] and dbeta[j] (j over the 2h columns of the partials): block x
// takes 64 consecutive columns; its kColWaves waves sum every kColWaves-th
// block's partial (wave w the blocks w, w + kColWaves, ...; a wave's loads
// cover 256 contiguous bytes, eight in flight), and the waves' sums are
// added in wave order.  The sum is latency-bound (2h / 64 blocks, 256
// partials): with 4 waves per block the whole backward took 21.5 us at h =
// 3072, 1024 rows; with 16, 18.0 us.
constexpr int kColWaves = 16;
__global__ __launch_bounds__(64 * kColWaves) void col_sum_kernel(const float* __restrict__ part, int nblk, int h,
                                                                float* __restrict__ dgamma,
                                                                float* __restrict__ dbeta) {
  __shared__ float red[kColWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane;
  float acc = 0.f;
  if (j < 2 * h)
    for (int q0 = w; q0 < nblk; q0 += kColWaves * 8) {  // eight loads in flight, added in block order
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + kColWaves * u;
        v[u] = q < nblk ? part[(int64_t)q * 2 * h + j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
  red[w][lane] = acc;
  __syncthreads();
  if (w == 0 && j < 2 * h) {
    float v = red[0][lane];
#pragma unroll
    for (int q = 1; q < kColWaves; ++q) v += red[q][lane];
    if (j < h)
      dgamma[j] = v;
    else
      dbeta[j - h] = v;
  }
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
    LGS_LAUNCH(col_sum_kernel, dim3((2 * h + 63) / 64), dim3(64 * kColWaves), 0, s, (const float*)nullptr, 0, h,
               dgamma, dbeta);
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
  auto launch = [&](auto kc_c, auto rb_c) {
    constexpr int KC = decltype(kc_c)::value, RB = decltype(rb_c)::value;
    LGS_LAUNCH((layernorm_bwd_kernel<KC, RB>), dim3(nblk), dim3(kThreads), 0, s, (const bf16*)hs,
               (const bf16*)dy, (const bf16*)dhs, keep, keep_scale, (const bf16*)gamma, eps, rows, rpb, h,
               (bf16*)g, (bf16*)dz, (float*)scratch);
  };
  using I = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  if (kc <= 1)
    launch(I{}, I4{});
  else if (kc <= 2)
    launch(I2{}, I4{});
  else if (kc <= 4)
    launch(I4{}, I2{});
  else
    launch(std::integral_constant<int, 8>{}, I{});
  LGS_LAUNCH(col_sum_kernel, dim3((2 * h + 63) / 64), dim3(64 * kColWaves), 0, s, (const float*)scratch, nblk, h,
             dgamma, dbeta);
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
