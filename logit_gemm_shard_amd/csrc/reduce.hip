// One-device stand-ins for the two exchanges of the tensor-parallel path.
//
// * Sum of partials: out = sum_{r < t} part_r, fp32 accumulation in ascending
//   rank order (so the result does not depend on timing).  This is the
//   all-reduce of the row-parallel exit (g forward: Z = sum_i Z_i) and of the
//   column-parallel entry (f backward: dX = sum_i dX_i), "Mathematical
//   Foundations of Megatron-LM ...", "Row-Parallel Linear Layer" and
//   "Conjugate Communication Operators".  A pure HBM stream: 16-byte loads of
//   every rank's block per thread, t loads in flight before the adds, all
//   marked non-temporal (each byte is touched once, so caching it only evicts
//   what the GEMMs around it reuse; measured ~15% faster than plain accesses).
// * Sequence-parallel exit and entry ("Mathematical Foundations of
//   Megatron-LM ...", "Sequence Parallelism"): the reduce-scatter is the same
//   sum over only rank r's s/t rows of the (s, b, h) tensor (s outermost, so a
//   contiguous range), and the all-gather a copy of the t chunks into place.
// * CE merge: loss = M* + ln(sum_r l_r exp(m_r - M*)) - sum_r T_r with
//   M* = max_r m_r, the log-sum-exp identity over the ranks' slice partials,
//   or (for the backward) the log-sum-exp M* + ln L* alone.
#include "common.hpp"
#include "internal.hpp"

namespace lgs {

template <typename T> struct Vec8;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

template <> struct Vec8<bf16> {
  u32x4 v;
  __device__ __forceinline__ void load(const bf16* p) { v = ld_nt(p); }
  __device__ __forceinline__ void add_to(float (&a)[8]) const {
    const bf16x8 x = __builtin_bit_cast(bf16x8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] += (float)x[i];
  }
  __device__ __forceinline__ static void store(bf16* p, const float (&a)[8]) {
    bf16x8 x;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (bf16)a[i];
    st_nt(p, __builtin_bit_cast(u32x4, x));
  }
};
template <> struct Vec8<float> {
  u32x4 v0, v1;
  __device__ __forceinline__ void load(const float* p) {
    v0 = ld_nt(p);
    v1 = ld_nt(p + 4);
  }
  __device__ __forceinline__ void add_to(float (&a)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] += __uint_as_float(v0[i]);
      a[4 + i] += __uint_as_float(v1[i]);
    }
  }
  __device__ __forceinline__ static void store(float* p, const float (&a)[8]) {
    st_nt(p, u32x4{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]), __float_as_uint(a[3])});
    st_nt(p + 4, u32x4{__float_as_uint(a[4]), __float_as_uint(a[5]), __float_as_uint(a[6]), __float_as_uint(a[7])});
  }
};

constexpr int kChunkT = 8;  // ranks whose loads are issued together

// Vector path: n % 8 == 0 and every rank block 16-byte aligned (checked on the host).
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void psum_vec_kernel(const TI* __restrict__ parts, int64_t stride,
                                                       int t, int64_t n, TO* __restrict__ out) {
  const int64_t step = (int64_t)gridDim.x * 256 * 8;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += step) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int r0 = 0; r0 < t; r0 += kChunkT) {
      Vec8<TI> v[kChunkT];
#pragma unroll
      for (int r = 0; r < kChunkT; ++r)
        if (r0 + r < t) v[r].load(parts + (int64_t)(r0 + r) * stride + i);
#pragma unroll
      for (int r = 0; r < kChunkT; ++r)
        if (r0 + r < t) v[r].add_to(a);
    }
    Vec8<TO>::store(out + i, a);
  }
}

template <typename TI, typename TO>
__global__ __launch_bounds__(256) void psum_scalar_kernel(const TI* __restrict__ parts,
                                                          int64_t stride, int t, int64_t n,
                                                          TO* __restrict__ out) {
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += step) {
    float a = 0.f;
    for (int r = 0; r < t; ++r) a += (float)parts[(int64_t)r * stride + i];
    out[i] = (TO)a;
  }
}

template <typename TI, typename TO>
static hipError_t psum(int t, int64_t n, const void* parts, int64_t stride, void* out,
                       hipStream_t s) {
  const bool vec = (n % 8 == 0) && ((uintptr_t)parts % 16 == 0) && ((uintptr_t)out % 16 == 0) &&
                   ((stride * (int64_t)sizeof(TI)) % 16 == 0);
  const int64_t per_block = vec ? 256 * 8 : 256;
  const int64_t want = (n + per_block - 1) / per_block;
  const int blocks = (int)(want < 8192 ? (want < 1 ? 1 : want) : 8192);
  LGS_CHECK(t >= 1 && n >= 1 && (t == 1 || stride >= n));
  LGS_NEED(parts, (size_t)((t - 1) * stride + n) * sizeof(TI), "partials");
  LGS_NEED(out, (size_t)n * sizeof(TO), "sum of the partials");
  if (vec)
    LGS_LAUNCH((psum_vec_kernel<TI, TO>), dim3(blocks), dim3(256), 0, s, (const TI*)parts, stride, t, n,
               (TO*)out);
  else
    LGS_LAUNCH((psum_scalar_kernel<TI, TO>), dim3(blocks), dim3(256), 0, s, (const TI*)parts, stride, t, n,
               (TO*)out);
  return LGS_LAUNCH_STATUS();
}

hipError_t partial_sum(int t, int64_t n, bool in_bf16, bool out_bf16, const void* parts,
                       int64_t stride, void* out, hipStream_t s) {
  if (in_bf16)
    return out_bf16 ? psum<bf16, bf16>(t, n, parts, stride, out, s)
                    : psum<bf16, float>(t, n, parts, stride, out, s);
  return out_bf16 ? psum<float, bf16>(t, n, parts, stride, out, s)
                  : psum<float, float>(t, n, parts, stride, out, s);
}

hipError_t reduce_scatter(int t, int64_t chunk, int rank, bool in_bf16, bool out_bf16,
                          const void* parts, int64_t stride, void* out, hipStream_t s) {
  const char* base = (const char*)parts + (int64_t)rank * chunk * (in_bf16 ? 2 : 4);
  return partial_sum(t, chunk, in_bf16, out_bf16, base, stride, out, s);
}

// out[q * chunk + j] = shards[q * stride + j]: blockIdx.y is the chunk q, the
// blocks along x stride over it in 16-byte vectors (the vector path needs
// chunk bytes, stride bytes and both bases 16-byte aligned).
__global__ __launch_bounds__(256) void gather_vec_kernel(const char* __restrict__ shards,
                                                         int64_t stride_bytes, int64_t vecs,
                                                         char* __restrict__ out) {
  const int q = blockIdx.y;
  const char* src = shards + (int64_t)q * stride_bytes;
  char* dst = out + (int64_t)q * vecs * 16;
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < vecs; i += step)
    st_nt(dst + i * 16, ld_nt(src + i * 16));
}

template <typename T>
__global__ __launch_bounds__(256) void gather_scalar_kernel(const T* __restrict__ shards,
                                                            int64_t stride, int64_t chunk,
                                                            T* __restrict__ out) {
  const int q = blockIdx.y;
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < chunk; i += step)
    out[(int64_t)q * chunk + i] = shards[(int64_t)q * stride + i];
}

hipError_t all_gather(int t, int64_t chunk, bool bf16, const void* shards, int64_t stride,
                      void* out, hipStream_t s) {
  const int64_t esz = bf16 ? 2 : 4, bytes = chunk * esz;
  const bool vec = bytes % 16 == 0 && (stride * esz) % 16 == 0 && (uintptr_t)shards % 16 == 0 &&
                   (uintptr_t)out % 16 == 0;
  const int64_t units = vec ? bytes / 16 : chunk;
  const int64_t want = (units + 255) / 256;
  const int bx = (int)(want < 2048 ? (want < 1 ? 1 : want) : 2048);
  const dim3 grid(bx, t);
  LGS_CHECK(t >= 1 && t <= 65535 && chunk >= 1 && (t == 1 || stride >= chunk));
  LGS_NEED(shards, (size_t)((t - 1) * stride + chunk) * esz, "all-gather shards");
  LGS_NEED(out, (size_t)t * chunk * esz, "all-gather output");
  if (vec)
    LGS_LAUNCH(gather_vec_kernel, grid, dim3(256), 0, s, (const char*)shards, stride * esz, units, (char*)out);
  else if (bf16)
    LGS_LAUNCH((gather_scalar_kernel<uint16_t>), grid, dim3(256), 0, s, (const uint16_t*)shards, stride, chunk,
               (uint16_t*)out);
  else
    LGS_LAUNCH((gather_scalar_kernel<uint32_t>), grid, dim3(256), 0, s, (const uint32_t*)shards, stride, chunk,
               (uint32_t*)out);
  return LGS_LAUNCH_STATUS();
}

// parts: rank r's block at parts + r*stride holds m[n], l[n], T[n] (T is not
// read for the log-sum-exp alone).
// Ranks are taken in chunks of kCombineChunk whose loads are all issued
// before any is used (a runtime-length loop would wait on each load in turn);
// chunks merge with the online identity.  For t <= kCombineChunk this is the
// single pass best = max_r m_r, L = sum_r l_r exp(m_r - best).
constexpr int kCombineChunk = 8;
__global__ __launch_bounds__(256) void xent_combine_kernel(const float* __restrict__ parts,
                                                           int64_t stride, int t, int64_t n,
                                                           bool lse_only, float* __restrict__ loss) {
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += step) {
    float best = -INFINITY, L = 0.f, T = 0.f;
    for (int r0 = 0; r0 < t; r0 += kCombineChunk) {
      float m[kCombineChunk], l[kCombineChunk], tt[kCombineChunk];
#pragma unroll
      for (int r = 0; r < kCombineChunk; ++r) {
        const bool ok = r0 + r < t;
        const float* p = parts + (int64_t)(ok ? r0 + r : 0) * stride;
        m[r] = ok ? p[i] : -INFINITY;
        l[r] = ok ? p[n + i] : 0.f;
        tt[r] = ok && !lse_only ? p[2 * n + i] : 0.f;
      }
      float cm = best;
#pragma unroll
      for (int r = 0; r < kCombineChunk; ++r) cm = m[r] > cm ? m[r] : cm;
      float cl = r0 == 0 ? 0.f : L * __expf(best - cm);
#pragma unroll
      for (int r = 0; r < kCombineChunk; ++r) {
        if (r0 + r < t) cl += l[r] * __expf(m[r] - cm);
        T += tt[r];
      }
      best = cm;
      L = cl;
    }
    loss[i] = best + logf(L) - T;
  }
}

hipError_t xent_combine(int t, int64_t n, const float* parts, int64_t stride, bool lse_only,
                        float* loss, hipStream_t s) {
  const int64_t want = (n + 255) / 256;
  const int blocks = (int)(want < 8192 ? (want < 1 ? 1 : want) : 8192);
  const int64_t planes = lse_only ? 2 : 3;
  LGS_CHECK(t >= 1 && n >= 1 && stride >= planes * n);
  LGS_NEED(parts, (size_t)((t - 1) * stride + planes * n) * 4, "CE partials of every rank");
  LGS_NEED(loss, (size_t)n * 4, "CE merge output");
  LGS_LAUNCH(xent_combine_kernel, dim3(blocks), dim3(256), 0, s, parts, stride, t, n, lse_only, loss);
  return LGS_LAUNCH_STATUS();
}

}  // namespace lgs
