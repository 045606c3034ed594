// The cross-entropy partials of one vocabulary slice computed from logits
// that were written to HBM: per row, the slice max m, the sum of exp(z - m)
// and the target logit.  This is the streaming (unfused) form of the
// reductions that the fused CE keeps in registers; it exists to measure those
// reductions against the HBM roofline (each logit is read once), and is not
// part of the method's interface (declared in include/lgs_testing.h).
//
// One wave per row.  Each lane keeps a running (max, sum) over its 16-byte
// chunks with the online rescaling sum' = sum * exp(m - m') + sum exp(z - m')
// (one pass over the row), four chunk loads in flight, non-temporal loads
// (every byte is read once).  The lanes then combine with the same identity
// through lane shuffles.
#include "common.hpp"
#include "internal.hpp"

namespace lgs {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRowsPerBlock = 4;  // one row per wave
constexpr int kUnroll = 4;        // 16-byte chunks in flight per lane


__global__ __launch_bounds__(64 * kRowsPerBlock) void xent_rows_kernel(
    const bf16* __restrict__ Z, int64_t ldz, int M, int Vr, int vocab_start,
    const int32_t* __restrict__ targets, float* __restrict__ m_out, float* __restrict__ l_out,
    float* __restrict__ t_out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;  // whole waves only
  const bf16* z = Z + (int64_t)row * ldz;
  const int nchunk = Vr / 8;
  int tg = targets[row] - vocab_start;
  if (tg < 0 || tg >= Vr) tg = -1;  // not in this slice: the target logit stays +0
  float m = -INFINITY, l = 0.f, tv = 0.f;
  for (int c0 = lane; c0 < nchunk; c0 += 64 * kUnroll) {
    u32x4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + 64 * u;
      raw[u] = c < nchunk ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(z + 8 * c))
                          : u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};  // bf16 -inf
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bf16x8 v = __builtin_bit_cast(bf16x8, raw[u]);
      const int col = 8 * (c0 + 64 * u);
      float cm = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) cm = fmaxf(cm, (float)v[e]);
      const float nm = fmaxf(m, cm);
      const float sm = nm == -INFINITY ? 0.f : nm;
      float cs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cs += fast_exp((float)v[e] - sm);
        tv = col + e == tg ? (float)v[e] : tv;
      }
      l = l * fast_exp(m - sm) + cs;
      m = nm;
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float om = __shfl_xor(m, off), ol = __shfl_xor(l, off);
    const float nm = fmaxf(m, om);
    const float sm = nm == -INFINITY ? 0.f : nm;
    l = l * fast_exp(m - sm) + ol * fast_exp(om - sm);
    m = nm;
    tv += __shfl_xor(tv, off);
  }
  if (lane == 0) {
    m_out[row] = m;
    l_out[row] = l;
    t_out[row] = tv;
  }
}

}  // namespace

hipError_t xent_rows(int M, int Vr, int vocab_start, const void* Z, int64_t ldz,
                     const int32_t* targets, float* m, float* l, float* t, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(xent_rows_kernel, dim3((M + kRowsPerBlock - 1) / kRowsPerBlock),
                     dim3(64 * kRowsPerBlock), 0, s, (const bf16*)Z, ldz, M, Vr, vocab_start,
                     targets, m, l, t);
  return hipGetLastError();
}

}  // namespace lgs
