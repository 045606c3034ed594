// The cross-entropy partials of one vocabulary slice computed from logits
// that were written to HBM: per row, the slice max m, the sum of exp(z - m)
// and the target logit.  This is the streaming (unfused) form of the
// reductions that the fused CE keeps in registers; it exists to measure those
// reductions against the HBM roofline (each logit is read once), and is not
// part of the method's interface (declared in include/lgs_testing.h).
//
// One wave per row, non-temporal 16-byte loads (every byte is read once);
// the lanes' (max, sum) pairs combine through lane shuffles with the online
// log-sum-exp identity.  The exponentials (one per logit, quarter-rate on the
// vector ALU) rather than HBM set the pace unless the per-logit work stays
// at a handful of instructions, hence the batch structure below.
#include "common.hpp"
#include "internal.hpp"

namespace lgs {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRowsPerBlock = 8;  // one row per wave
constexpr int kBatch = 7;         // 16-byte chunks per lane held at once (3584 logits per wave)
constexpr float kLog2e = 1.4426950408889634f;

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
  // Batches of kBatch chunks per lane (two for a 6400-logit slice): all
  // loads of a batch in flight together, one max pass over the registers,
  // then one sum pass with a single shift; batches combine with the online
  // identity l' = l exp(m - m') + sum exp(z - m').
  for (int base = 0; base < nchunk; base += 64 * kBatch) {
    u32x4 raw[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = base + lane + 64 * u;
      raw[u] = c < nchunk ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(z + 8 * c))
                          : u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};  // bf16 -inf
    }
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bf16x8 v = __builtin_bit_cast(bf16x8, raw[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) bm = fmaxf(bm, (float)v[e]);
    }
    const float nm = fmaxf(m, bm);
    const float sm = nm == -INFINITY ? 0.f : nm;  // a row of -inf adds exp(-inf) = 0
    const float shift = sm * kLog2e;
    float bs = 0.f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bf16x8 v = __builtin_bit_cast(bf16x8, raw[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) bs += __builtin_amdgcn_exp2f(fmaf((float)v[e], kLog2e, -shift));
      const int col = 8 * (base + lane + 64 * u);
      if (tg >= col && tg < col + 8) tv = (float)v[tg - col];  // one lane, one chunk per row
    }
    l = l * __builtin_amdgcn_exp2f(fmaf(m, kLog2e, -shift)) + bs;
    m = nm;
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
