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
// vector ALU) and the other per-logit arithmetic compete with the loads, so
// the per-logit work is kept to a handful of instructions: batches of
// kBatch chunks per lane, the next batch's loads issued before the current
// one is reduced, and the target logit read straight from memory by one lane
// instead of picked out of the registers.  Measured on the 8.3B slice
// ([8192, 6400], three rotating buffers): 21.7 us (7 chunks per batch, no
// prefetch, register pick) -> 19.2-19.5 us (5 per batch, prefetch) ->
// 18.7-19.0 us (7 per batch: a row is two batches, the second 79% full,
// instead of 2.5) -> 18.67 us against 18.86 (best of ten, alternating:
// bounds checks only in a row's last, partial batch).  A probe without the
// exponentials (wrong results) takes 18.1-18.2 us, so the per-logit
// arithmetic costs about 4%.  Variants that measured slower: 4, 5, 6, 8, 10
// or 13 chunks per batch, 4 or 16 rows per block, two alternating register
// sets instead of copying the prefetched batch, the last batch specialised
// by its length (seven copies of the row loop).
#include "common.hpp"
#include "internal.hpp"

namespace lgs {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRowsPerBlock = 8;  // one row per wave
constexpr int kBatch = 7;         // 16-byte chunks per lane per batch (3584 logits per wave)
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
  // Batches that lie wholly inside the row load without bounds checks; only
  // the last, partial one checks each chunk (and pads with -inf).
  auto load = [&](int base, u32x4 (&dst)[kBatch], auto checked_c) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = base + lane + 64 * u;
      if constexpr (decltype(checked_c)::value)
        dst[u] = c < nchunk ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(z + 8 * c))
                            : u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};  // bf16 -inf
      else
        dst[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(z + 8 * c));
    }
  };
  const int nfull = nchunk / (64 * kBatch);
  const int nbatch = (nchunk + 64 * kBatch - 1) / (64 * kBatch);
  auto load_batch = [&](int b, u32x4 (&dst)[kBatch]) {
    if (b < nfull)
      load(64 * kBatch * b, dst, std::false_type{});
    else
      load(64 * kBatch * b, dst, std::true_type{});
  };
  float m = -INFINITY, l = 0.f;
  // Batches combine with the online identity l' = l exp(m - m') + sum exp(z - m'):
  // one max pass over a batch's registers, then one sum pass with a single shift.
  u32x4 next[kBatch];
  if (nbatch > 0) load_batch(0, next);
  for (int b = 0; b < nbatch; ++b) {
    u32x4 raw[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) raw[u] = next[u];
    if (b + 1 < nbatch) load_batch(b + 1, next);
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
  }
  if (lane == 0) {
    const int tg = targets[row] - vocab_start;
    m_out[row] = m;
    l_out[row] = l;
    t_out[row] = (tg >= 0 && tg < Vr) ? (float)z[tg] : 0.f;  // not in this slice: +0
  }
}

}  // namespace

hipError_t xent_rows(int M, int Vr, int vocab_start, const void* Z, int64_t ldz,
                     const int32_t* targets, float* m, float* l, float* t, hipStream_t s) {
  if (M == 0) return hipSuccess;
  LGS_NEED(Z, debug::mat_bytes(M, ldz, Vr, 2), "materialised logits");
  LGS_NEED(targets, (size_t)M * 4, "targets");
  LGS_NEED(m, (size_t)M * 4, "m");
  LGS_NEED(l, (size_t)M * 4, "l");
  LGS_NEED(t, (size_t)M * 4, "T");
  LGS_LAUNCH(xent_rows_kernel, dim3((M + kRowsPerBlock - 1) / kRowsPerBlock), dim3(64 * kRowsPerBlock), 0, s,
             (const bf16*)Z, ldz, M, Vr, vocab_start, targets, m, l, t);
  return LGS_LAUNCH_STATUS();
}

}  // namespace lgs
