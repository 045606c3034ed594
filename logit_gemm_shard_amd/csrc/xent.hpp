// Fused vocab-parallel cross-entropy: the logit GEMM's epilogue reduces each
// row of the wave's logit tile to (max, sum of exp relative to that max,
// target logit, first argmax) and writes those four numbers per row and per
// wave column-slab.  Logits never leave the chip: they go from the matrix
// cores' accumulators through LDS to the reductions.  A small merge kernel
// then folds the slabs of the rank's vocabulary slice into the rank's partials.
//
// "LIT-022: Megatron-LM ..." (dmarx anthology), "Key takeaways": fusing the
// parallel logit GEMM into the loss replaces the b*s*v all-gather of logits
// with O(b*s) numbers per rank.
#pragma once

#include "common.hpp"
#include "gemm_bf16.hpp"

namespace lgs {

struct XentSlabs {
  float* m;      // [slabs][M] slab max
  float* l;      // [slabs][M] sum exp(z - slab max)
  float* t;      // [slabs][M] target logit if the target is in the slab, else +0
  int32_t* idx;  // [slabs][M] slice-local column of the slab's first maximum
};

struct EpiXent {
  XentSlabs s;
  const int32_t* targets;  // [M] global vocabulary ids
  int vocab_start;         // first global id of this rank's slice
  int M, N;                // tokens, slice width
  int WN;                  // wave tile width: slab = wave column

  // A staged slice holds 32 rows x WN logits.  Two lanes share a row, each
  // reducing a contiguous half of it (columns visited in increasing order),
  // then the two combine with a lane shuffle.
  template <int WNt, int LD>
  __device__ __forceinline__ void slice(const float* st, int m0, int nb, int lane) const {
    static_assert(WNt % 8 == 0, "a half row is read as float4s");
    constexpr int Q = WNt / 2;
    const int r = lane >> 1, part = lane & 1;
    const int m = m0 + r;
    const int c0 = part * Q;
    const float* row = st + r * LD + c0;
    const int ncols = min(Q, N - (nb + c0));  // valid columns of this half (may be <= 0)
    const int tl = (m < M ? targets[m] - vocab_start : -1) - (nb + c0);
    float best = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll 4
    for (int c = 0; c < Q; c += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + c);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c + k < ncols && v[k] > best) { best = v[k]; bi = nb + c0 + c + k; }
    }
    {
      const float ob = __shfl_xor(best, 1);
      const int oi = __shfl_xor(bi, 1);
      if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    float sum = 0.f, tv = 0.f;
#pragma unroll 4
    for (int c = 0; c < Q; c += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + c);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c + k < ncols) {
          sum += fast_exp(v[k] - best);
          if (c + k == tl) tv = v[k];
        }
    }
    sum += __shfl_xor(sum, 1);
    tv += __shfl_xor(tv, 1);
    if (part == 0 && m < M) {
      const int64_t o = (int64_t)(nb / WN) * M + m;
      s.m[o] = best;
      s.l[o] = sum;
      s.t[o] = tv;
      s.idx[o] = bi;
    }
  }
};

}  // namespace lgs
