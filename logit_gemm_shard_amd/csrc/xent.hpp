// Fused vocab-parallel cross-entropy: the logit GEMM's epilogue reduces each
// row of the wave's logit tile to (max, sum of exp relative to that max,
// target logit, first argmax) and writes those four numbers per row and per
// wave column-slab.  Logits never leave registers.  A small merge kernel then
// folds the slabs of the rank's vocabulary slice into the rank's partials.
//
// "LIT-022: Megatron-LM ..." (dmarx anthology), "Key takeaways": fusing the
// parallel logit GEMM into the loss replaces the b*s*v all-gather of logits
// with O(b*s) numbers per rank.
#pragma once

#include "common.hpp"

namespace lgs {

struct XentSlabs {
  float* m;      // [slabs][M] slab max
  float* l;      // [slabs][M] sum exp(z - slab max)
  float* t;      // [slabs][M] target logit if the target is in the slab, else +0
  int32_t* idx;  // [slabs][M] slab-local column of the first maximum
};

struct EpiXent {
  static constexpr bool kWholeTile = true;
  XentSlabs s;
  const int32_t* targets;  // [M] global vocabulary ids
  int vocab_start;         // first global id of this rank's slice
  int M, N;                // tokens, slice width
  int WN;                  // wave tile width: slab = wave column

  template <int TM, int TN>
  __device__ __forceinline__ void tile(const f32x4 (&acc)[TM][TN], int mb, int nb, int lane) const {
    const int slab = nb / WN;
    const int g = lane >> 4;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = mb + i * 16 + (lane & 15);
      const bool mv = m < M;
      const int tl = mv ? targets[m] - vocab_start : -1;
      // lane-local max / first argmax, columns visited in increasing order
      float best = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = nb + j * 16 + 4 * g + r;
          const float v = acc[i][j][r];
          if (n < N && v > best) { best = v; bi = n; }
        }
      // the row is spread over the four 16-lane groups of the wave
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
        const float ob = __shfl_xor(best, off);
        const int oi = __shfl_xor(bi, off);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
      }
      float sum = 0.f, tv = 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = nb + j * 16 + 4 * g + r;
          const float v = acc[i][j][r];
          if (n < N) {
            sum += __expf(v - best);
            if (n == tl) tv = v;
          }
        }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      tv += __shfl_xor(tv, 16);
      tv += __shfl_xor(tv, 32);
      if (g == 0 && mv) {
        const int64_t o = (int64_t)slab * M + m;
        s.m[o] = best;
        s.l[o] = sum;
        s.t[o] = tv;
        s.idx[o] = bi;
      }
    }
  }
};

}  // namespace lgs
