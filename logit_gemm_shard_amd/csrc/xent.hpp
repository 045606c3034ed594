// Fused vocab-parallel cross-entropy: the logit GEMM's epilogue reduces each
// row of the wave's logit tile to (max, sum of exp relative to that max,
// target logit, first argmax) and writes those four numbers per row and per
// wave column-slab.  Logits never leave the chip: the reductions read them
// from the matrix cores' accumulator registers.  A small merge kernel
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
  int32_t* idx;  // [slabs][M] slice-local column of the slab's first maximum (may be null)
};

// One launch covers columns [col0, col0 + N) of the rank's slice (the whole
// slice, or one of the column ranges a launch plan splits it into); its
// slabs are numbered from slab0.
struct EpiXent {
  static constexpr bool kDirect = true;
  XentSlabs s;
  const int32_t* targets;  // [M] global vocabulary ids
  int vocab_start;         // global id of this launch's column 0 (slice start + col0)
  int M, N;                // tokens, columns of this launch
  int WN;                  // wave tile width: slab = slab0 + wave column
  int col0, slab0;         // slice-local column of this launch's column 0; its first slab

  // A launch of tile width bn writes slabs [slab0, slab0 + ceil(N / bn) bn / WN)
  // of every plane (a wave column wholly past N writes -inf / 0 partials).
  void debug_spans(int bn) const {
    const size_t slabs = (size_t)((N + bn - 1) / bn) * bn / WN, bytes = slabs * M * 4;
    LGS_CHECK(bn % WN == 0);
    LGS_NEED(s.m + (int64_t)slab0 * M, bytes, "EpiXent slab maxima");
    LGS_NEED(s.l + (int64_t)slab0 * M, bytes, "EpiXent slab sums");
    LGS_NEED(s.t + (int64_t)slab0 * M, bytes, "EpiXent slab targets");
    if (s.idx) LGS_NEED(s.idx + (int64_t)slab0 * M, bytes, "EpiXent slab argmax");
    LGS_NEED(targets, (size_t)M * 4, "EpiXent targets");
  }

  // Reduces the wave's logit tile straight from the accumulators.  In the
  // 32x32 MFMA output layout lane l holds, for row 32i + l%32 of the wave
  // tile, the 16 TN columns 32j + 8q + 4(l/32) + e (j < TN, q < 4, e < 4) in
  // acc[i][j][4q + e]: every row is split over lanes l and l ^ 32.  Each lane
  // reduces its half and the pair combines through one lane exchange.
  template <int TM, int TN, int WNt>
  __device__ __forceinline__ void direct(f32x16 (&acc)[TM][TN], int mb, int nb, int lane) const {
    const int cb = nb + 4 * (lane >> 5);  // this launch's column of acc[.][0][0]
    if (N - nb < WNt) {
      // Last wave column of the launch: columns past its end become -inf,
      // which neither wins the max nor adds to the sum.
      const int left = N - cb;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * j + 8 * (r >> 2) + (r & 3) >= left) acc[i][j][r] = -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) row_tile<TN>(acc[i], mb + 32 * i + (lane & 31), nb, cb, lane);
  }

  template <int TN>
  __device__ __forceinline__ void row_tile(const f32x16 (&a)[TN], int m, int nb, int cb,
                                           int lane) const {
    int tl = -0x40000000;  // target column relative to cb; far below 0 if not in this launch
    if (m < M) {
      const int tg = targets[m] - vocab_start;
      if (tg >= 0 && tg < N) tl = tg - cb;
    }
    // Row maximum over both halves (NaNs never win: a NaN row stays NaN
    // through its sum).
    float best = -INFINITY;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) best = __builtin_fmaxf(best, a[j][r]);
    best = __builtin_fmaxf(best, __shfl_xor(best, 32));
    // Sum of exponentials relative to the row maximum, and the target logit.
    // A row with no finite maximum (only -inf entries, e.g. a wave column
    // wholly past the slice end) is shifted by 0 so that they add exp(-inf) = 0.
    const float shift = (best == -INFINITY ? 0.f : best) * 1.4426950408889634f;
    float sum = 0.f, tv = 0.f;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(fmaf(a[j][r], 1.4426950408889634f, -shift));
    // The target pick runs only where some row of the wave has its target in
    // this wave's columns (about one row tile in ten at V_r = 6400).
    if (__any(tl >= -4 && tl < 32 * TN)) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) tv = 32 * j + 8 * (r >> 2) + (r & 3) == tl ? a[j][r] : tv;
    }
    sum += __shfl_xor(sum, 32);
    tv += __shfl_xor(tv, 32);
    // First column holding the maximum: each lane walks its columns from the
    // last to the first, so the lowest match survives; then the pair keeps
    // the lower of the two.
    int bi = 0x7fffffff;
    if (s.idx) {
      int bc = -1;
      if (best > -INFINITY) {
#pragma unroll
        for (int j = TN - 1; j >= 0; --j)
#pragma unroll
          for (int r = 15; r >= 0; --r)
            bc = a[j][r] == best ? 32 * j + 8 * (r >> 2) + (r & 3) : bc;
      }
      bi = bc < 0 ? 0x7fffffff : col0 + cb + bc;  // slice-local column
      bi = min(bi, __shfl_xor(bi, 32));
    }
    if (lane < 32 && m < M) {
      const int64_t o = (int64_t)(slab0 + nb / WN) * M + m;
      s.m[o] = best;
      s.l[o] = sum;
      s.t[o] = tv;
      if (s.idx) s.idx[o] = bi;
    }
  }
};

}  // namespace lgs
