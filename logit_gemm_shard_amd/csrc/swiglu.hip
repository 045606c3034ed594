// One tensor-parallel rank's SwiGLU MLP shard, forward and backward.
//
// The mohashari.github.io page on tensor parallelism for fine-tuning 70B
// models with Megatron-LM, section "The MLP Block": the gate and up
// weights are split by columns, the down weight by rows; rank i computes
// Y_i = Swish(X W_gate,i) * (X W_up,i) and the partial Z_i = Y_i W_down,i,
// and one all-reduce sums the partials.  The backward is the chain rule
// through those equations: dZ reaches every rank unchanged, dX_i is a
// partial, as in the GeLU block.
//
// Operand layouts (row-major, explicit leading dimensions), f = ffn / t:
//   X [M, h]; W_gu = [W_gate,i | W_up,i] [h, 2f]; W_down,i [f, h];
//   GU = [G | U] and dGU = [dG | dU] [M, 2f]; Y [M, f]; Z, dZ, dX [M, h];
//   dW_gu [h, 2f] (same split as W_gu); dW_down [f, h].
// Products:
//   [G | U] = X W_gu    : one paired GEMM (N = 2f), the epilogue forms Y
//   Z   = Y W_down      : Y K-contiguous, W_down N-contiguous
//   dY  = dZ W_down^T   : both K-contiguous; the epilogue reads G, U
//   dX  = dGU W_gu^T    : both K-contiguous, K = 2f
//   dW_gu = X^T dGU     : X M-contiguous (K = tokens), dGU N-contiguous
//   dW_down = Y^T dZ    : Y M-contiguous, dZ N-contiguous
#include "dispatch.hpp"
#include "epilogues.hpp"
#include "internal.hpp"

namespace lgs {

hipError_t swiglu_fwd(int M, int h, int f, const void* X, int64_t ldx, const void* Wgu,
                      int64_t ldwgu, const void* Wd, int64_t ldwd, void* GU, int64_t ldgu, void* Y,
                      int64_t ldy, void* Z, int64_t ldz, hipStream_t s) {
  const bf16 *x = (const bf16*)X, *wgu = (const bf16*)Wgu, *wd = (const bf16*)Wd;
  const EpiSwigluFwd e1{EpiPairStore<bf16>{(bf16*)GU, ldgu, M, f}, EpiStore<bf16>{(bf16*)Y, ldy, M, f}, f};
  hipError_t e = gemm_bf16<true, false, kPairedTiles>(pick_tile(M, 2 * f, kPairedTiles), x, ldx, wgu,
                                                      ldwgu, M, 2 * f, h, e1, s);
  if (e != hipSuccess) return e;
  EpiStore<bf16> e2{(bf16*)Z, ldz, M, h};
  return gemm_bf16<true, false>(pick_tile(M, h), (const bf16*)Y, ldy, wd, ldwd, M, h, f, e2, s);
}

hipError_t swiglu_bwd(int M, int h, int f, const void* X, int64_t ldx, const void* Wgu,
                      int64_t ldwgu, const void* Wd, int64_t ldwd, const void* GU, int64_t ldgu,
                      const void* dZ, int64_t lddz, void* dX, int64_t lddx, void* dWgu,
                      int64_t lddwgu, void* dWd, int64_t lddwd, void* Yws, void* dGUws,
                      hipStream_t s) {
  const bf16 *x = (const bf16*)X, *wgu = (const bf16*)Wgu, *wd = (const bf16*)Wd, *dz = (const bf16*)dZ;
  bf16 *y = (bf16*)Yws, *dgu = (bf16*)dGUws;
  const int f2 = 2 * f;  // scratch Y [M, f] and dGU [M, 2f] are dense
  // (the 256x320 tile would spill with this epilogue's inputs; not built)
  constexpr unsigned kTiles = kAllTiles & ~(1u << T256x320);
  const EpiSwigluBwd e1{(const bf16*)GU, ldgu, dgu, f2, y, f, M, f};
  hipError_t e = gemm_bf16<true, true, kTiles>(pick_tile(M, f, kTiles), dz, lddz, wd, ldwd, M, f, h, e1, s);
  if (e != hipSuccess) return e;
  // One grouped launch of the three products.  dX reduces over 2f, the two
  // weight gradients over the M tokens; the longer-K problem goes first so
  // that the later, shorter tiles fill the compute units it leaves free (at
  // the 70B shape 2f = 7168 against M = 4096).
  EpiStore<bf16> ex{(bf16*)dX, lddx, M, h};
  EpiStore<bf16> ew{(bf16*)dWgu, lddwgu, h, f2};
  EpiStore<bf16> ed{(bf16*)dWd, lddwd, f, h};
  if (f >= 256 && h >= 256 && M >= 256)
    return launch_gemm_pp_group3(pp_problem<256, 256, true, true>(dgu, f2, wgu, ldwgu, M, h, f2, ex),
                                 pp_problem<256, 256, false, false>(x, ldx, dgu, f2, h, f2, M, ew),
                                 pp_problem<256, 256, false, false>(y, f, dz, lddz, f, h, M, ed), s);
  return launch_gemm_pp_group3(pp_problem<128, 128, true, true>(dgu, f2, wgu, ldwgu, M, h, f2, ex),
                               pp_problem<128, 128, false, false>(x, ldx, dgu, f2, h, f2, M, ew),
                               pp_problem<128, 128, false, false>(y, f, dz, lddz, f, h, M, ed), s);
}

}  // namespace lgs
