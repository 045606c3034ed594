// Vocab-parallel cross-entropy backward for one rank's slice.
//
// The forward ("LIT-022: Megatron-LM ...", "Key takeaways") fuses the logit
// GEMM into the loss so ranks exchange O(b*s) numbers; the backward is the
// derivative of sum_k dloss_k * loss_k.  With the merged per-token log-sum-exp
// lse_k (from the same exchange) rank r needs nothing else from the others:
//
//   G_r  = (exp(z_r - lse) - onehot_r(y)) * dloss,   z_r = H E_r^T
//   dH_r = G_r E_r      [M, h]  (a partial: dH = sum_r dH_r)
//   dE_r = G_r^T H      [Vr, h] (rank r's rows of dE)
//
// The logits are recomputed by the same GEMM as the forward rather than
// stored by it; its epilogue turns them into G_r (bf16, the MFMA operand type
// of the two products that follow), and one grouped launch runs both
// products.  Operand orientations (no transposes):
//   z    = H E_r^T : H K-contiguous, E_r K-contiguous (row j is vocab entry j)
//   dH_r = G E_r   : G K-contiguous (K = Vr), E_r N-contiguous
//   dE_r = G^T H   : G M-contiguous (K = tokens), H N-contiguous
#include "dispatch.hpp"
#include "epilogues.hpp"
#include "internal.hpp"

namespace lgs {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// The row's values an 8-column chunk of G needs.
struct RowGrad {
  float lse_log2;  // lse_k * log2(e)
  float w;         // dloss_k
  int tg;          // target column within the slice (outside [0, Vr) if not here)
};

// acc = z; G = (exp(z - lse) - [col == target]) * w, rounded to bf16.
struct EpiXentGrad {
  static constexpr bool kDirect = false, kLoads = true;
  bf16* G;
  int64_t ldg;
  const float* lse;
  const float* w;  // may be null: 1 per token
  const int32_t* targets;
  int vocab_start, M, N;
  void debug_spans(int) const {
    LGS_NEED(G, debug::mat_bytes(M, ldg, N, 2), "EpiXentGrad G");
    LGS_NEED(lse, (size_t)M * 4, "EpiXentGrad lse");
    if (w) LGS_NEED(w, (size_t)M * 4, "EpiXentGrad dloss");
    LGS_NEED(targets, (size_t)M * 4, "EpiXentGrad targets");
  }
  __device__ __forceinline__ RowGrad load8(int m, int) const {
    if (m >= M) return RowGrad{0.f, 0.f, -1};
    return RowGrad{lse[m] * kLog2e, w ? w[m] : 1.f, targets[m] - vocab_start};
  }
  __device__ __forceinline__ void apply8(int m, int n, const float* z, RowGrad r) const {
    if (m >= M || n >= N) return;
    float g[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(z[i], kLog2e, -r.lse_log2));
      g[i] = (n + i == r.tg ? p - 1.0f : p) * r.w;
    }
    store_vec<8>(G + (int64_t)m * ldg + n, g);
  }
};

}  // namespace

size_t xent_bwd_scratch_bytes(int M, int Vr) { return (size_t)M * (size_t)Vr * 2u; }

hipError_t xent_bwd(int M, int h, int Vr, int vocab_start, const void* H, int64_t ldh,
                    const void* E, int64_t lde, const int32_t* targets, const float* lse,
                    const float* dloss, void* dH, int64_t lddh, void* dE, int64_t ldde,
                    void* scratch, hipStream_t s) {
  const bf16 *hh = (const bf16*)H, *e = (const bf16*)E;
  bf16* g = (bf16*)scratch;  // G [M, Vr], dense
  // The slice's columns in one launch or two (plan_columns, on the ping-pong
  // tiles): the second covers columns [c1, Vr) with its own tile, writing G
  // from column c1.
  const ColumnPlan plan = plan_columns(M, Vr, false, kPPTiles);
  const EpiXentGrad eg{g, Vr, lse, dloss, targets, vocab_start, M, plan.c1};
  hipError_t err = gemm_bf16<true, true>(plan.main, hh, ldh, e, lde, M, plan.c1, h, eg, s);
  if (err != hipSuccess) return err;
  if (plan.c1 < Vr) {
    const EpiXentGrad et{g + plan.c1, Vr, lse, dloss, targets, vocab_start + plan.c1, M, Vr - plan.c1};
    err = gemm_bf16<true, true>(plan.tail, hh, ldh, e + (int64_t)plan.c1 * lde, lde, M, Vr - plan.c1, h,
                                et, s);
    if (err != hipSuccess) return err;
  }
  // dE_r reduces over the M tokens, dH_r over the slice's Vr entries: the
  // longer K first.
  const EpiStore<bf16> ee{(bf16*)dE, ldde, Vr, h};
  const EpiStore<bf16> eh{(bf16*)dH, lddh, M, h};
  if (M >= 256 && Vr >= 256 && h >= 256) {
    if (M >= Vr)
      return launch_gemm_pp_group2(pp_problem<256, 256, false, false>(g, Vr, hh, ldh, Vr, h, M, ee),
                                   pp_problem<256, 256, true, false>(g, Vr, e, lde, M, h, Vr, eh), s);
    return launch_gemm_pp_group2(pp_problem<256, 256, true, false>(g, Vr, e, lde, M, h, Vr, eh),
                                 pp_problem<256, 256, false, false>(g, Vr, hh, ldh, Vr, h, M, ee), s);
  }
  return launch_gemm_pp_group2(pp_problem<128, 128, false, false>(g, Vr, hh, ldh, Vr, h, M, ee),
                               pp_problem<128, 128, true, false>(g, Vr, e, lde, M, h, Vr, eh), s);
}

}  // namespace lgs
