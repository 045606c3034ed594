// One rank's attention projections under tensor parallelism.
//
// "Mathematical Foundations of Megatron-LM ..." (llms.blog), "Self-Attention
// Layer Decomposition", and the mohashari.github.io 70B page, "The
// Multi-Head Attention Block": Q, K and V are split by columns so rank i
// holds whole heads (n_q/t query and n_kv/t key/value heads), and the output
// projection W_O by rows so rank i's product is a partial that one
// all-reduce sums.  The attention core between the two runs on the rank's
// own heads and is not part of this library.
//
// Products (row-major operands, explicit leading dimensions):
//   QKV_i = X W_qkv,i     [M, nqkv]   X K-contiguous, W N-contiguous
//   Z_i   = A_i W_O,i     [M, h]      A_i K-contiguous, W_O,i N-contiguous
//   dX_i  = dQKV_i W_qkv,i^T [M, h]   both K-contiguous (K = nqkv)
//   dW_qkv,i = X^T dQKV_i [h, nqkv]   X M-contiguous (K = tokens), dQKV N-contiguous
//   dA_i  = dZ W_O,i^T    [M, hq]     both K-contiguous (K = h)
//   dW_O,i = A_i^T dZ     [hq, h]     A_i M-contiguous, dZ N-contiguous
// Each backward runs its two products in one grouped launch, the longer K
// first.
#include "dispatch.hpp"
#include "epilogues.hpp"
#include "internal.hpp"

namespace lgs {

namespace {

constexpr int kCUs = 256;

// C1 = A1 B1 (K-major A, K-major B: the input gradient) and C2 = A2^T B2
// (M-major A, N-major B: the weight gradient) in one launch.
hipError_t input_and_weight_grads(const bf16* a1, int64_t lda1, const bf16* b1, int64_t ldb1, int M1,
                                  int N1, int K1, const EpiStore<bf16>& e1, const bf16* a2, int64_t lda2,
                                  const bf16* b2, int64_t ldb2, int M2, int N2, int K2,
                                  const EpiStore<bf16>& e2, hipStream_t s) {
  const bool big = M1 >= 256 && N1 >= 256 && M2 >= 256 && N2 >= 256;
  if (big) {
    const auto p1 = pp_problem<256, 256, true, true>(a1, lda1, b1, ldb1, M1, N1, K1, e1);
    const auto p2 = pp_problem<256, 256, false, false>(a2, lda2, b2, ldb2, M2, N2, K2, e2);
    return K2 >= K1 ? launch_gemm_pp_group2(p2, p1, s) : launch_gemm_pp_group2(p1, p2, s);
  }
  const auto p1 = pp_problem<128, 128, true, true>(a1, lda1, b1, ldb1, M1, N1, K1, e1);
  const auto p2 = pp_problem<128, 128, false, false>(a2, lda2, b2, ldb2, M2, N2, K2, e2);
  return K2 >= K1 ? launch_gemm_pp_group2(p2, p1, s) : launch_gemm_pp_group2(p1, p2, s);
}

}  // namespace

// The QKV product is skinny (at the 70B shape 4096 x 1280 outputs: 80 tiles of
// 256x256 for 256 compute units) and deep (K = h = 8192).  Split-K fills the
// chip: every tile's K range in S parts, each an ordinary GEMM, reduced
// inside the launch (the last part of a tile to finish adds the parts' fp32
// partials in part order and stores the bf16 tile).  Used when the unsplit
// tiles would occupy at most half of the compute units and K is long enough
// for the parts to stay efficient.
namespace {
int qkv_kchunk(int h, int splits) { return ((h + splits - 1) / splits + 31) / 32 * 32; }
}  // namespace

int attn_qkv_splits(int M, int h, int nqkv) {
  if (M < 256 || nqkv < 256 || h < 2048) return 0;
  const int tiles = ((M + 255) / 256) * ((nqkv + 255) / 256);
  if (tiles > kCUs / 2) return 0;
  int splits = kCUs / tiles < 4 ? kCUs / tiles : 4;
  splits = (h + qkv_kchunk(h, splits) - 1) / qkv_kchunk(h, splits);
  return splits >= 2 ? splits : 0;
}

// K-split scratch of `tiles` 256x256 tiles in `parts` parts: one fp32 slot
// per tile and part, then one counter per tile.
static size_t split_slots_bytes(int tiles, int parts) { return (size_t)tiles * parts * 256 * 256 * sizeof(float); }
static size_t split_scratch_bytes(int tiles, int parts) {
  return parts ? split_slots_bytes(tiles, parts) + (size_t)tiles * sizeof(int) : 0;
}
static KSplit split_of(void* scratch, int tiles, int parts, int kchunk) {
  return KSplit{(float*)scratch, (int*)((char*)scratch + split_slots_bytes(tiles, parts)), parts, kchunk};
}

size_t attn_qkv_scratch_bytes(int M, int h, int nqkv) {
  const int tiles = ((M + 255) / 256) * ((nqkv + 255) / 256);
  return split_scratch_bytes(tiles, attn_qkv_splits(M, h, nqkv));
}

hipError_t attn_qkv_fwd(int M, int h, int nqkv, const void* X, int64_t ldx, const void* W,
                        int64_t ldw, void* QKV, int64_t ldqkv, void* scratch, hipStream_t s) {
  const int splits = attn_qkv_splits(M, h, nqkv);
  const EpiStore<bf16> e{(bf16*)QKV, ldqkv, M, nqkv};
  if (splits && scratch) {
    const auto p = pp_problem<256, 256, true, false>((const bf16*)X, ldx, (const bf16*)W, ldw, M, nqkv, h, e);
    return launch_gemm_pp_ksplit(p, split_of(scratch, p.tiles(), splits, qkv_kchunk(h, splits)), s);
  }
  return gemm_bf16<true, false>(pick_tile(M, nqkv), (const bf16*)X, ldx, (const bf16*)W, ldw, M, nqkv,
                                h, e, s);
}

hipError_t attn_out_fwd(int M, int hq, int h, const void* A, int64_t lda, const void* Wo,
                        int64_t ldwo, void* Z, int64_t ldz, hipStream_t s) {
  const EpiStore<bf16> e{(bf16*)Z, ldz, M, h};
  return gemm_bf16<true, false>(pick_tile(M, h), (const bf16*)A, lda, (const bf16*)Wo, ldwo, M, h, hq,
                                e, s);
}

hipError_t attn_qkv_bwd(int M, int h, int nqkv, const void* X, int64_t ldx, const void* W,
                        int64_t ldw, const void* dQKV, int64_t lddqkv, void* dX, int64_t lddx,
                        void* dW, int64_t lddw, hipStream_t s) {
  return input_and_weight_grads((const bf16*)dQKV, lddqkv, (const bf16*)W, ldw, M, h, nqkv,
                                EpiStore<bf16>{(bf16*)dX, lddx, M, h}, (const bf16*)X, ldx,
                                (const bf16*)dQKV, lddqkv, h, nqkv, M,
                                EpiStore<bf16>{(bf16*)dW, lddw, h, nqkv}, s);
}

// The output projection's backward at the 70B shape: dA (4096 x 1024, K =
// h = 8192) is 64 tiles and dW_O (1024 x 8192, K = 4096) 128, so one grouped
// launch leaves a quarter of the chip idle while the dA tiles, twice as long,
// finish.  Splitting dA's K in two makes 256 blocks of equal length; the two
// halves of a dA tile are reduced inside the launch.
bool attn_out_bwd_split(int M, int hq, int h) {
  if (M < 256 || hq < 256 || h < 4096 || h % 64 != 0) return false;
  const int ta = ((M + 255) / 256) * ((hq + 255) / 256);
  const int tw = ((hq + 255) / 256) * ((h + 255) / 256);
  return 2 * ta + tw <= kCUs && ta + tw < kCUs;
}

size_t attn_out_bwd_scratch_bytes(int M, int hq, int h) {
  const int ta = ((M + 255) / 256) * ((hq + 255) / 256);
  return split_scratch_bytes(ta, attn_out_bwd_split(M, hq, h) ? 2 : 0);
}

hipError_t attn_out_bwd(int M, int hq, int h, const void* A, int64_t lda, const void* Wo,
                        int64_t ldwo, const void* dZ, int64_t lddz, void* dA, int64_t ldda,
                        void* dWo, int64_t lddwo, void* scratch, hipStream_t s) {
  if (scratch && attn_out_bwd_split(M, hq, h)) {
    // dA = dZ W_O^T over K = h in two halves (both operands K-contiguous, so a
    // half is the operands moved by h/2 columns), and dW_O = A^T dZ.
    const bf16* dz = (const bf16*)dZ;
    const auto pa = pp_problem<256, 256, true, true>(dz, lddz, (const bf16*)Wo, ldwo, M, hq, h,
                                                     EpiStore<bf16>{(bf16*)dA, ldda, M, hq});
    const auto pw = pp_problem<256, 256, false, false>((const bf16*)A, lda, dz, lddz, hq, h, M,
                                                       EpiStore<bf16>{(bf16*)dWo, lddwo, hq, h});
    return launch_gemm_pp_group2_ksplit(pa, pw, split_of(scratch, pa.tiles(), 2, h / 2), s);
  }
  return input_and_weight_grads((const bf16*)dZ, lddz, (const bf16*)Wo, ldwo, M, hq, h,
                                EpiStore<bf16>{(bf16*)dA, ldda, M, hq}, (const bf16*)A, lda,
                                (const bf16*)dZ, lddz, hq, h, M,
                                EpiStore<bf16>{(bf16*)dWo, lddwo, hq, h}, s);
}

}  // namespace lgs
