// Internal launchers behind the C ABI.  Arguments are already validated;
// every function only enqueues kernels on `s` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lgs {

// One rank's MLP shard forward.  M tokens, h hidden, f = ffn / t columns.
//   U = X A_i (stored if U != null), Y = GeLU(U), Z = Y B_i.
hipError_t mlp_fwd(bool bf16, int M, int h, int f, int act, const void* X, int64_t ldx,
                   const void* A, int64_t lda, const void* B, int64_t ldb, void* U, int64_t ldu,
                   void* Y, int64_t ldy, void* Z, int64_t ldz, hipStream_t s);

// One rank's MLP shard backward from the saved X and U and the incoming dZ.
//   dY = dZ B_i^T, dU = dY * GeLU'(U), Y = GeLU(U)  (Y, dU in scratch)
//   dB_i = Y^T dZ, dA_i = X^T dU, dX_i = dU A_i^T
//   splitws: partial sums and counters of the K-split dB / dA (bf16 only,
//   mlp_bwd_split_bytes of them; may be null when that is 0).
hipError_t mlp_bwd(bool bf16, int M, int h, int f, int act, const void* X, int64_t ldx,
                   const void* A, int64_t lda, const void* B, int64_t ldb, const void* U,
                   int64_t ldu, const void* dZ, int64_t lddz, void* dX, int64_t lddx, void* dA,
                   int64_t ldda, void* dB, int64_t lddb, void* Yws, void* dUws, void* splitws,
                   hipStream_t s);

// How the bf16 backward's grouped launch splits dB and dA over K (the
// tokens): parts (1 = not split) of kchunk K rows each, over every dB and dA
// tile (tail == 0, `tiles` = their count) or over the last `tail` dA tiles
// only (tiles == tail).
struct BwdSplit {
  int parts, kchunk, tiles, tail;
};
BwdSplit mlp_bwd_wsplit(int M, int h, int f);
size_t mlp_bwd_split_bytes(int M, int h, int f);  // 0 when not split

// The same backward in three parts: dgelu (dY, dU = dY GeLU'(U), Y into
// scratch), then dx (dX_i = dU A_i^T) and dw (dB_i = Y^T dZ, dA_i = X^T dU),
// independent of each other.
hipError_t mlp_bwd_dgelu(bool bf16, int M, int h, int f, int act, const void* B, int64_t ldb,
                         const void* U, int64_t ldu, const void* dZ, int64_t lddz, void* Yws,
                         void* dUws, hipStream_t s);
hipError_t mlp_bwd_dx(bool bf16, int M, int h, int f, const void* A, int64_t lda, const void* dUws,
                      void* dX, int64_t lddx, hipStream_t s);
hipError_t mlp_bwd_dw(bool bf16, int M, int h, int f, const void* X, int64_t ldx, const void* dZ,
                      int64_t lddz, const void* Yws, const void* dUws, void* dA, int64_t ldda,
                      void* dB, int64_t lddb, hipStream_t s);

// One rank's SwiGLU MLP shard (bf16).  f = ffn / t; W_gu = [W_gate,i | W_up,i].
//   [G | U] = X W_gu (stored if GU != null), Y = Swish(G) * U, Z = Y W_down,i.
hipError_t swiglu_fwd(int M, int h, int f, const void* X, int64_t ldx, const void* Wgu,
                      int64_t ldwgu, const void* Wd, int64_t ldwd, void* GU, int64_t ldgu, void* Y,
                      int64_t ldy, void* Z, int64_t ldz, hipStream_t s);
//   dY = dZ W_down^T; dG = dY * U * Swish'(G), dU = dY * Swish(G), Y recomputed
//   (Y, dGU in scratch); dX = dGU W_gu^T, dW_gu = X^T dGU, dW_down = Y^T dZ.
hipError_t swiglu_bwd(int M, int h, int f, const void* X, int64_t ldx, const void* Wgu,
                      int64_t ldwgu, const void* Wd, int64_t ldwd, const void* GU, int64_t ldgu,
                      const void* dZ, int64_t lddz, void* dX, int64_t lddx, void* dWgu,
                      int64_t lddwgu, void* dWd, int64_t lddwd, void* Yws, void* dGUws,
                      hipStream_t s);

// One rank's attention projections (bf16): nqkv = (n_q + 2 n_kv) d / t
// columns of [Q | K | V], hq = n_q d / t columns of the heads' outputs.
// Split-K schedule of the QKV projection: the parts (0 = unsplit) and the
// scratch their in-launch reduction needs (fp32 slots and counters); the
// projection runs unsplit when scratch is null.
int attn_qkv_splits(int M, int h, int nqkv);
size_t attn_qkv_scratch_bytes(int M, int h, int nqkv);
hipError_t attn_qkv_fwd(int M, int h, int nqkv, const void* X, int64_t ldx, const void* W,
                        int64_t ldw, void* QKV, int64_t ldqkv, void* scratch, hipStream_t s);
hipError_t attn_out_fwd(int M, int hq, int h, const void* A, int64_t lda, const void* Wo,
                        int64_t ldwo, void* Z, int64_t ldz, hipStream_t s);
hipError_t attn_qkv_bwd(int M, int h, int nqkv, const void* X, int64_t ldx, const void* W,
                        int64_t ldw, const void* dQKV, int64_t lddqkv, void* dX, int64_t lddx,
                        void* dW, int64_t lddw, hipStream_t s);
// The output projection's backward splits dA's K in two (reduced inside the
// launch: fp32 slots and counters in scratch) when that fills the chip;
// unsplit when scratch is null.
bool attn_out_bwd_split(int M, int hq, int h);
size_t attn_out_bwd_scratch_bytes(int M, int hq, int h);
hipError_t attn_out_bwd(int M, int hq, int h, const void* A, int64_t lda, const void* Wo,
                        int64_t ldwo, const void* dZ, int64_t lddz, void* dA, int64_t ldda,
                        void* dWo, int64_t lddwo, void* scratch, hipStream_t s);

// Fused logit GEMM + CE partials for one vocabulary slice of Vr rows.
size_t xent_scratch_bytes(int M, int Vr);
hipError_t xent_fwd(int M, int h, int Vr, int vocab_start, const void* H, int64_t ldh,
                    const void* E, int64_t lde, const int32_t* targets, float* m_r, float* l_r,
                    float* t_r, int32_t* argmax_r, float* loss, void* scratch, hipStream_t s);

// The allocation-free variant's slab partials: a file-scope device array of
// kXentStaticScratchBytes per device (xent.hip), resolved to its address on
// the device that runs stream `s` (looked up once per device, then cached).
constexpr size_t kXentStaticScratchBytes = (size_t)16 << 20;
hipError_t xent_static_scratch(hipStream_t s, void** out);

// CE backward for one vocabulary slice: G = (exp(z - lse) - onehot) * dloss
// (z = H E_r^T recomputed, G in bf16 scratch [M, Vr]), dH_r = G E_r,
// dE_r = G^T H.  dloss may be null (1 per token).
size_t xent_bwd_scratch_bytes(int M, int Vr);
hipError_t xent_bwd(int M, int h, int Vr, int vocab_start, const void* H, int64_t ldh,
                    const void* E, int64_t lde, const int32_t* targets, const float* lse,
                    const float* dloss, void* dH, int64_t lddh, void* dE, int64_t ldde,
                    void* scratch, hipStream_t s);

// Sum of t partials (fp32 accumulate, ascending rank order) or the CE merge.
hipError_t partial_sum(int t, int64_t n, bool in_bf16, bool out_bf16, const void* parts,
                       int64_t stride, void* out, hipStream_t s);
// Sequence-parallel stand-ins: rank's chunk of the sum (chunk elements at
// offset rank * chunk of every part), and the copy of t chunks into place.
hipError_t reduce_scatter(int t, int64_t chunk, int rank, bool in_bf16, bool out_bf16,
                          const void* parts, int64_t stride, void* out, hipStream_t s);
hipError_t all_gather(int t, int64_t chunk, bool bf16, const void* shards, int64_t stride,
                      void* out, hipStream_t s);
// The sequence-parallel region of rank r's `rows` rows (bf16): the sum of the
// t partials' rows (rank r's chunk of each), dropout with the keep mask (if
// any), the residual add (hs) and LayerNorm over h (y).  h <= rs_layernorm_max_h().
int rs_layernorm_max_h();
// Its backward on `rows` rows (bf16): g = dhs + LayerNorm's dx at hs, dz = the
// masked and scaled g, and the rows' dgamma, dbeta (fp32; column partials of
// layernorm_bwd_scratch_bytes in scratch, then summed in order).
size_t layernorm_bwd_scratch_bytes(int rows, int h);
hipError_t layernorm_bwd(int rows, int h, const void* hs, const void* dy, const void* dhs, const uint8_t* keep,
                         float keep_scale, const void* gamma, float eps, void* g, void* dz, float* dgamma,
                         float* dbeta, void* scratch, hipStream_t s);
hipError_t rs_layernorm(int t, int rows, int h, int rank, const void* parts, int64_t stride,
                        const void* residual, const uint8_t* keep, float keep_scale, const void* gamma,
                        const void* beta, float eps, void* hs, void* y, hipStream_t s);
hipError_t xent_rows(int M, int Vr, int vocab_start, const void* Z, int64_t ldz,
                     const int32_t* targets, float* m, float* l, float* t, hipStream_t s);
hipError_t xent_combine(int t, int64_t n, const float* parts, int64_t stride, bool lse_only,
                        float* loss, hipStream_t s);

// Matrix-core rate: `blocks` workgroups of `waves` waves, each running
// 64 iters8 MFMAs per accumulator chain on register operands (ops: 16 x 64
// lanes x 8 bf16); accumulators to out (mfma_rate_out_floats floats), each
// wave's shader-clock and 100 MHz reference counts to clocks (2 per wave).
size_t mfma_rate_out_floats(int blocks, int waves);
hipError_t mfma_rate(int blocks, int waves, int iters8, const void* ops, float* out, uint64_t* clocks,
                     hipStream_t s);

// The bf16 GEMM core with a store epilogue and an explicit tile (-1: picked).
int num_tiles();
bool tile_shape(int tile, int* bm, int* bn);
int picked_tile(int M, int N);
hipError_t gemm_store_bf16(int tile, bool a_kmajor, bool b_kmajor, int M, int N, int K,
                           const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                           int64_t ldc, hipStream_t s);

}  // namespace lgs
