/*
 * lgs.h -- C ABI of liblgs.so: one tensor-parallel (TP) rank's shard of a
 * transformer block on an AMD Instinct MI355X (gfx950).
 *
 * The method (Megatron-LM 1D tensor parallelism) as the source pages state it:
 *   - "Tensor Parallelism and Pipeline Parallelism: Mathematical Foundations of
 *     Megatron-LM 1D Slicing, Sequence Parallelism, and 1F1B Scheduling"
 *     (llms.blog), sections "Column-Parallel Linear Layer", "Row-Parallel
 *     Linear Layer" and "Conjugate Communication Operators";
 *   - "Cutting a Model Into Pieces" (learn.kartikeya.me, lecture 3), section
 *     "Megatron-LM: cutting inside the layer": Y = GeLU(X A), Z = Y B, A split
 *     by columns, B by rows, one all-reduce per block;
 *   - "LIT-022: Megatron-LM: Training Multi-Billion Parameter Language Models
 *     Using Model Parallelism" (dmarx.github.io anthology), "Key takeaways":
 *     the parallel logit GEMM fused into the cross-entropy, the vocabulary
 *     padded so each rank's slice is a multiple of 128;
 *   - the mohashari.github.io page on tensor parallelism for fine-tuning 70B
 *     models with Megatron-LM, section "The MLP Block": the gated (SwiGLU)
 *     MLP of Llama-3 under the same column-then-row split.
 *
 * Conventions shared by every entry point
 *   - Shapes follow the pages: b (micro-batch), s (sequence length), h (hidden
 *     size), ffn (MLP inner width over all ranks), t (TP size), rank in [0, t),
 *     vocab (padded vocabulary over all ranks).  Tokens are the M = b*s rows of
 *     every activation (the pages' (s, b, h) tensor flattened; each operation
 *     here is per token, so the order of the rows is the caller's).
 *   - Matrices are row-major with an explicit leading dimension ld (elements
 *     between consecutive rows, ld >= row width).
 *   - Every pointer is a DEVICE pointer owned by the caller.  The library never
 *     allocates, frees or keeps a pointer after the call returns, never
 *     synchronizes, and keeps no mutable global state (one exception:
 *     vocab_parallel_xent_fwd_noalloc's static device scratch); calls on
 *     different streams with disjoint outputs may run concurrently.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued asynchronously on it; a device-side fault surfaces at the
 *     caller's next synchronization, as for any HIP launch.
 *   - dtype LGS_BF16: bf16 in and out, fp32 accumulation, outputs rounded to
 *     nearest-even.  LGS_F32: fp32 throughout.
 *   - Alignment: h and ffn/t must be multiples of 8; for LGS_BF16
 *     every matrix base pointer must be 16-byte aligned and every ld a multiple
 *     of 8 (the kernels move 16-byte vectors).  Token counts are unrestricted.
 *   - Errors are reported synchronously by the return value, before anything
 *     is enqueued, except LGS_ERR_HIP (the runtime rejected a launch; earlier
 *     launches of the same call may have run).  On any other non-zero return
 *     nothing was enqueued.  lgs_last_error() gives a
 *     thread-local message for the last failure on the calling thread.
 *   - Device data such as target ids is not validated (documented
 *     preconditions below).
 */
#ifndef LGS_H_
#define LGS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LGS_OK = 0,
  LGS_ERR_INVALID_ARG = 1, /* bad size, rank, leading dimension or NULL pointer */
  LGS_ERR_UNSUPPORTED = 2, /* dtype / activation / alignment not supported    */
  LGS_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the query       */
  LGS_ERR_HIP = 4          /* the HIP runtime rejected a launch                 */
} lgs_status;

typedef enum { LGS_F32 = 0, LGS_BF16 = 1 } lgs_dtype;

/* GeLU(u) = u * Phi(u) (ERF, the exact form) or its tanh approximation
   u/2 * (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))) (TANH). */
typedef enum { LGS_GELU_ERF = 0, LGS_GELU_TANH = 1 } lgs_gelu;

typedef enum { LGS_REDUCE_SUM = 0, LGS_REDUCE_XENT = 1, LGS_REDUCE_XENT_LSE = 2 } lgs_reduce_op;

/* Library version as major*10000 + minor*100 + patch. */
int lgs_version(void);

/* Static description of a status code; never NULL. */
const char* lgs_status_string(int status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* lgs_last_error(void);

/* ------------------------------------------------------------------------ */
/* Workspace queries: bytes of device scratch the matching call needs.       */
/* Return 0 when none is needed (or the arguments are invalid).              */

/* tp_mlp_fwd: 0 if the caller passes Y_i, else M * ffn/t * sizeof(dtype). */
size_t lgs_mlp_fwd_workspace_bytes(int b, int s, int h, int ffn, int t, int dtype, int y_given);
/* tp_mlp_bwd: room for the recomputed Y_i and for dU_i, both [M, ffn/t]. */
size_t lgs_mlp_bwd_workspace_bytes(int b, int s, int h, int ffn, int t, int dtype);
/* tp_swiglu_fwd: 0 if the caller passes Y_i, else M * ffn/t * 2 (bf16). */
size_t lgs_swiglu_fwd_workspace_bytes(int b, int s, int h, int ffn, int t, int dtype, int y_given);
/* tp_swiglu_bwd: room for the recomputed Y_i [M, ffn/t] and for dGU_i [M, 2 ffn/t]. */
size_t lgs_swiglu_bwd_workspace_bytes(int b, int s, int h, int ffn, int t, int dtype);
/* vocab_parallel_xent_fwd: per-token partials of each column slab of the slice. */
size_t lgs_xent_workspace_bytes(int b, int s, int h, int vocab, int t, int dtype);
/* vocab_parallel_xent_bwd: the slice's logit gradient G, M * vocab/t bf16. */
size_t lgs_xent_bwd_workspace_bytes(int b, int s, int h, int vocab, int t, int dtype);

/* ------------------------------------------------------------------------ */
/*
 * tp_mlp_fwd -- one rank's forward shard of the GeLU MLP block.
 *
 * "Mathematical Foundations of Megatron-LM", "Column-Parallel Linear Layer":
 * A = [A_1 ... A_t] split by columns, every rank holds the full input X (the
 * f operator is the identity forward), and the nonlinearity applies to each
 * column block independently.  "Row-Parallel Linear Layer": B = [B_1; ...; B_t]
 * split by rows, rank i computes the partial Z_i = Y_i B_i, and Z = sum_i Z_i
 * (the g all-reduce; on one device, shard_partial_sum).  With f = ffn / t:
 *
 *   U_i = X A_i      [M, f]   (stored only if U_i != NULL; saved for backward)
 *   Y_i = GeLU(U_i)  [M, f]   (stored in Y_i if given, else in the workspace)
 *   Z_i = Y_i B_i    [M, h]   (this rank's partial)
 *
 * X    [M, h]  ldx >= h     (replicated input)
 * A_i  [h, f]  lda >= f     (rank's column block: pass A + rank*f with lda = ffn
 *                            to use a full A [h, ffn])
 * B_i  [f, h]  ldb >= h     (rank's row block: B + rank*f*ldb of a full B [ffn, h])
 * U_i, Y_i [M, f], Z_i [M, h]: outputs, same dtype.  rank only validates.
 * Workspace: lgs_mlp_fwd_workspace_bytes(..., Y_i != NULL).
 */
int tp_mlp_fwd(int b, int s, int h, int ffn, int t, int rank, int dtype, int act,
               const void* X, int64_t ldx, const void* A_i, int64_t lda, const void* B_i,
               int64_t ldb, void* U_i, int64_t ldu, void* Y_i, int64_t ldy, void* Z_i,
               int64_t ldz, void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_mlp_bwd -- one rank's backward shard of the GeLU MLP block.
 *
 * "Mathematical Foundations of Megatron-LM", "Conjugate Communication
 * Operators": g* is the identity, so the same dZ [M, h] reaches every rank;
 * f* all-reduces the input gradient, so dX_i is a partial (dX = sum_i dX_i,
 * shard_partial_sum on one device).  The products are the chain rule through
 * the forward equations:
 *
 *   dY_i = dZ B_i^T,  dU_i = dY_i * GeLU'(U_i),  Y_i = GeLU(U_i) (recomputed)
 *   dB_i = Y_i^T dZ   [f, h]
 *   dA_i = X^T dU_i   [h, f]
 *   dX_i = dU_i A_i^T [M, h]
 *
 * Inputs X [M,h], A_i [h,f], B_i [f,h] as in tp_mlp_fwd; U_i [M, f] the saved
 * pre-activation; dZ [M, h].  Outputs dX_i, dA_i, dB_i (same dtype, each with
 * its ld).  dA_i / dB_i may point into full [h, ffn] / [ffn, h] gradients.
 * Workspace: lgs_mlp_bwd_workspace_bytes (holds Y_i and dU_i; for bf16 shapes
 * whose weight gradients are split over the tokens, also their fp32 partial
 * sums and per-tile counters, which the call clears itself).  Calls that share
 * one workspace must not overlap.
 */
int tp_mlp_bwd(int b, int s, int h, int ffn, int t, int rank, int dtype, int act,
               const void* X, int64_t ldx, const void* A_i, int64_t lda, const void* B_i,
               int64_t ldb, const void* U_i, int64_t ldu, const void* dZ, int64_t lddz,
               void* dX_i, int64_t lddx, void* dA_i, int64_t ldda, void* dB_i, int64_t lddb,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_swiglu_fwd -- one rank's forward shard of the SwiGLU (gated) MLP block.
 *
 * The mohashari.github.io page on tensor parallelism for fine-tuning 70B
 * models with Megatron-LM, section "The MLP Block": the block is
 * (Swish(X W_gate) * (X W_up)) W_down with * elementwise; W_gate and W_up are
 * split by columns, W_down by rows, and rank i computes
 *
 *   G_i = X W_gate,i,  U_i = X W_up,i                [M, f] each
 *   Y_i = Swish(G_i) * U_i, Swish(g) = g / (1 + exp(-g))      [M, f]
 *   Z_i = Y_i W_down,i                                [M, h] (this rank's partial)
 *
 * and Z = sum_i Z_i (one all-reduce; on one device, shard_partial_sum).
 * f = ffn / t, ffn the inner width of W_gate [h, ffn] over all ranks.
 *
 * X      [M, h]   ldx >= h      (replicated input)
 * Wgu_i  [h, 2f]  ldwgu >= 2f   (the rank's two column blocks side by side:
 *                                W_gate,i in columns [0, f), W_up,i in [f, 2f))
 * Wd_i   [f, h]   ldwd >= h     (the rank's row block of W_down [ffn, h])
 * GU_i   [M, 2f]: optional output (NULL: not stored), G_i in columns [0, f) and
 *                 U_i in [f, 2f): the pre-activations tp_swiglu_bwd takes.
 * Y_i    [M, f]:  optional output (NULL: kept in the workspace).
 * Z_i    [M, h]:  output.  dtype must be LGS_BF16 (else LGS_ERR_UNSUPPORTED).
 * Workspace: lgs_swiglu_fwd_workspace_bytes(..., Y_i != NULL).
 */
int tp_swiglu_fwd(int b, int s, int h, int ffn, int t, int rank, int dtype, const void* X,
                  int64_t ldx, const void* Wgu_i, int64_t ldwgu, const void* Wd_i, int64_t ldwd,
                  void* GU_i, int64_t ldgu, void* Y_i, int64_t ldy, void* Z_i, int64_t ldz,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_swiglu_bwd -- one rank's backward shard of the SwiGLU MLP block: the
 * chain rule through the equations of tp_swiglu_fwd, with dZ reaching every
 * rank unchanged and dX_i a partial (dX = sum_i dX_i), as for the GeLU block:
 *
 *   dY_i = dZ Wd_i^T
 *   dG_i = dY_i * U_i * Swish'(G_i),  dU_i = dY_i * Swish(G_i)
 *   Y_i  = Swish(G_i) * U_i                    (recomputed)
 *   dWd_i  = Y_i^T dZ                          [f, h]
 *   dWgu_i = X^T [dG_i | dU_i]                 [h, 2f] (gate, up side by side)
 *   dX_i   = dG_i W_gate,i^T + dU_i W_up,i^T   [M, h]
 *
 * Inputs X, Wgu_i, Wd_i as in tp_swiglu_fwd; GU_i [M, 2f] the saved [G_i | U_i];
 * dZ [M, h].  Outputs dX_i, dWgu_i, dWd_i (bf16, each with its ld).
 * Workspace: lgs_swiglu_bwd_workspace_bytes (holds Y_i and [dG_i | dU_i]).
 */
int tp_swiglu_bwd(int b, int s, int h, int ffn, int t, int rank, int dtype, const void* X,
                  int64_t ldx, const void* Wgu_i, int64_t ldwgu, const void* Wd_i, int64_t ldwd,
                  const void* GU_i, int64_t ldgu, const void* dZ, int64_t lddz, void* dX_i,
                  int64_t lddx, void* dWgu_i, int64_t lddwgu, void* dWd_i, int64_t lddwd,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_mlp_bwd_dgelu / tp_mlp_bwd_dx / tp_mlp_bwd_dw -- tp_mlp_bwd in three
 * parts, for callers that overlap the input gradient's exchange with the
 * weight gradients ("Conjugate Communication Operators": only dX_i goes
 * through f*'s all-reduce; dA_i and dB_i stay on the rank):
 *
 *   dgelu: dY_i = dZ B_i^T; dU_i = dY_i * GeLU'(U_i) and Y_i = GeLU(U_i) into
 *          the workspace
 *   dx:    dX_i = dU_i A_i^T                 (reads the workspace)
 *   dw:    dB_i = Y_i^T dZ, dA_i = X^T dU_i  (reads the workspace)
 *
 * Arguments as in tp_mlp_bwd; the three calls share one workspace of
 * lgs_mlp_bwd_workspace_bytes.  dx and dw may run in either order or
 * concurrently on different streams once dgelu has completed (the caller
 * orders them, e.g. with events).  tp_mlp_bwd runs dx and dw as one launch,
 * which is faster when nothing overlaps them.  Results: dgelu and dx give
 * tp_mlp_bwd's bits.  dw gives tp_mlp_bwd's bits where tp_mlp_bwd runs dB_i
 * and dA_i unsplit.  For some bf16 shapes tp_mlp_bwd splits their sums over
 * token ranges inside its launch (its workspace then exceeds the two [M, f]
 * buffers): both of them where the tokens are many against small h and f
 * (e.g. M = 2200, h = 1064, f = 1048), or only the last dA_i tiles where its
 * launch would end in a partly filled round of long tiles (e.g. M = 4096,
 * h = 8192, f = 3584).  dw, which never splits, then equals it up to the
 * fp32 summation order of the split tiles.
 */
int tp_mlp_bwd_dgelu(int b, int s, int h, int ffn, int t, int rank, int dtype, int act,
                     const void* B_i, int64_t ldb, const void* U_i, int64_t ldu, const void* dZ,
                     int64_t lddz, void* workspace, size_t workspace_bytes, void* stream);
int tp_mlp_bwd_dx(int b, int s, int h, int ffn, int t, int rank, int dtype, const void* A_i,
                  int64_t lda, void* dX_i, int64_t lddx, void* workspace, size_t workspace_bytes,
                  void* stream);
int tp_mlp_bwd_dw(int b, int s, int h, int ffn, int t, int rank, int dtype, const void* X,
                  int64_t ldx, const void* dZ, int64_t lddz, void* dA_i, int64_t ldda, void* dB_i,
                  int64_t lddb, void* workspace, size_t workspace_bytes, void* stream);

/*
 * vocab_parallel_xent_fwd -- the fused vocab-parallel logit GEMM + cross-entropy
 * partials of one rank ("LIT-022: Megatron-LM ...", "Key takeaways": the
 * parallel logit GEMM is fused into the loss so ranks exchange O(b*s) numbers
 * rather than all-gathering b*s*vocab logits).
 *
 * Rank r owns the contiguous vocabulary rows [r*V_r, (r+1)*V_r), V_r = vocab/t.
 * With logits z = H E_r^T (never written to memory), per token k:
 *   m_r[k]      = max_j z[k, j]
 *   l_r[k]      = sum_j exp(z[k, j] - m_r[k])
 *   tgt_r[k]    = z[k, targets[k] - r*V_r] if the target is in the slice, else +0.0
 *   argmax_r[k] = global id of the slice's largest logit, lowest id on ties
 *                 (-1 if the row has no ordered value, e.g. all NaN); may be NULL
 *   loss[k]     = m_r + ln l_r - tgt_r, only for t == 1 (the full vocabulary);
 *                 must be NULL when t > 1 (merge ranks with shard_partial_sum)
 *
 * H [M, h] ldh >= h (bf16 hidden rows), E_r [V_r, h] lde >= h (the rank's rows
 * of the output embedding [vocab, h]: pass E + r*V_r*lde), targets [M] int32
 * global ids in [0, vocab) (precondition, not checked).  Outputs are fp32 / int32
 * [M] arrays.  dtype must be LGS_BF16.  Workspace: lgs_xent_workspace_bytes.
 */
int vocab_parallel_xent_fwd(int b, int s, int h, int vocab, int t, int rank, int dtype,
                            const void* H, int64_t ldh, const void* E_r, int64_t lde,
                            const int32_t* targets, float* m_r, float* l_r, float* tgt_r,
                            int32_t* argmax_r, float* loss, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * vocab_parallel_xent_fwd_noalloc -- vocab_parallel_xent_fwd for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, results and rules
 * as vocab_parallel_xent_fwd (the same kernels), without the workspace: the
 * slab partials go to a static device array of LGS_XENT_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that the library holds on each device it runs on until the
 * process ends.  The call allocates nothing (no hipMalloc, no allocating
 * library routine); its first call on a device looks up that device's copy
 * of the array once.
 *
 * Limit: lgs_xent_workspace_bytes(b, s, h, vocab, t, dtype) must not exceed
 * LGS_XENT_NOALLOC_SCRATCH_BYTES (e.g. 8192 tokens at vocab/t = 6400 need
 * 6 MiB; about 22,000 tokens fit at that slice width); larger calls return
 * LGS_ERR_UNSUPPORTED before anything is enqueued.
 *
 * Every call on one device shares that device's array, so calls that overlap
 * on one device (different streams, or different host threads) race: order
 * them on one stream, or use vocab_parallel_xent_fwd with separate
 * workspaces.  Nothing in the array needs clearing: each call writes every
 * entry it reads.
 */
#define LGS_XENT_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int vocab_parallel_xent_fwd_noalloc(int b, int s, int h, int vocab, int t, int rank, int dtype,
                                    const void* H, int64_t ldh, const void* E_r, int64_t lde,
                                    const int32_t* targets, float* m_r, float* l_r, float* tgt_r,
                                    int32_t* argmax_r, float* loss, void* stream);

/*
 * vocab_parallel_xent_bwd -- one rank's backward of the vocab-parallel
 * cross-entropy.  The pages give the forward ("LIT-022: Megatron-LM ...",
 * "Key takeaways"); this is the derivative of sum_k dloss[k] * loss[k].  With
 * the per-token log-sum-exp over the whole vocabulary, lse[k] = M* + ln L*
 * (shard_partial_sum(LGS_REDUCE_XENT_LSE) of the forward's partials), rank r
 * needs nothing else from the other ranks:
 *
 *   z       = H E_r^T                 (recomputed, never stored)
 *   G[k, j] = (exp(z[k, j] - lse[k]) - [j == targets[k] - r*V_r]) * dloss[k]
 *   dH_r    = G E_r     [M, h]        (a partial: dH = sum_r dH_r)
 *   dE_r    = G^T H     [V_r, h]      (rank r's rows of dE)
 *
 * H [M, h] ldh >= h and E_r [V_r, h] lde >= h as in vocab_parallel_xent_fwd;
 * targets [M] int32 global ids (precondition: in [0, vocab)); lse [M] fp32;
 * dloss [M] fp32 or NULL (1 for every token, the gradient of the summed loss;
 * pass 1/M per token for the mean).  Outputs dH_r, dE_r bf16, each with its
 * ld.  dtype must be LGS_BF16; h and vocab/t multiples of 8; G (M x V_r bf16)
 * under 2 GiB.  Workspace: lgs_xent_bwd_workspace_bytes (holds G, bf16).
 */
int vocab_parallel_xent_bwd(int b, int s, int h, int vocab, int t, int rank, int dtype,
                            const void* H, int64_t ldh, const void* E_r, int64_t lde,
                            const int32_t* targets, const float* lse, const float* dloss,
                            void* dH_r, int64_t lddh, void* dE_r, int64_t ldde, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * shard_partial_sum -- the one-device stand-in for the exchanges of the path.
 *
 * LGS_REDUCE_SUM: out[j] = sum_{r=0}^{t-1} parts[r*part_stride + j], j < n,
 *   accumulated in fp32 in ascending r (deterministic).  The g all-reduce of
 *   the row-parallel exit (Z = sum_i Z_i, "Row-Parallel Linear Layer") and the
 *   f* all-reduce of the input gradient (dX = sum_i dX_i).  in_dtype / out_dtype
 *   each LGS_F32 or LGS_BF16.  Each rank's block is n dense elements.
 * LGS_REDUCE_XENT: merge of the ranks' cross-entropy partials.  parts is fp32;
 *   rank r's block at parts + r*part_stride holds m_r[n], l_r[n], tgt_r[n]
 *   back to back (part_stride >= 3n).  out[j] (fp32) = M* + ln L* - sum_r tgt_r
 *   with M* = max_r m_r and L* = sum_r l_r exp(m_r - M*): the log-sum-exp
 *   identity, equal to the full-vocabulary loss.  Both dtypes must be LGS_F32.
 * LGS_REDUCE_XENT_LSE: the same merge's log-sum-exp alone, out[j] = M* + ln L*
 *   (the lse that vocab_parallel_xent_bwd takes).  Rank blocks as for
 *   LGS_REDUCE_XENT (tgt_r is not read); part_stride >= 2n.
 * `out` must not overlap `parts`.
 */
int shard_partial_sum(int op, int t, int64_t n, int in_dtype, int out_dtype, const void* parts,
                      int64_t part_stride, void* out, void* stream);

/*
 * Attention projections of one rank ("Mathematical Foundations of
 * Megatron-LM", "Self-Attention Layer Decomposition"; the mohashari.github.io
 * 70B page, "The Multi-Head Attention Block"): W_Q, W_K, W_V are split by
 * columns so rank i holds whole heads, n_q/t query heads and n_kv/t key/value
 * heads of head_dim d (grouped-query attention: query head k uses KV head
 * k / (n_q/n_kv)); W_O is split by rows so rank i's product is a partial
 * (Z = sum_i Z_i, one all-reduce; on one device shard_partial_sum).  The
 * attention core on the rank's heads runs between the two projections and is
 * not part of this library.  With q = (n_q/t) d and kv = (n_kv/t) d:
 *
 *   tp_attn_qkv_fwd: QKV_i = X Wqkv_i                      [M, q + 2 kv]
 *   tp_attn_qkv_bwd: dX_i = dQKV_i Wqkv_i^T (a partial)    [M, h]
 *                    dWqkv_i = X^T dQKV_i                  [h, q + 2 kv]
 *   tp_attn_out_fwd: Z_i = A_i Wo_i (a partial)            [M, h]
 *   tp_attn_out_bwd: dA_i = dZ Wo_i^T, dWo_i = A_i^T dZ    [M, q], [q, h]
 *
 * X [M, h]; Wqkv_i [h, q + 2 kv] = [W_Q^i | W_K^i | W_V^i], the rank's heads'
 * columns side by side (head k of Q in columns [k d, (k+1) d) of W_Q);
 * QKV_i and dQKV_i [M, q + 2 kv] in the same order; A_i [M, q] the rank's
 * heads' outputs side by side; Wo_i [q, h] rows [i q, (i+1) q) of W_O.  Every
 * matrix row-major with its ld.  dtype must be LGS_BF16; h and head_dim
 * multiples of 8; n_q and n_kv divisible by t, n_q by n_kv.
 *
 * Workspace (tp_attn_qkv_fwd and tp_attn_out_bwd, optional): when the
 * rank's QKV product, or the dA_i product of the output projection's
 * backward, has few output tiles and a long K (= h), a workspace of the
 * queried size (256-byte aligned) lets it run split over K (fp32 partials,
 * then summed into the bf16 output); NULL, or a smaller one, runs it unsplit
 * with the same result up to fp32 summation order.  The queries return 0 when
 * no split applies.  tp_attn_qkv_bwd and tp_attn_out_fwd take none.
 */
size_t lgs_attn_qkv_fwd_workspace_bytes(int b, int s, int h, int n_q_heads, int n_kv_heads,
                                        int head_dim, int t, int dtype);
size_t lgs_attn_out_bwd_workspace_bytes(int b, int s, int h, int n_q_heads, int head_dim, int t,
                                        int dtype);
int tp_attn_qkv_fwd(int b, int s, int h, int n_q_heads, int n_kv_heads, int head_dim, int t,
                    int rank, int dtype, const void* X, int64_t ldx, const void* Wqkv_i,
                    int64_t ldw, void* QKV_i, int64_t ldqkv, void* workspace,
                    size_t workspace_bytes, void* stream);
int tp_attn_qkv_bwd(int b, int s, int h, int n_q_heads, int n_kv_heads, int head_dim, int t,
                    int rank, int dtype, const void* X, int64_t ldx, const void* Wqkv_i,
                    int64_t ldw, const void* dQKV_i, int64_t lddqkv, void* dX_i, int64_t lddx,
                    void* dWqkv_i, int64_t lddw, void* stream);
int tp_attn_out_fwd(int b, int s, int h, int n_q_heads, int head_dim, int t, int rank, int dtype,
                    const void* A_i, int64_t lda, const void* Wo_i, int64_t ldwo, void* Z_i,
                    int64_t ldz, void* stream);
int tp_attn_out_bwd(int b, int s, int h, int n_q_heads, int head_dim, int t, int rank, int dtype,
                    const void* A_i, int64_t lda, const void* Wo_i, int64_t ldwo, const void* dZ,
                    int64_t lddz, void* dA_i, int64_t ldda, void* dWo_i, int64_t lddwo,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * shard_reduce_scatter / shard_all_gather -- one-device stand-ins for the
 * sequence-parallel exit and entry ("Mathematical Foundations of Megatron-LM",
 * "Sequence Parallelism", "Splitting All-Reduce into Reduce-Scatter and
 * All-Gather").  The row-parallel exit's all-reduce becomes a reduce-scatter
 * that sums the t partials and leaves rank r only its s/t chunk of the
 * sequence; LayerNorm, dropout and the residual then run on (s/t, b, h); an
 * all-gather rebuilds (s, b, h) before the next column-parallel GEMM.  Both
 * halves together move what the all-reduce moves.
 *
 * Token rows are the pages' (s, b) order flattened s-outermost (row
 * s_idx * b + b_idx of an [s*b, h] matrix), so rank r's chunk is the
 * contiguous rows [r*(s/t)*b, (r+1)*(s/t)*b).  s must be divisible by t.
 *
 * shard_reduce_scatter: out[j] = sum_{i<t} parts[i*part_stride + r*c + j],
 *   j < c = (s/t)*b*h, accumulated in fp32 in ascending i (the same bits as
 *   the matching rows of shard_partial_sum(LGS_REDUCE_SUM)).  Each part is a
 *   dense [s*b, h]; part_stride >= s*b*h.  in_dtype / out_dtype each LGS_F32
 *   or LGS_BF16.
 * shard_all_gather: out[q*c + j] = shards[q*shard_stride + j] for q < t,
 *   j < c: the dense [s*b, h] tensor from the t chunks, rank order along s.
 *   shard_stride >= c.  A copy (dtype in = out).
 * `out` must not overlap the inputs.
 */
int shard_reduce_scatter(int t, int rank, int s, int b, int h, int in_dtype, int out_dtype,
                         const void* parts, int64_t part_stride, void* out, void* stream);
int shard_all_gather(int t, int s, int b, int h, int dtype, const void* shards,
                     int64_t shard_stride, void* out, void* stream);

/*
 * shard_reduce_scatter_layernorm -- the sequence-parallel region between the
 * two halves, fused with the reduce-scatter ("Mathematical Foundations of
 * Megatron-LM", "Sequence Parallelism": LayerNorm, the residual addition and
 * dropout run locally on the rank's (s/t, b, h) chunk).  For every row j of
 * rank r's chunk (rows as for shard_reduce_scatter):
 *
 *   z_j  = sum_{i<t} parts[i*part_stride + (r*(s/t)*b + j)*h + (0..h-1)]
 *          (fp32, ascending i: the bits shard_reduce_scatter sums to)
 *   d_j  = keep ? (keep[j*h + c] != 0 ? z_j[c] * keep_scale : 0) : z_j[c]
 *   hs_j = residual_j + d_j                      -> hs   [(s/t)*b, h] bf16
 *   y_j  = (hs_j - mean) / sqrt(var + eps) * gamma + beta
 *                                                -> y    [(s/t)*b, h] bf16
 *
 * with mean and the biased (1/h) variance of the row's fp32 hs_j (before its
 * rounding to bf16) over the h features.  Readings: dropout acts on the
 * block's output before the residual add and LayerNorm is the next
 * sub-layer's, applied after it; the keep mask is an input (one byte per
 * element, non-zero = keep; NULL = no dropout), keep_scale normally 1/(1-p).
 *
 * dtype must be LGS_BF16 (else LGS_ERR_UNSUPPORTED); parts as for
 * shard_reduce_scatter (part_stride >= s*b*h and a multiple of 8 when
 * t > 1); residual, hs, y dense [(s/t)*b, h]; gamma, beta [h]; all 16-byte
 * aligned, keep 8-byte aligned.  h must be a multiple of 8 and at most 16384
 * (LGS_ERR_UNSUPPORTED otherwise); eps > 0 and finite.  hs and y must not
 * overlap the inputs or each other.
 */
int shard_reduce_scatter_layernorm(int t, int rank, int s, int b, int h, int dtype, const void* parts,
                                   int64_t part_stride, const void* residual, const uint8_t* keep,
                                   float keep_scale, const void* gamma, const void* beta, float eps,
                                   void* hs, void* y, void* stream);

/*
 * shard_layernorm_bwd -- the backward of shard_reduce_scatter_layernorm's
 * region on rank r's rows, from dy (the gradient of y) and dhs (the gradient
 * later layers send back along the residual stream; NULL = none).  LayerNorm's
 * statistics are recomputed from the stored hs (bf16).  Per row j:
 *
 *   xhat  = (hs_j - mean) / sqrt(var + eps),   dxhat = dy_j * gamma
 *   g_j   = (dxhat - mean_h(dxhat) - xhat * mean_h(dxhat * xhat))
 *           / sqrt(var + eps) + dhs_j            -> g  [(s/t)*b, h] bf16
 *           (the gradient of hs, which is also the residual input's)
 *   dz_j  = keep ? (keep[j*h + c] != 0 ? g_j[c] * keep_scale : 0) : g_j[c]
 *                                                -> dz [(s/t)*b, h] bf16
 *           (the gradient of the rank's rows of sum_i Z_i: in the backward
 *           the all-gather of the t ranks' dz feeds the row-parallel GEMM)
 *   dgamma = sum_j dy_j * xhat,  dbeta = sum_j dy_j   -> [h] fp32 each
 *           (the rank's rows only: the ranks' sums add up to the whole's)
 *
 * The column sums go through fp32 partials in the workspace
 * (lgs_layernorm_bwd_workspace_bytes, 16-byte aligned) and are added in a
 * fixed order.  Same dtype, alignment and h rules as the forward; eps must be
 * the forward's.  Outputs must not overlap the inputs or each other.
 */
size_t lgs_layernorm_bwd_workspace_bytes(int t, int s, int b, int h, int dtype);
int shard_layernorm_bwd(int t, int rank, int s, int b, int h, int dtype, const void* hs, const void* dy,
                        const void* dhs, const uint8_t* keep, float keep_scale, const void* gamma, float eps,
                        void* g, void* dz, float* dgamma, float* dbeta, void* workspace, size_t workspace_bytes,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LGS_H_ */
