/*
 * lgs_testing.h -- the bf16 GEMM core of liblgs.so exposed for tests and
 * tile-shape sweeps, with the measurement hooks of the benchmark.  Not part
 * of the method's interface (include/lgs.h); every entry point of lgs.h runs
 * on this core.
 *
 * Conventions as in lgs.h (device pointers owned by the caller, row-major with
 * leading dimensions, asynchronous on `stream`, status codes before launch).
 */
#ifndef LGS_TESTING_H_
#define LGS_TESTING_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of block-tile shapes the core is built with; tile ids are 0..n-1. */
int lgs_test_num_tiles(void);
/* Block tile of id `tile` (rows x cols of C per workgroup); -1 if no such id. */
int lgs_test_tile_shape(int tile, int* bm, int* bn);
/* The tile id the library picks for an M x N output. */
int lgs_test_pick_tile(int M, int N);

/*
 * C[M, N] = A B in bf16 (fp32 accumulation, round-to-nearest-even output) with
 * the block tile `tile` (-1: the library's choice).
 *   a_kmajor = 1: A is [M, K] row-major (element (m, k) at A[m*lda + k]);
 *   a_kmajor = 0: A is stored transposed, [K, M] (element (m, k) at A[k*lda + m]).
 *   b_kmajor = 1: B is stored transposed, [N, K] (element (k, n) at B[n*ldb + k]);
 *   b_kmajor = 0: B is [K, N] row-major (element (k, n) at B[k*ldb + n]).
 * Supported layout pairs (those the path uses): (1,0), (1,1), (0,0).
 * The contiguous dimension of each operand must be a multiple of 8 (K for a
 * K-major operand, M or N otherwise), as must N; 16-byte aligned bases, ld % 8 == 0.
 */
int lgs_test_gemm_bf16(int tile, int a_kmajor, int b_kmajor, int M, int N, int K, const void* A,
                       int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                       void* stream);

/*
 * The bf16 MLP backward's plan for the weight gradients of an M-token shard
 * with hidden size h and f = ffn/t columns: *parts = 1 when tp_mlp_bwd runs
 * dB_i and dA_i unsplit (then tp_mlp_bwd_dw, which never splits, gives the
 * same bits), else the number of token ranges it splits them into, with
 * *kchunk tokens per range.  *tail = 0 when every dB_i and dA_i tile is
 * split (or none), else the number of 256x256 dA_i tiles split, the last
 * ones launched; dB_i is then unsplit.  Returns 0, or -1 for non-positive
 * sizes.
 */
int lgs_test_mlp_bwd_plan(int M, int h, int f, int* parts, int* kchunk, int* tail);

/*
 * Streaming form of the cross-entropy slice partials, for measuring the CE
 * reductions against the HBM roofline (the product path fuses them into the
 * logit GEMM, vocab_parallel_xent_fwd, and never writes logits).  Z holds a
 * slice's logits, [M, Vr] bf16 row-major (ld ldz); per row it writes the
 * slice max m, the sum of exp(z - m) l, and the target logit T (targets are
 * global ids; T is +0.0 when targets[k] - vocab_start is outside [0, Vr)).
 * Vr must be a multiple of 8; Z 16-byte aligned, ldz % 8 == 0.
 */
int lgs_test_xent_rows_bf16(int M, int Vr, int vocab_start, const void* Z, int64_t ldz,
                            const int32_t* targets, float* m, float* l, float* T, void* stream);

/*
 * The matrix cores' bf16 rate with nothing else to run, the ceiling against
 * which the GEMM kernels' fractions of the spec peak are read.  Launches
 * `blocks` workgroups of `waves` wave64s (1..8); each wave loads 8 operand
 * pairs from `ops` (16 x 64 x 8 bf16: pair k is A_k at ops[(2k) * 512 + 8 lane
 * + e], B_k at ops[(2k+1) * 512 + 8 lane + e], in v_mfma_f32_32x32x16_bf16's
 * register layout) and runs 8 accumulator chains of 8 * iters8 MFMAs each,
 * chain c in step j multiplying A_{(c+j)%8} by B_c, so chain c ends holding
 * iters8 * (sum_k A_k) B_c.  Per wave: the chains' accumulators to `out`
 * (wave w's float (c * 16 + r) * 64 + lane at out[w * 8192 + ...]: element r
 * of lane `lane` of chain c), and to clocks[2w], clocks[2w+1] the shader clock
 * cycles (s_memtime) and 100 MHz reference ticks (s_memrealtime) elapsed over
 * the MFMA loop.  FLOPs per launch: blocks * waves * iters8 * 64 * 32768.
 * `out` holds blocks * waves * 8192 floats, `clocks` 2 * blocks * waves
 * uint64; `ops` 16-byte aligned.  1 <= blocks <= 65536, 0 <= iters8 <= 2^24.
 */
int lgs_test_mfma_rate(int blocks, int waves, int iters8, const void* ops, float* out, uint64_t* clocks,
                       void* stream);

/*
 * Debug builds (liblgs_debug.so, compiled with -DLGS_DEBUG): every entry point
 * records the device spans it validated, and every launcher checks, on the
 * host before each kernel launch, that each span the kernel reads or writes
 * lies inside one of them (printing the span and aborting if not).
 *   lgs_test_debug_build:  1 in a debug build, 0 in the product build.
 *   lgs_test_set_dry_run:  debug builds: with on != 0 the entry points make
 *                          no HIP call at all (no launch, no error query, no
 *                          symbol lookup) but run every check, so fake device
 *                          pointers may be passed; returns 0 (-1 in the
 *                          product build, where it does nothing).
 *   lgs_test_debug_checks: checks run so far in this process (0 in the
 *                          product build).
 */
int lgs_test_debug_build(void);
int lgs_test_set_dry_run(int on);
long lgs_test_debug_checks(void);
/* The check itself: registers [allowed, allowed + allowed_bytes) as a validated
   span, then checks [p, p + bytes) against it (aborting with a message if it
   is not inside), then drops the span; returns 0 (-1 in the product build). */
int lgs_test_debug_span(const void* allowed, size_t allowed_bytes, const void* p, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* LGS_TESTING_H_ */
