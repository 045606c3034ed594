// The extern "C" entry points of liblgs.so (declared in include/lgs.h):
// argument validation, workspace carving and dispatch to the launchers.
// Validation touches no HIP API, so a rejected call never initialises the
// runtime or enqueues anything.
#include <stdarg.h>
#include <stdio.h>

#include <climits>
#include <cmath>

#include "debug.hpp"
#include "internal.hpp"
#include "lgs.h"
#include "lgs_testing.h"

#define LGS_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  lgs::debug::end_call();
  return code;
}

int ok() {
  g_err[0] = 0;
  lgs::debug::end_call();
  return LGS_OK;
}

// Drop an error a previous launch left behind, so that the status after this
// call's launches is this call's own (no HIP call in a debug dry run).
void clear_hip_error() {
  if (!lgs::debug::dry_run()) clear_hip_error();
}

// Debug builds: a device span this call validated (debug.hpp).
void allow(const void* p, size_t bytes) { lgs::debug::allow(p, bytes); }

size_t elt(int dtype) { return dtype == LGS_BF16 ? 2u : 4u; }
size_t round256(size_t x) { return (x + 255u) & ~(size_t)255u; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Shared shape checks.  Returns LGS_OK or a failure code (message set).
int check_bst(int b, int s, int h, int t, int rank) {
  if (b <= 0 || s <= 0 || h <= 0 || t <= 0)
    return fail(LGS_ERR_INVALID_ARG, "b, s, h and t must be positive (got b=%d s=%d h=%d t=%d)", b,
                s, h, t);
  if ((int64_t)b * s > INT_MAX)
    return fail(LGS_ERR_INVALID_ARG, "b*s = %lld tokens exceeds INT_MAX", (long long)b * s);
  if (rank < 0 || rank >= t) return fail(LGS_ERR_INVALID_ARG, "rank %d not in [0, %d)", rank, t);
  return LGS_OK;
}

int check_dtype(int dtype) {
  if (dtype != LGS_F32 && dtype != LGS_BF16)
    return fail(LGS_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  return LGS_OK;
}

// A matrix operand of `rows` rows: non-null (if required), ld >= width, the
// dtype's alignment, and (bf16, read with 32-bit buffer offsets) < 2 GiB.
int check_mat(const char* name, const void* p, int64_t rows, int64_t ld, int64_t width, int dtype,
              bool required) {
  if (!p) {
    if (required) return fail(LGS_ERR_INVALID_ARG, "%s is NULL", name);
    return LGS_OK;
  }
  if (ld < width)
    return fail(LGS_ERR_INVALID_ARG, "%s: leading dimension %lld < row width %lld", name,
                (long long)ld, (long long)width);
  if (dtype == LGS_BF16) {
    if (!aligned(p, 16) || ld % 8 != 0)
      return fail(LGS_ERR_UNSUPPORTED, "%s: bf16 operands need a 16-byte aligned base and ld %% 8 == 0",
                  name);
    if (((rows - 1) * ld + width) * 2 >= ((int64_t)1 << 31))
      return fail(LGS_ERR_UNSUPPORTED, "%s: bf16 operands must span less than 2 GiB", name);
  } else if (!aligned(p, 4)) {
    return fail(LGS_ERR_UNSUPPORTED, "%s: fp32 operands need a 4-byte aligned base", name);
  }
  allow(p, lgs::debug::mat_bytes(rows, ld, width, elt(dtype)));
  return LGS_OK;
}

int check_mlp(int b, int s, int h, int ffn, int t, int rank, int dtype, int act) {
  int st = check_bst(b, s, h, t, rank);
  if (st) return st;
  if (ffn <= 0 || ffn % t != 0)
    return fail(LGS_ERR_INVALID_ARG, "ffn=%d must be positive and divisible by t=%d", ffn, t);
  if ((st = check_dtype(dtype))) return st;
  if (act != LGS_GELU_ERF && act != LGS_GELU_TANH)
    return fail(LGS_ERR_UNSUPPORTED, "unknown GeLU variant %d", act);
  if (h % 8 != 0 || (ffn / t) % 8 != 0)
    return fail(LGS_ERR_UNSUPPORTED, "h=%d and ffn/t=%d must be multiples of 8", h, ffn / t);
  return LGS_OK;
}

int launched(hipError_t e) {
  if (e != hipSuccess) return fail(LGS_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

LGS_API int lgs_version(void) { return 100; }

LGS_API const char* lgs_status_string(int status) {
  switch (status) {
    case LGS_OK: return "ok";
    case LGS_ERR_INVALID_ARG: return "invalid argument";
    case LGS_ERR_UNSUPPORTED: return "unsupported dtype, variant or alignment";
    case LGS_ERR_WORKSPACE: return "workspace missing or too small";
    case LGS_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

LGS_API const char* lgs_last_error(void) { return g_err; }

LGS_API size_t lgs_mlp_fwd_workspace_bytes(int b, int s, int h, int ffn, int t, int dtype,
                                           int y_given) {
  if (b <= 0 || s <= 0 || h <= 0 || t <= 0 || ffn <= 0 || ffn % t) return 0;
  if (y_given) return 0;
  return round256((size_t)b * s * (ffn / t) * elt(dtype));
}

// Y_i and dU_i, then (bf16, when the grouped launch splits dB and dA over K)
// their partial sums and counters.
LGS_API size_t lgs_mlp_bwd_workspace_bytes(int b, int s, int h, int ffn, int t, int dtype) {
  if (b <= 0 || s <= 0 || h <= 0 || t <= 0 || ffn <= 0 || ffn % t) return 0;
  if ((int64_t)b * s > INT_MAX) return 0;
  const size_t split = dtype == LGS_BF16 ? lgs::mlp_bwd_split_bytes(b * s, h, ffn / t) : 0;
  return 2 * round256((size_t)b * s * (ffn / t) * elt(dtype)) + split;
}

namespace {

// The workspace of the backward (and of its three parts): Y_i then dU_i.
int bwd_workspace(int b, int s, int h, int ffn, int t, int dtype, void* workspace,
                  size_t workspace_bytes, char** y, char** du);

}  // namespace

LGS_API size_t lgs_swiglu_fwd_workspace_bytes(int b, int s, int h, int ffn, int t, int dtype,
                                              int y_given) {
  if (b <= 0 || s <= 0 || h <= 0 || t <= 0 || ffn <= 0 || ffn % t) return 0;
  if (y_given) return 0;
  return round256((size_t)b * s * (ffn / t) * elt(dtype));
}

LGS_API size_t lgs_swiglu_bwd_workspace_bytes(int b, int s, int h, int ffn, int t, int dtype) {
  if (b <= 0 || s <= 0 || h <= 0 || t <= 0 || ffn <= 0 || ffn % t) return 0;
  const size_t mf = (size_t)b * s * (ffn / t) * elt(dtype);
  return round256(mf) + round256(2 * mf);
}

LGS_API size_t lgs_xent_workspace_bytes(int b, int s, int h, int vocab, int t, int dtype) {
  (void)dtype;
  if (b <= 0 || s <= 0 || h <= 0 || t <= 0 || vocab <= 0 || vocab % t) return 0;
  if ((int64_t)b * s > INT_MAX) return 0;
  return round256(lgs::xent_scratch_bytes(b * s, vocab / t));
}

LGS_API int tp_mlp_fwd(int b, int s, int h, int ffn, int t, int rank, int dtype, int act,
                       const void* X, int64_t ldx, const void* A_i, int64_t lda, const void* B_i,
                       int64_t ldb, void* U_i, int64_t ldu, void* Y_i, int64_t ldy, void* Z_i,
                       int64_t ldz, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_mlp(b, s, h, ffn, t, rank, dtype, act);
  if (st) return st;
  const int M = b * s, f = ffn / t;
  if ((st = check_mat("X", X, M, ldx, h, dtype, true))) return st;
  if ((st = check_mat("A_i", A_i, h, lda, f, dtype, true))) return st;
  if ((st = check_mat("B_i", B_i, f, ldb, h, dtype, true))) return st;
  if ((st = check_mat("U_i", U_i, M, ldu, f, dtype, false))) return st;
  if ((st = check_mat("Y_i", Y_i, M, ldy, f, dtype, false))) return st;
  if ((st = check_mat("Z_i", Z_i, M, ldz, h, dtype, true))) return st;
  if (!Y_i) {
    const size_t need = lgs_mlp_fwd_workspace_bytes(b, s, h, ffn, t, dtype, 0);
    if (!workspace || workspace_bytes < need)
      return fail(LGS_ERR_WORKSPACE, "workspace of %zu bytes needed for Y_i, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(LGS_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  allow(workspace, workspace_bytes);
    Y_i = workspace;
    ldy = f;
  }
  clear_hip_error();
  return launched(lgs::mlp_fwd(dtype == LGS_BF16, M, h, f, act, X, ldx, A_i, lda, B_i, ldb, U_i,
                               ldu, Y_i, ldy, Z_i, ldz, (hipStream_t)stream));
}

LGS_API int tp_mlp_bwd(int b, int s, int h, int ffn, int t, int rank, int dtype, int act,
                       const void* X, int64_t ldx, const void* A_i, int64_t lda, const void* B_i,
                       int64_t ldb, const void* U_i, int64_t ldu, const void* dZ, int64_t lddz,
                       void* dX_i, int64_t lddx, void* dA_i, int64_t ldda, void* dB_i,
                       int64_t lddb, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_mlp(b, s, h, ffn, t, rank, dtype, act);
  if (st) return st;
  const int M = b * s, f = ffn / t;
  if ((st = check_mat("X", X, M, ldx, h, dtype, true))) return st;
  if ((st = check_mat("A_i", A_i, h, lda, f, dtype, true))) return st;
  if ((st = check_mat("B_i", B_i, f, ldb, h, dtype, true))) return st;
  if ((st = check_mat("U_i", U_i, M, ldu, f, dtype, true))) return st;
  if ((st = check_mat("dZ", dZ, M, lddz, h, dtype, true))) return st;
  if ((st = check_mat("dX_i", dX_i, M, lddx, h, dtype, true))) return st;
  if ((st = check_mat("dA_i", dA_i, h, ldda, f, dtype, true))) return st;
  if ((st = check_mat("dB_i", dB_i, f, lddb, h, dtype, true))) return st;
  const size_t need = lgs_mlp_bwd_workspace_bytes(b, s, h, ffn, t, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(LGS_ERR_WORKSPACE, "workspace of %zu bytes needed for Y_i and dU_i, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(LGS_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  allow(workspace, workspace_bytes);
  const size_t half = round256((size_t)M * f * elt(dtype));
  char* y = (char*)workspace;
  char* du = y + half;
  char* split = need > 2 * half ? y + 2 * half : nullptr;
  clear_hip_error();
  return launched(lgs::mlp_bwd(dtype == LGS_BF16, M, h, f, act, X, ldx, A_i, lda, B_i, ldb, U_i,
                               ldu, dZ, lddz, dX_i, lddx, dA_i, ldda, dB_i, lddb, y, du, split,
                               (hipStream_t)stream));
}

namespace {

// The SwiGLU calls share the GeLU block's shape rules; the gate takes no
// variant and only bf16 is built.
int check_swiglu(int b, int s, int h, int ffn, int t, int rank, int dtype) {
  int st = check_mlp(b, s, h, ffn, t, rank, dtype, LGS_GELU_ERF);
  if (st) return st;
  if (dtype != LGS_BF16) return fail(LGS_ERR_UNSUPPORTED, "the SwiGLU block takes bf16 only");
  return LGS_OK;
}

}  // namespace

LGS_API int tp_swiglu_fwd(int b, int s, int h, int ffn, int t, int rank, int dtype,
                          const void* X, int64_t ldx, const void* Wgu_i, int64_t ldwgu,
                          const void* Wd_i, int64_t ldwd, void* GU_i, int64_t ldgu, void* Y_i,
                          int64_t ldy, void* Z_i, int64_t ldz, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int st = check_swiglu(b, s, h, ffn, t, rank, dtype);
  if (st) return st;
  const int M = b * s, f = ffn / t;
  if ((st = check_mat("X", X, M, ldx, h, dtype, true))) return st;
  if ((st = check_mat("Wgu_i", Wgu_i, h, ldwgu, 2 * f, dtype, true))) return st;
  if ((st = check_mat("Wd_i", Wd_i, f, ldwd, h, dtype, true))) return st;
  if ((st = check_mat("GU_i", GU_i, M, ldgu, 2 * f, dtype, false))) return st;
  if ((st = check_mat("Y_i", Y_i, M, ldy, f, dtype, false))) return st;
  if ((st = check_mat("Z_i", Z_i, M, ldz, h, dtype, true))) return st;
  if (!Y_i) {
    const size_t need = lgs_swiglu_fwd_workspace_bytes(b, s, h, ffn, t, dtype, 0);
    if (!workspace || workspace_bytes < need)
      return fail(LGS_ERR_WORKSPACE, "workspace of %zu bytes needed for Y_i, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(LGS_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  allow(workspace, workspace_bytes);
    Y_i = workspace;
    ldy = f;
  }
  clear_hip_error();
  return launched(lgs::swiglu_fwd(M, h, f, X, ldx, Wgu_i, ldwgu, Wd_i, ldwd, GU_i, ldgu, Y_i, ldy,
                                  Z_i, ldz, (hipStream_t)stream));
}

LGS_API int tp_swiglu_bwd(int b, int s, int h, int ffn, int t, int rank, int dtype,
                          const void* X, int64_t ldx, const void* Wgu_i, int64_t ldwgu,
                          const void* Wd_i, int64_t ldwd, const void* GU_i, int64_t ldgu,
                          const void* dZ, int64_t lddz, void* dX_i, int64_t lddx, void* dWgu_i,
                          int64_t lddwgu, void* dWd_i, int64_t lddwd, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int st = check_swiglu(b, s, h, ffn, t, rank, dtype);
  if (st) return st;
  const int M = b * s, f = ffn / t;
  if ((st = check_mat("X", X, M, ldx, h, dtype, true))) return st;
  if ((st = check_mat("Wgu_i", Wgu_i, h, ldwgu, 2 * f, dtype, true))) return st;
  if ((st = check_mat("Wd_i", Wd_i, f, ldwd, h, dtype, true))) return st;
  if ((st = check_mat("GU_i", GU_i, M, ldgu, 2 * f, dtype, true))) return st;
  if ((st = check_mat("dZ", dZ, M, lddz, h, dtype, true))) return st;
  if ((st = check_mat("dX_i", dX_i, M, lddx, h, dtype, true))) return st;
  if ((st = check_mat("dWgu_i", dWgu_i, h, lddwgu, 2 * f, dtype, true))) return st;
  if ((st = check_mat("dWd_i", dWd_i, f, lddwd, h, dtype, true))) return st;
  const size_t need = lgs_swiglu_bwd_workspace_bytes(b, s, h, ffn, t, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(LGS_ERR_WORKSPACE, "workspace of %zu bytes needed for Y_i and dGU_i, %zu given",
                need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(LGS_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  allow(workspace, workspace_bytes);
  char* y = (char*)workspace;
  char* dgu = y + round256((size_t)M * f * 2);
  clear_hip_error();
  return launched(lgs::swiglu_bwd(M, h, f, X, ldx, Wgu_i, ldwgu, Wd_i, ldwd, GU_i, ldgu, dZ, lddz,
                                  dX_i, lddx, dWgu_i, lddwgu, dWd_i, lddwd, y, dgu,
                                  (hipStream_t)stream));
}

namespace {

int bwd_workspace(int b, int s, int h, int ffn, int t, int dtype, void* workspace,
                  size_t workspace_bytes, char** y, char** du) {
  const size_t need = lgs_mlp_bwd_workspace_bytes(b, s, h, ffn, t, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(LGS_ERR_WORKSPACE, "workspace of %zu bytes needed for Y_i and dU_i, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(LGS_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  allow(workspace, workspace_bytes);
  *y = (char*)workspace;
  *du = *y + round256((size_t)b * s * (ffn / t) * elt(dtype));
  return LGS_OK;
}

}  // namespace

LGS_API int tp_mlp_bwd_dgelu(int b, int s, int h, int ffn, int t, int rank, int dtype, int act,
                             const void* B_i, int64_t ldb, const void* U_i, int64_t ldu,
                             const void* dZ, int64_t lddz, void* workspace, size_t workspace_bytes,
                             void* stream) {
  int st = check_mlp(b, s, h, ffn, t, rank, dtype, act);
  if (st) return st;
  const int M = b * s, f = ffn / t;
  if ((st = check_mat("B_i", B_i, f, ldb, h, dtype, true))) return st;
  if ((st = check_mat("U_i", U_i, M, ldu, f, dtype, true))) return st;
  if ((st = check_mat("dZ", dZ, M, lddz, h, dtype, true))) return st;
  char *y, *du;
  if ((st = bwd_workspace(b, s, h, ffn, t, dtype, workspace, workspace_bytes, &y, &du))) return st;
  clear_hip_error();
  return launched(lgs::mlp_bwd_dgelu(dtype == LGS_BF16, M, h, f, act, B_i, ldb, U_i, ldu, dZ, lddz, y,
                                     du, (hipStream_t)stream));
}

LGS_API int tp_mlp_bwd_dx(int b, int s, int h, int ffn, int t, int rank, int dtype,
                          const void* A_i, int64_t lda, void* dX_i, int64_t lddx, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int st = check_mlp(b, s, h, ffn, t, rank, dtype, LGS_GELU_ERF);
  if (st) return st;
  const int M = b * s, f = ffn / t;
  if ((st = check_mat("A_i", A_i, h, lda, f, dtype, true))) return st;
  if ((st = check_mat("dX_i", dX_i, M, lddx, h, dtype, true))) return st;
  char *y, *du;
  if ((st = bwd_workspace(b, s, h, ffn, t, dtype, workspace, workspace_bytes, &y, &du))) return st;
  clear_hip_error();
  return launched(lgs::mlp_bwd_dx(dtype == LGS_BF16, M, h, f, A_i, lda, du, dX_i, lddx,
                                  (hipStream_t)stream));
}

LGS_API int tp_mlp_bwd_dw(int b, int s, int h, int ffn, int t, int rank, int dtype, const void* X,
                          int64_t ldx, const void* dZ, int64_t lddz, void* dA_i, int64_t ldda,
                          void* dB_i, int64_t lddb, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int st = check_mlp(b, s, h, ffn, t, rank, dtype, LGS_GELU_ERF);
  if (st) return st;
  const int M = b * s, f = ffn / t;
  if ((st = check_mat("X", X, M, ldx, h, dtype, true))) return st;
  if ((st = check_mat("dZ", dZ, M, lddz, h, dtype, true))) return st;
  if ((st = check_mat("dA_i", dA_i, h, ldda, f, dtype, true))) return st;
  if ((st = check_mat("dB_i", dB_i, f, lddb, h, dtype, true))) return st;
  char *y, *du;
  if ((st = bwd_workspace(b, s, h, ffn, t, dtype, workspace, workspace_bytes, &y, &du))) return st;
  clear_hip_error();
  return launched(lgs::mlp_bwd_dw(dtype == LGS_BF16, M, h, f, X, ldx, dZ, lddz, y, du, dA_i, ldda, dB_i,
                                  lddb, (hipStream_t)stream));
}

namespace {

// Argument rules of the fused CE forward (both variants).
int check_xent_fwd(int b, int s, int h, int vocab, int t, int rank, int dtype, const void* H,
                   int64_t ldh, const void* E_r, int64_t lde, const int32_t* targets, float* m_r,
                   float* l_r, float* tgt_r, int32_t* argmax_r, float* loss) {
  int st = check_bst(b, s, h, t, rank);
  if (st) return st;
  if (vocab <= 0 || vocab % t != 0)
    return fail(LGS_ERR_INVALID_ARG, "vocab=%d must be positive and divisible by t=%d", vocab, t);
  if (dtype != LGS_BF16) return fail(LGS_ERR_UNSUPPORTED, "the fused cross-entropy takes bf16 only");
  if (h % 8 != 0) return fail(LGS_ERR_UNSUPPORTED, "h=%d must be a multiple of 8", h);
  const int M = b * s, Vr = vocab / t;
  if ((st = check_mat("H", H, M, ldh, h, dtype, true))) return st;
  if ((st = check_mat("E_r", E_r, Vr, lde, h, dtype, true))) return st;
  if (!targets || !m_r || !l_r || !tgt_r)
    return fail(LGS_ERR_INVALID_ARG, "targets, m_r, l_r and tgt_r are required");
  if (!aligned(targets, 4) || !aligned(m_r, 4) || !aligned(l_r, 4) || !aligned(tgt_r, 4) ||
      !aligned(argmax_r, 4) || !aligned(loss, 4))
    return fail(LGS_ERR_UNSUPPORTED, "per-token arrays must be 4-byte aligned");
  if (loss && t != 1)
    return fail(LGS_ERR_INVALID_ARG, "loss needs the whole vocabulary (t == 1); merge ranks with shard_partial_sum");
  for (const void* a : {(const void*)targets, (const void*)m_r, (const void*)l_r, (const void*)tgt_r,
                        (const void*)argmax_r, (const void*)loss})
    allow(a, (size_t)M * 4);
  return LGS_OK;
}

}  // namespace

LGS_API int vocab_parallel_xent_fwd(int b, int s, int h, int vocab, int t, int rank, int dtype,
                                    const void* H, int64_t ldh, const void* E_r, int64_t lde,
                                    const int32_t* targets, float* m_r, float* l_r, float* tgt_r,
                                    int32_t* argmax_r, float* loss, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  int st = check_xent_fwd(b, s, h, vocab, t, rank, dtype, H, ldh, E_r, lde, targets, m_r, l_r, tgt_r,
                          argmax_r, loss);
  if (st) return st;
  const int M = b * s, Vr = vocab / t;
  const size_t need = lgs_xent_workspace_bytes(b, s, h, vocab, t, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(LGS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(LGS_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  allow(workspace, workspace_bytes);
  clear_hip_error();
  return launched(lgs::xent_fwd(M, h, Vr, rank * Vr, H, ldh, E_r, lde, targets, m_r, l_r, tgt_r,
                                argmax_r, loss, workspace, (hipStream_t)stream));
}

static_assert(LGS_XENT_NOALLOC_SCRATCH_BYTES == lgs::kXentStaticScratchBytes,
              "the header states the static scratch's size");

LGS_API int vocab_parallel_xent_fwd_noalloc(int b, int s, int h, int vocab, int t, int rank,
                                            int dtype, const void* H, int64_t ldh, const void* E_r,
                                            int64_t lde, const int32_t* targets, float* m_r,
                                            float* l_r, float* tgt_r, int32_t* argmax_r,
                                            float* loss, void* stream) {
  int st = check_xent_fwd(b, s, h, vocab, t, rank, dtype, H, ldh, E_r, lde, targets, m_r, l_r, tgt_r,
                          argmax_r, loss);
  if (st) return st;
  const int M = b * s, Vr = vocab / t;
  const size_t need = lgs_xent_workspace_bytes(b, s, h, vocab, t, dtype);
  if (need > LGS_XENT_NOALLOC_SCRATCH_BYTES)
    return fail(LGS_ERR_UNSUPPORTED,
                "%zu bytes of slab partials needed, the static scratch holds %zu: use "
                "vocab_parallel_xent_fwd with a workspace",
                need, (size_t)LGS_XENT_NOALLOC_SCRATCH_BYTES);
  clear_hip_error();
  void* scratch = nullptr;
  const hipError_t e = lgs::xent_static_scratch((hipStream_t)stream, &scratch);
  if (e != hipSuccess)
    return fail(LGS_ERR_HIP, "looking up the static scratch failed (nothing enqueued): %s",
                hipGetErrorString(e));
  return launched(lgs::xent_fwd(M, h, Vr, rank * Vr, H, ldh, E_r, lde, targets, m_r, l_r, tgt_r,
                                argmax_r, loss, scratch, (hipStream_t)stream));
}

LGS_API size_t lgs_xent_bwd_workspace_bytes(int b, int s, int h, int vocab, int t, int dtype) {
  (void)dtype;
  if (b <= 0 || s <= 0 || h <= 0 || t <= 0 || vocab <= 0 || vocab % t) return 0;
  if ((int64_t)b * s > INT_MAX) return 0;
  return round256(lgs::xent_bwd_scratch_bytes(b * s, vocab / t));
}

LGS_API int vocab_parallel_xent_bwd(int b, int s, int h, int vocab, int t, int rank, int dtype,
                                    const void* H, int64_t ldh, const void* E_r, int64_t lde,
                                    const int32_t* targets, const float* lse, const float* dloss,
                                    void* dH_r, int64_t lddh, void* dE_r, int64_t ldde,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_bst(b, s, h, t, rank);
  if (st) return st;
  if (vocab <= 0 || vocab % t != 0)
    return fail(LGS_ERR_INVALID_ARG, "vocab=%d must be positive and divisible by t=%d", vocab, t);
  if (dtype != LGS_BF16) return fail(LGS_ERR_UNSUPPORTED, "the cross-entropy backward takes bf16 only");
  const int M = b * s, Vr = vocab / t;
  if (h % 8 != 0 || Vr % 8 != 0)
    return fail(LGS_ERR_UNSUPPORTED, "h=%d and vocab/t=%d must be multiples of 8", h, Vr);
  if ((st = check_mat("H", H, M, ldh, h, dtype, true))) return st;
  if ((st = check_mat("E_r", E_r, Vr, lde, h, dtype, true))) return st;
  if ((st = check_mat("dH_r", dH_r, M, lddh, h, dtype, true))) return st;
  if ((st = check_mat("dE_r", dE_r, Vr, ldde, h, dtype, true))) return st;
  if (!targets || !lse) return fail(LGS_ERR_INVALID_ARG, "targets and lse are required");
  if (!aligned(targets, 4) || !aligned(lse, 4) || !aligned(dloss, 4))
    return fail(LGS_ERR_UNSUPPORTED, "per-token arrays must be 4-byte aligned");
  for (const void* a : {(const void*)targets, (const void*)lse, (const void*)dloss}) allow(a, (size_t)M * 4);
  if ((int64_t)M * Vr * 2 >= ((int64_t)1 << 31))
    return fail(LGS_ERR_UNSUPPORTED, "the slice's gradient G (M x vocab/t bf16) must span less than 2 GiB");
  const size_t need = lgs_xent_bwd_workspace_bytes(b, s, h, vocab, t, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(LGS_ERR_WORKSPACE, "workspace of %zu bytes needed for G, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(LGS_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  allow(workspace, workspace_bytes);
  clear_hip_error();
  return launched(lgs::xent_bwd(M, h, Vr, rank * Vr, H, ldh, E_r, lde, targets, lse, dloss, dH_r,
                                lddh, dE_r, ldde, workspace, (hipStream_t)stream));
}

LGS_API int shard_partial_sum(int op, int t, int64_t n, int in_dtype, int out_dtype,
                              const void* parts, int64_t part_stride, void* out, void* stream) {
  if (t <= 0 || n < 0) return fail(LGS_ERR_INVALID_ARG, "t must be positive and n non-negative");
  int st;
  if ((st = check_dtype(in_dtype)) || (st = check_dtype(out_dtype))) return st;
  if (op == LGS_REDUCE_SUM) {
    if (n > 0 && (!parts || !out)) return fail(LGS_ERR_INVALID_ARG, "parts and out are required");
    if (t > 1 && part_stride < n)
      return fail(LGS_ERR_INVALID_ARG, "part_stride %lld < n %lld", (long long)part_stride, (long long)n);
    if (!aligned(parts, elt(in_dtype)) || !aligned(out, elt(out_dtype)))
      return fail(LGS_ERR_UNSUPPORTED, "misaligned parts or out");
    if (n == 0) return ok();
    allow(parts, (size_t)((t - 1) * part_stride + n) * elt(in_dtype));
    allow(out, (size_t)n * elt(out_dtype));
    clear_hip_error();
    return launched(lgs::partial_sum(t, n, in_dtype == LGS_BF16, out_dtype == LGS_BF16, parts,
                                     part_stride, out, (hipStream_t)stream));
  }
  if (op == LGS_REDUCE_XENT || op == LGS_REDUCE_XENT_LSE) {
    const bool lse_only = op == LGS_REDUCE_XENT_LSE;
    const int64_t per = lse_only ? 2 : 3;  // planes read per rank block
    if (in_dtype != LGS_F32 || out_dtype != LGS_F32)
      return fail(LGS_ERR_UNSUPPORTED, "the cross-entropy merge is fp32 in and out");
    if (n > 0 && (!parts || !out)) return fail(LGS_ERR_INVALID_ARG, "parts and out are required");
    if (part_stride < per * n)
      return fail(LGS_ERR_INVALID_ARG, "part_stride %lld < %lldn = %lld", (long long)part_stride,
                  (long long)per, (long long)(per * n));
    if (!aligned(parts, 4) || !aligned(out, 4)) return fail(LGS_ERR_UNSUPPORTED, "misaligned parts or out");
    if (n == 0) return ok();
    allow(parts, (size_t)((t - 1) * part_stride + per * n) * 4);
    allow(out, (size_t)n * 4);
    clear_hip_error();
    return launched(lgs::xent_combine(t, n, (const float*)parts, part_stride, lse_only, (float*)out,
                                      (hipStream_t)stream));
  }
  return fail(LGS_ERR_UNSUPPORTED, "unknown reduce op %d", op);
}

namespace {

int check_sp(int t, int s, int b, int h) {
  if (t <= 0 || s <= 0 || b <= 0 || h <= 0)
    return fail(LGS_ERR_INVALID_ARG, "t, s, b and h must be positive (got t=%d s=%d b=%d h=%d)", t,
                s, b, h);
  if (s % t != 0) return fail(LGS_ERR_INVALID_ARG, "s=%d must be divisible by t=%d", s, t);
  return LGS_OK;
}

}  // namespace

LGS_API int shard_reduce_scatter(int t, int rank, int s, int b, int h, int in_dtype, int out_dtype,
                                 const void* parts, int64_t part_stride, void* out, void* stream) {
  int st = check_sp(t, s, b, h);
  if (st) return st;
  if (rank < 0 || rank >= t) return fail(LGS_ERR_INVALID_ARG, "rank %d not in [0, %d)", rank, t);
  if ((st = check_dtype(in_dtype)) || (st = check_dtype(out_dtype))) return st;
  const int64_t n = (int64_t)s * b * h, chunk = n / t;
  if (!parts || !out) return fail(LGS_ERR_INVALID_ARG, "parts and out are required");
  if (t > 1 && part_stride < n)
    return fail(LGS_ERR_INVALID_ARG, "part_stride %lld < s*b*h = %lld", (long long)part_stride,
                (long long)n);
  if (!aligned(parts, elt(in_dtype)) || !aligned(out, elt(out_dtype)))
    return fail(LGS_ERR_UNSUPPORTED, "misaligned parts or out");
  allow(parts, (size_t)((t - 1) * (t > 1 ? part_stride : 0) + n) * elt(in_dtype));
  allow(out, (size_t)chunk * elt(out_dtype));
  clear_hip_error();
  return launched(lgs::reduce_scatter(t, chunk, rank, in_dtype == LGS_BF16, out_dtype == LGS_BF16,
                                      parts, part_stride, out, (hipStream_t)stream));
}

LGS_API int shard_reduce_scatter_layernorm(int t, int rank, int s, int b, int h, int dtype,
                                           const void* parts, int64_t part_stride, const void* residual,
                                           const uint8_t* keep, float keep_scale, const void* gamma,
                                           const void* beta, float eps, void* hs, void* y, void* stream) {
  int st = check_sp(t, s, b, h);
  if (st) return st;
  if (rank < 0 || rank >= t) return fail(LGS_ERR_INVALID_ARG, "rank %d not in [0, %d)", rank, t);
  if ((st = check_dtype(dtype))) return st;
  if (dtype != LGS_BF16) return fail(LGS_ERR_UNSUPPORTED, "the fused sequence-parallel region is bf16 only");
  if (h % 8 != 0 || h > lgs::rs_layernorm_max_h())
    return fail(LGS_ERR_UNSUPPORTED, "h=%d must be a multiple of 8 and at most %d", h, lgs::rs_layernorm_max_h());
  if (!parts || !residual || !gamma || !beta || !hs || !y)
    return fail(LGS_ERR_INVALID_ARG, "parts, residual, gamma, beta, hs and y are required");
  if (!(eps > 0.f) || !std::isfinite(eps) || !std::isfinite(keep_scale))
    return fail(LGS_ERR_INVALID_ARG, "eps must be positive and finite, keep_scale finite");
  const int64_t n = (int64_t)s * b * h, chunk = n / t;
  if (t > 1 && part_stride < n)
    return fail(LGS_ERR_INVALID_ARG, "part_stride %lld < s*b*h = %lld", (long long)part_stride,
                (long long)n);
  if (t > 1 && part_stride % 8 != 0) return fail(LGS_ERR_UNSUPPORTED, "part_stride must be a multiple of 8");
  for (const void* p : {parts, residual, gamma, beta, (const void*)hs, (const void*)y})
    if (!aligned(p, 16)) return fail(LGS_ERR_UNSUPPORTED, "parts, residual, gamma, beta, hs and y need 16-byte alignment");
  if (keep && !aligned(keep, 8)) return fail(LGS_ERR_UNSUPPORTED, "the keep mask needs 8-byte alignment");
  allow(parts, (size_t)((t - 1) * (t > 1 ? part_stride : 0) + n) * 2);
  allow(residual, (size_t)chunk * 2);
  if (keep) allow(keep, (size_t)chunk);
  allow(gamma, (size_t)h * 2);
  allow(beta, (size_t)h * 2);
  allow(hs, (size_t)chunk * 2);
  allow(y, (size_t)chunk * 2);
  clear_hip_error();
  return launched(lgs::rs_layernorm(t, (s / t) * b, h, rank, parts, t > 1 ? part_stride : 0, residual, keep,
                                    keep_scale, gamma, beta, eps, hs, y, (hipStream_t)stream));
}

LGS_API size_t lgs_layernorm_bwd_workspace_bytes(int t, int s, int b, int h, int dtype) {
  if (t <= 0 || s <= 0 || b <= 0 || h <= 0 || s % t != 0 || dtype != LGS_BF16 || h % 8 != 0 ||
      h > lgs::rs_layernorm_max_h() || (int64_t)(s / t) * b > INT_MAX)
    return 0;
  return round256(lgs::layernorm_bwd_scratch_bytes((s / t) * b, h));
}

LGS_API int shard_layernorm_bwd(int t, int rank, int s, int b, int h, int dtype, const void* hs, const void* dy,
                                const void* dhs, const uint8_t* keep, float keep_scale, const void* gamma,
                                float eps, void* g, void* dz, float* dgamma, float* dbeta, void* workspace,
                                size_t workspace_bytes, void* stream) {
  int st = check_sp(t, s, b, h);
  if (st) return st;
  if (rank < 0 || rank >= t) return fail(LGS_ERR_INVALID_ARG, "rank %d not in [0, %d)", rank, t);
  if ((st = check_dtype(dtype))) return st;
  if (dtype != LGS_BF16) return fail(LGS_ERR_UNSUPPORTED, "the sequence-parallel region's backward is bf16 only");
  if (h % 8 != 0 || h > lgs::rs_layernorm_max_h())
    return fail(LGS_ERR_UNSUPPORTED, "h=%d must be a multiple of 8 and at most %d", h, lgs::rs_layernorm_max_h());
  if (!hs || !dy || !gamma || !g || !dz || !dgamma || !dbeta)
    return fail(LGS_ERR_INVALID_ARG, "hs, dy, gamma, g, dz, dgamma and dbeta are required");
  if (!(eps > 0.f) || !std::isfinite(eps) || !std::isfinite(keep_scale))
    return fail(LGS_ERR_INVALID_ARG, "eps must be positive and finite, keep_scale finite");
  for (const void* p : {hs, dy, dhs, gamma, (const void*)g, (const void*)dz, (const void*)dgamma, (const void*)dbeta})
    if (p && !aligned(p, 16))
      return fail(LGS_ERR_UNSUPPORTED, "hs, dy, dhs, gamma, g, dz, dgamma and dbeta need 16-byte alignment");
  if (keep && !aligned(keep, 8)) return fail(LGS_ERR_UNSUPPORTED, "the keep mask needs 8-byte alignment");
  const int rows = (s / t) * b;
  const size_t need = lgs::layernorm_bwd_scratch_bytes(rows, h);
  if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
    return fail(LGS_ERR_WORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, %zu given", need,
                workspace ? workspace_bytes : 0);
  const size_t chunk = (size_t)rows * h;
  for (const void* p : {hs, dy, dhs, (const void*)g, (const void*)dz})
    if (p) allow(p, chunk * 2);
  if (keep) allow(keep, chunk);
  allow(gamma, (size_t)h * 2);
  allow(dgamma, (size_t)h * 4);
  allow(dbeta, (size_t)h * 4);
  if (need) allow(workspace, need);
  clear_hip_error();
  return launched(lgs::layernorm_bwd(rows, h, hs, dy, dhs, keep, keep_scale, gamma, eps, g, dz, dgamma, dbeta,
                                     workspace, (hipStream_t)stream));
}

LGS_API int shard_all_gather(int t, int s, int b, int h, int dtype, const void* shards,
                             int64_t shard_stride, void* out, void* stream) {
  int st = check_sp(t, s, b, h);
  if (st) return st;
  if ((st = check_dtype(dtype))) return st;
  const int64_t chunk = (int64_t)(s / t) * b * h;
  if (!shards || !out) return fail(LGS_ERR_INVALID_ARG, "shards and out are required");
  if (t > 1 && shard_stride < chunk)
    return fail(LGS_ERR_INVALID_ARG, "shard_stride %lld < (s/t)*b*h = %lld", (long long)shard_stride,
                (long long)chunk);
  if (t > 65535) return fail(LGS_ERR_UNSUPPORTED, "t=%d exceeds the launch grid", t);
  if (!aligned(shards, elt(dtype)) || !aligned(out, elt(dtype)))
    return fail(LGS_ERR_UNSUPPORTED, "misaligned shards or out");
  allow(shards, (size_t)((t - 1) * (t > 1 ? shard_stride : 0) + chunk) * elt(dtype));
  allow(out, (size_t)t * chunk * elt(dtype));
  clear_hip_error();
  return launched(lgs::all_gather(t, chunk, dtype == LGS_BF16, shards, shard_stride, out,
                                  (hipStream_t)stream));
}

namespace {

// Shape rules of the attention projections; sets the per-rank widths.
int check_attn(int b, int s, int h, int n_q, int n_kv, int d, int t, int rank, int dtype, int* nqkv,
               int* hq) {
  int st = check_bst(b, s, h, t, rank);
  if (st) return st;
  if (n_q <= 0 || n_kv <= 0 || d <= 0)
    return fail(LGS_ERR_INVALID_ARG, "head counts and head_dim must be positive");
  if (n_q % t != 0 || n_kv % t != 0)
    return fail(LGS_ERR_INVALID_ARG, "n_q_heads=%d and n_kv_heads=%d must divide by t=%d", n_q, n_kv, t);
  if (n_q % n_kv != 0)
    return fail(LGS_ERR_INVALID_ARG, "n_q_heads=%d must be a multiple of n_kv_heads=%d", n_q, n_kv);
  if (dtype != LGS_BF16) return fail(LGS_ERR_UNSUPPORTED, "the attention projections take bf16 only");
  if (h % 8 != 0 || d % 8 != 0)
    return fail(LGS_ERR_UNSUPPORTED, "h=%d and head_dim=%d must be multiples of 8", h, d);
  const int64_t q = (int64_t)(n_q / t) * d, kv = (int64_t)(n_kv / t) * d;
  if (q + 2 * kv > INT_MAX) return fail(LGS_ERR_INVALID_ARG, "per-rank projection width overflows");
  *nqkv = (int)(q + 2 * kv);
  *hq = (int)q;
  return LGS_OK;
}

}  // namespace

LGS_API size_t lgs_attn_qkv_fwd_workspace_bytes(int b, int s, int h, int n_q_heads, int n_kv_heads,
                                               int head_dim, int t, int dtype) {
  int nqkv, hq;
  if (check_attn(b, s, h, n_q_heads, n_kv_heads, head_dim, t, 0, dtype, &nqkv, &hq)) {
    g_err[0] = 0;  // a query, not a failed call
    return 0;
  }
  return round256(lgs::attn_qkv_scratch_bytes(b * s, h, nqkv));
}

LGS_API int tp_attn_qkv_fwd(int b, int s, int h, int n_q_heads, int n_kv_heads, int head_dim, int t,
                            int rank, int dtype, const void* X, int64_t ldx, const void* Wqkv_i,
                            int64_t ldw, void* QKV_i, int64_t ldqkv, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int nqkv, hq;
  int st = check_attn(b, s, h, n_q_heads, n_kv_heads, head_dim, t, rank, dtype, &nqkv, &hq);
  if (st) return st;
  const int M = b * s;
  if ((st = check_mat("X", X, M, ldx, h, dtype, true))) return st;
  if ((st = check_mat("Wqkv_i", Wqkv_i, h, ldw, nqkv, dtype, true))) return st;
  if ((st = check_mat("QKV_i", QKV_i, M, ldqkv, nqkv, dtype, true))) return st;
  // The workspace is optional: given (at least the queried size, 256-byte
  // aligned) it enables the split-K schedule, else the product runs unsplit.
  const size_t need = lgs::attn_qkv_scratch_bytes(M, h, nqkv);
  if (workspace && !aligned(workspace, 256))
    return fail(LGS_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  void* scratch = (need && workspace && workspace_bytes >= need) ? workspace : nullptr;
  if (scratch) allow(scratch, workspace_bytes);
  clear_hip_error();
  return launched(lgs::attn_qkv_fwd(M, h, nqkv, X, ldx, Wqkv_i, ldw, QKV_i, ldqkv, scratch,
                                    (hipStream_t)stream));
}

LGS_API int tp_attn_qkv_bwd(int b, int s, int h, int n_q_heads, int n_kv_heads, int head_dim, int t,
                            int rank, int dtype, const void* X, int64_t ldx, const void* Wqkv_i,
                            int64_t ldw, const void* dQKV_i, int64_t lddqkv, void* dX_i, int64_t lddx,
                            void* dWqkv_i, int64_t lddw, void* stream) {
  int nqkv, hq;
  int st = check_attn(b, s, h, n_q_heads, n_kv_heads, head_dim, t, rank, dtype, &nqkv, &hq);
  if (st) return st;
  const int M = b * s;
  if ((st = check_mat("X", X, M, ldx, h, dtype, true))) return st;
  if ((st = check_mat("Wqkv_i", Wqkv_i, h, ldw, nqkv, dtype, true))) return st;
  if ((st = check_mat("dQKV_i", dQKV_i, M, lddqkv, nqkv, dtype, true))) return st;
  if ((st = check_mat("dX_i", dX_i, M, lddx, h, dtype, true))) return st;
  if ((st = check_mat("dWqkv_i", dWqkv_i, h, lddw, nqkv, dtype, true))) return st;
  clear_hip_error();
  return launched(lgs::attn_qkv_bwd(M, h, nqkv, X, ldx, Wqkv_i, ldw, dQKV_i, lddqkv, dX_i, lddx,
                                    dWqkv_i, lddw, (hipStream_t)stream));
}

LGS_API int tp_attn_out_fwd(int b, int s, int h, int n_q_heads, int head_dim, int t, int rank,
                            int dtype, const void* A_i, int64_t lda, const void* Wo_i, int64_t ldwo,
                            void* Z_i, int64_t ldz, void* stream) {
  int nqkv, hq;
  // (the output projection involves no KV heads: check the query heads only)
  int st = check_attn(b, s, h, n_q_heads, n_q_heads, head_dim, t, rank, dtype, &nqkv, &hq);
  if (st) return st;
  const int M = b * s;
  if ((st = check_mat("A_i", A_i, M, lda, hq, dtype, true))) return st;
  if ((st = check_mat("Wo_i", Wo_i, hq, ldwo, h, dtype, true))) return st;
  if ((st = check_mat("Z_i", Z_i, M, ldz, h, dtype, true))) return st;
  clear_hip_error();
  return launched(lgs::attn_out_fwd(M, hq, h, A_i, lda, Wo_i, ldwo, Z_i, ldz, (hipStream_t)stream));
}

LGS_API size_t lgs_attn_out_bwd_workspace_bytes(int b, int s, int h, int n_q_heads, int head_dim,
                                               int t, int dtype) {
  int nqkv, hq;
  if (check_attn(b, s, h, n_q_heads, n_q_heads, head_dim, t, 0, dtype, &nqkv, &hq)) {
    g_err[0] = 0;  // a query, not a failed call
    return 0;
  }
  return round256(lgs::attn_out_bwd_scratch_bytes(b * s, hq, h));
}

LGS_API int tp_attn_out_bwd(int b, int s, int h, int n_q_heads, int head_dim, int t, int rank,
                            int dtype, const void* A_i, int64_t lda, const void* Wo_i, int64_t ldwo,
                            const void* dZ, int64_t lddz, void* dA_i, int64_t ldda, void* dWo_i,
                            int64_t lddwo, void* workspace, size_t workspace_bytes, void* stream) {
  int nqkv, hq;
  // (the output projection involves no KV heads: check the query heads only)
  int st = check_attn(b, s, h, n_q_heads, n_q_heads, head_dim, t, rank, dtype, &nqkv, &hq);
  if (st) return st;
  const int M = b * s;
  if ((st = check_mat("A_i", A_i, M, lda, hq, dtype, true))) return st;
  if ((st = check_mat("Wo_i", Wo_i, hq, ldwo, h, dtype, true))) return st;
  if ((st = check_mat("dZ", dZ, M, lddz, h, dtype, true))) return st;
  if ((st = check_mat("dA_i", dA_i, M, ldda, hq, dtype, true))) return st;
  if ((st = check_mat("dWo_i", dWo_i, hq, lddwo, h, dtype, true))) return st;
  const size_t need = lgs::attn_out_bwd_scratch_bytes(M, hq, h);
  if (workspace && !aligned(workspace, 256))
    return fail(LGS_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  void* scratch = (need && workspace && workspace_bytes >= need) ? workspace : nullptr;
  if (scratch) allow(scratch, workspace_bytes);
  clear_hip_error();
  return launched(lgs::attn_out_bwd(M, hq, h, A_i, lda, Wo_i, ldwo, dZ, lddz, dA_i, ldda, dWo_i,
                                    lddwo, scratch, (hipStream_t)stream));
}

LGS_API int lgs_test_num_tiles(void) { return lgs::num_tiles(); }

LGS_API int lgs_test_tile_shape(int tile, int* bm, int* bn) {
  int m = 0, n = 0;
  if (!lgs::tile_shape(tile, &m, &n)) return -1;
  if (bm) *bm = m;
  if (bn) *bn = n;
  return 0;
}

LGS_API int lgs_test_pick_tile(int M, int N) {
  if (M <= 0 || N <= 0) return -1;
  return lgs::picked_tile(M, N);
}

LGS_API int lgs_test_mlp_bwd_plan(int M, int h, int f, int* parts, int* kchunk, int* tail) {
  if (M <= 0 || h <= 0 || f <= 0) return -1;
  const lgs::BwdSplit k = lgs::mlp_bwd_wsplit(M, h, f);
  if (parts) *parts = k.parts;
  if (kchunk) *kchunk = k.parts > 1 ? k.kchunk : M;
  if (tail) *tail = k.parts > 1 ? k.tail : 0;
  return 0;
}

LGS_API int lgs_test_gemm_bf16(int tile, int a_kmajor, int b_kmajor, int M, int N, int K,
                               const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                               int64_t ldc, void* stream) {
  if (M <= 0 || N <= 0 || K <= 0) return fail(LGS_ERR_INVALID_ARG, "M, N, K must be positive");
  if (tile < -1 || tile >= lgs::num_tiles()) return fail(LGS_ERR_INVALID_ARG, "no tile id %d", tile);
  if (!a_kmajor && b_kmajor) return fail(LGS_ERR_UNSUPPORTED, "layout pair (0, 1) is not built");
  if (N % 8 != 0) return fail(LGS_ERR_UNSUPPORTED, "N must be a multiple of 8");
  if ((a_kmajor || b_kmajor) && K % 8 != 0)
    return fail(LGS_ERR_UNSUPPORTED, "K of a K-major operand must be a multiple of 8");
  if (!a_kmajor && M % 8 != 0) return fail(LGS_ERR_UNSUPPORTED, "M of an M-major A must be a multiple of 8");
  int st;
  if ((st = check_mat("A", A, a_kmajor ? M : K, lda, a_kmajor ? K : M, LGS_BF16, true))) return st;
  if ((st = check_mat("B", B, b_kmajor ? N : K, ldb, b_kmajor ? K : N, LGS_BF16, true))) return st;
  if ((st = check_mat("C", C, M, ldc, N, LGS_BF16, true))) return st;
  clear_hip_error();
  return launched(lgs::gemm_store_bf16(tile, a_kmajor != 0, b_kmajor != 0, M, N, K, A, lda, B, ldb,
                                       C, ldc, (hipStream_t)stream));
}

LGS_API int lgs_test_mfma_rate(int blocks, int waves, int iters8, const void* ops, float* out,
                               uint64_t* clocks, void* stream) {
  if (blocks < 1 || blocks > 65536) return fail(LGS_ERR_INVALID_ARG, "blocks must be in [1, 65536]");
  if (waves < 1 || waves > 8) return fail(LGS_ERR_INVALID_ARG, "waves must be in [1, 8]");
  if (iters8 < 0 || iters8 > (1 << 24)) return fail(LGS_ERR_INVALID_ARG, "iters8 must be in [0, 2^24]");
  if (!ops || !out || !clocks) return fail(LGS_ERR_INVALID_ARG, "ops, out and clocks are required");
  if (!aligned(ops, 16)) return fail(LGS_ERR_UNSUPPORTED, "ops must be 16-byte aligned");
  allow(ops, (size_t)16 * 64 * 16);
  allow(out, lgs::mfma_rate_out_floats(blocks, waves) * 4);
  allow(clocks, (size_t)blocks * waves * 16);
  clear_hip_error();
  return launched(lgs::mfma_rate(blocks, waves, iters8, ops, out, clocks, (hipStream_t)stream));
}

LGS_API int lgs_test_xent_rows_bf16(int M, int Vr, int vocab_start, const void* Z, int64_t ldz,
                                    const int32_t* targets, float* m, float* l, float* T,
                                    void* stream) {
  if (M < 0 || Vr <= 0) return fail(LGS_ERR_INVALID_ARG, "M must be >= 0 and Vr > 0");
  if (Vr % 8 != 0) return fail(LGS_ERR_UNSUPPORTED, "Vr must be a multiple of 8");
  int st;
  if ((st = check_mat("Z", Z, M, ldz, Vr, LGS_BF16, M > 0))) return st;
  if (M > 0 && (!targets || !m || !l || !T))
    return fail(LGS_ERR_INVALID_ARG, "targets, m, l and T are required");
  for (const void* a : {(const void*)targets, (const void*)m, (const void*)l, (const void*)T})
    allow(a, (size_t)M * 4);
  if (M == 0) return ok();
  clear_hip_error();
  return launched(lgs::xent_rows(M, Vr, vocab_start, Z, ldz, targets, m, l, T, (hipStream_t)stream));
}
