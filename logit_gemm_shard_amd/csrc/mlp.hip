// One tensor-parallel rank's GeLU MLP shard, forward and backward.
//
// "Tensor Parallelism and Pipeline Parallelism: Mathematical Foundations of
// Megatron-LM ..." (llms.blog), "Column-Parallel Linear Layer" and
// "Row-Parallel Linear Layer": with A split by columns and B by rows, rank i
// computes Y_i = GeLU(X A_i) and the partial Z_i = Y_i B_i without any
// exchange; the g operator then sums the partials.  The backward follows the
// "Conjugate Communication Operators" section: dZ arrives unchanged on every
// rank, and dX_i is a partial that f* sums.
//
// Operand layouts (row-major, explicit leading dimensions):
//   X [M, h], A_i [h, f] (a column block of A [h, ffn]),
//   B_i [f, h] (a row block of B [ffn, h]), U, Y, dU [M, f], Z, dZ, dX [M, h],
//   dA_i [h, f], dB_i [f, h].
// GEMM operand majorness per product (A operand rows x K, B operand K x cols):
//   U  = X A_i      : X K-contiguous,            A_i N-contiguous
//   Z  = Y B_i      : Y K-contiguous,            B_i N-contiguous
//   dY = dZ B_i^T   : dZ K-contiguous,           B_i K-contiguous
//   dX = dU A_i^T   : dU K-contiguous,           A_i K-contiguous
//   dB = Y^T dZ     : Y M-contiguous (K=tokens), dZ N-contiguous
//   dA = X^T dU     : X M-contiguous,            dU N-contiguous
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <tuple>
#include <vector>

#include "dispatch.hpp"
#include "epilogues.hpp"
#include "gemm_f32.hpp"
#include "internal.hpp"

namespace lgs {

namespace {

// Finish time, in K tiles of one 256x256 tile, of a launch whose blocks are
// dealt in launch order to the first free of the 256 compute units.  items:
// (K tiles per block, blocks), in launch order.
int dispatch_makespan(const std::vector<std::pair<int, int>>& items) {
  std::priority_queue<int, std::vector<int>, std::greater<int>> cu;
  for (int i = 0; i < 256; ++i) cu.push(0);
  int end = 0;
  for (const auto& it : items)
    for (int b = 0; b < it.second; ++b) {
      const int t = cu.top() + it.first;
      cu.pop();
      cu.push(t);
      end = t > end ? t : end;
    }
  return end;
}

int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace

// The grouped backward launch (dB, dA over K = M tokens; dX over K = f) ends
// when its longest tiles do: at the 8.3B shape 144 dB / dA tiles of 256 K
// tiles each, while the whole launch would fill 256 compute units for 216.
// Splitting dB and dA over K into parts reduced inside the launch shortens
// them.  The plan simulates the dispatch for 1 to 4 parts, charging each part
// two K tiles for its partial slot and the last part two per slot it adds.
// The partial slots' memory traffic also slows every other tile's K loop,
// which the simulation does not see: measured, a predicted 7% gain (8.3B
// shape, 3 parts) ran 14% slower, a predicted 41% gain (M = 2200, h = 1064,
// f = 1048, 2 parts) ran faster.  So the plan splits only where the
// simulation predicts 30% or more, and takes one more part only when that
// part's predicted time is at least 5% lower (each part adds slot traffic
// the simulation cannot price).
//
// No split can reach 30% when the longest tile is short against the whole
// launch: list dispatch finishes within W/256 + L (W the launch's K tiles
// over all blocks, L the longest block's), while any split needs at least
// W/256, so if 0.3 W/256 >= 0.7 L the full split is not simulated (both 70B
// shapes).  Such launches can still end in a partly filled round of long
// tiles (70B: 448 + 448 + 512 blocks, five and a half rounds).  There the
// tail split halves only the last dA tiles (mlp_bwd_tail_split).
// Plans are cached per shape: the workspace query, the entry point's check
// and the launch each ask.
namespace {

// Only the last `tail` dA tiles split in two over the tokens, their parts
// launched after dX: the unsplit blocks make whole rounds and the parts,
// half as long, the last one; the slot traffic meets only that round.  The
// simulation charges every block the fixed cost of a tile (prologue, LDS
// fill and stores: about 12 K tiles' time) and each part four more K tiles
// for its slot, and the plan is taken for a predicted gain of 4% or more.
BwdSplit mlp_bwd_tail_split(int M, int tw, int tx, int nkw, int nkx) {
  constexpr int kFixed = 12, kSlot = 4;
  BwdSplit best{1, 0, 0, 0};
  if (M < 512) return best;
  const int kchunk = cdiv(cdiv(M, 2), 32) * 32, u = kchunk / 32, last = nkw - u;
  const int unsplit = dispatch_makespan({{nkw + kFixed, 2 * tw}, {nkx + kFixed, tx}});
  int best_cost = unsplit * 96 / 100;
  for (int tail = 8; tail <= tw; tail += 8) {
    const int cost = dispatch_makespan({{nkw + kFixed, 2 * tw - tail},
                                        {nkx + kFixed, tx},
                                        {u + kFixed + kSlot, tail},
                                        {last + kFixed + kSlot, tail}});
    if (cost < best_cost) {
      best_cost = cost;
      best = BwdSplit{2, kchunk, tail, tail};
    }
  }
  return best;
}

}  // namespace

BwdSplit mlp_bwd_wsplit(int M, int h, int f) {
  BwdSplit no{1, 0, 0, 0};
  if (M < 256 || h < 256 || f < 256) return no;
  const int tw = cdiv(f, 256) * cdiv(h, 256), tx = cdiv(M, 256) * cdiv(h, 256);
  const int nkw = cdiv(M, 32), nkx = cdiv(f, 32);

  static std::mutex mu;
  static std::map<std::tuple<int, int, int>, BwdSplit> cache;
  const auto key = std::make_tuple(M, h, f);
  {
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  BwdSplit best = no;
  const double work = (2.0 * tw * nkw + (double)tx * nkx) / 256.0;
  if (0.3 * work < 0.7 * (nkw > nkx ? nkw : nkx)) {
    const int unsplit = dispatch_makespan({{nkw, 2 * tw}, {nkx, tx}});
    int best_cost = unsplit;
    for (int parts = 2; parts <= 4; ++parts) {
      const int kchunk = cdiv(cdiv(M, parts), 32) * 32, n = cdiv(M, kchunk);
      if (n < 2 || n == best.parts) continue;
      const int u = kchunk / 32, last = nkw - (n - 1) * u;
      // launch order: dB's parts (part-major), dA's parts, dX
      const std::vector<std::pair<int, int>> items = {{u + 2, tw * (n - 1)}, {last + 2, tw},
                                                      {u + 2, tw * (n - 1)}, {last + 2, tw}, {nkx, tx}};
      const int cost = dispatch_makespan(items) + 2 * n;
      if (cost * 10 < unsplit * 7 && cost * 20 < best_cost * 19) {
        best_cost = cost;
        best = BwdSplit{n, kchunk, 2 * tw, 0};
      }
    }
  }
  if (best.parts < 2) best = mlp_bwd_tail_split(M, tw, tx, nkw, nkx);
  std::lock_guard<std::mutex> lock(mu);
  if (cache.size() >= 256) cache.clear();
  cache[key] = best;
  return best;
}

size_t mlp_bwd_split_bytes(int M, int h, int f) {
  const BwdSplit k = mlp_bwd_wsplit(M, h, f);
  if (k.parts < 2) return 0;
  const size_t part = (size_t)k.tiles * k.parts * 256 * 256 * sizeof(float);
  return part + (((size_t)k.tiles * sizeof(int) + 255) & ~(size_t)255);
}

hipError_t mlp_fwd(bool is_bf16, int M, int h, int f, int act, const void* X, int64_t ldx,
                   const void* A, int64_t lda, const void* B, int64_t ldb, void* U, int64_t ldu,
                   void* Y, int64_t ldy, void* Z, int64_t ldz, hipStream_t s) {
  hipError_t e;
  if (is_bf16) {
    EpiGeluFwd<bf16> e1{(bf16*)U, ldu, (bf16*)Y, ldy, M, f, act};
    e = gemm_bf16<true, false>(pick_tile(M, f), (const bf16*)X, ldx, (const bf16*)A, lda, M, f, h,
                               e1, s);
    if (e != hipSuccess) return e;
    EpiStore<bf16> e2{(bf16*)Z, ldz, M, h};
    return gemm_bf16<true, false>(pick_tile(M, h), (const bf16*)Y, ldy, (const bf16*)B, ldb, M, h,
                                  f, e2, s);
  }
  EpiGeluFwd<float> e1{(float*)U, ldu, (float*)Y, ldy, M, f, act};
  e = launch_gemm_f32<true, false>((const float*)X, ldx, (const float*)A, lda, M, f, h, e1, s);
  if (e != hipSuccess) return e;
  EpiStore<float> e2{(float*)Z, ldz, M, h};
  return launch_gemm_f32<true, false>((const float*)Y, ldy, (const float*)B, ldb, M, h, f, e2, s);
}

hipError_t mlp_bwd(bool is_bf16, int M, int h, int f, int act, const void* X, int64_t ldx,
                   const void* A, int64_t lda, const void* B, int64_t ldb, const void* U,
                   int64_t ldu, const void* dZ, int64_t lddz, void* dX, int64_t lddx, void* dA,
                   int64_t ldda, void* dB, int64_t lddb, void* Yws, void* dUws, void* splitws,
                   hipStream_t s) {
  hipError_t e;
  const int64_t ldw = f;  // scratch Y / dU are dense [M, f]
  if (is_bf16) {
    const bf16 *x = (const bf16*)X, *a = (const bf16*)A, *b = (const bf16*)B, *dz = (const bf16*)dZ;
    bf16 *y = (bf16*)Yws, *du = (bf16*)dUws;
    EpiGeluBwd<bf16> e1{(const bf16*)U, ldu, du, ldw, y, ldw, M, f, act};
    e = gemm_bf16<true, true>(pick_tile(M, f), dz, lddz, b, ldb, M, f, h, e1, s);
    if (e != hipSuccess) return e;
    // dB and dA reduce over all M tokens (the longest K), dX over f: one
    // grouped launch, long tiles first, so the dX tiles fill the compute
    // units the few weight-gradient tiles leave idle.
    EpiStore<bf16> eb{(bf16*)dB, lddb, f, h};
    EpiStore<bf16> ea{(bf16*)dA, ldda, h, f};
    EpiStore<bf16> ex{(bf16*)dX, lddx, M, h};
    if (f >= 256 && h >= 256 && M >= 256) {
      const auto pb = pp_problem<256, 256, false, false>(y, ldw, dz, lddz, f, h, M, eb);
      const auto pa = pp_problem<256, 256, false, false>(x, ldx, du, ldw, h, f, M, ea);
      const auto px = pp_problem<256, 256, true, true>(du, ldw, a, lda, M, h, f, ex);
      const BwdSplit k = mlp_bwd_wsplit(M, h, f);
      if (k.parts > 1 && splitws) {
        float* part = (float*)splitws;
        int* count = (int*)((char*)splitws + (size_t)k.tiles * k.parts * 256 * 256 * sizeof(float));
        if (k.tail) return launch_gemm_pp_group3_tail(pb, pa, px, KSplit{part, count, k.parts, k.kchunk}, k.tail, s);
        return launch_gemm_pp_group3_ksplit(pb, pa, px, KSplit{part, count, k.parts, k.kchunk}, s);
      }
      return launch_gemm_pp_group3(pb, pa, px, s);
    }
    return launch_gemm_pp_group3(pp_problem<128, 128, false, false>(y, ldw, dz, lddz, f, h, M, eb),
                                 pp_problem<128, 128, false, false>(x, ldx, du, ldw, h, f, M, ea),
                                 pp_problem<128, 128, true, true>(du, ldw, a, lda, M, h, f, ex), s);
  }
  const float *x = (const float*)X, *a = (const float*)A, *b = (const float*)B, *dz = (const float*)dZ;
  float *y = (float*)Yws, *du = (float*)dUws;
  EpiGeluBwd<float> e1{(const float*)U, ldu, du, ldw, y, ldw, M, f, act};
  e = launch_gemm_f32<true, true>(dz, lddz, b, ldb, M, f, h, e1, s);
  if (e != hipSuccess) return e;
  EpiStore<float> eb{(float*)dB, lddb, f, h};
  e = launch_gemm_f32<false, false>(y, ldw, dz, lddz, f, h, M, eb, s);
  if (e != hipSuccess) return e;
  EpiStore<float> ea{(float*)dA, ldda, h, f};
  e = launch_gemm_f32<false, false>(x, ldx, du, ldw, h, f, M, ea, s);
  if (e != hipSuccess) return e;
  EpiStore<float> ex{(float*)dX, lddx, M, h};
  return launch_gemm_f32<true, true>(du, ldw, a, lda, M, h, f, ex, s);
}

// The backward in three parts, for callers that overlap the input gradient's
// exchange with the weight gradients (dX's all-reduce needs dX only; dA and
// dB need no exchange): dgelu writes dU and Y into the scratch, after which
// dx and dw are independent and may run on different streams.
hipError_t mlp_bwd_dgelu(bool is_bf16, int M, int h, int f, int act, const void* B, int64_t ldb,
                         const void* U, int64_t ldu, const void* dZ, int64_t lddz, void* Yws,
                         void* dUws, hipStream_t s) {
  const int64_t ldw = f;
  if (is_bf16) {
    EpiGeluBwd<bf16> e1{(const bf16*)U, ldu, (bf16*)dUws, ldw, (bf16*)Yws, ldw, M, f, act};
    return gemm_bf16<true, true>(pick_tile(M, f), (const bf16*)dZ, lddz, (const bf16*)B, ldb, M, f, h,
                                 e1, s);
  }
  EpiGeluBwd<float> e1{(const float*)U, ldu, (float*)dUws, ldw, (float*)Yws, ldw, M, f, act};
  return launch_gemm_f32<true, true>((const float*)dZ, lddz, (const float*)B, ldb, M, f, h, e1, s);
}

hipError_t mlp_bwd_dx(bool is_bf16, int M, int h, int f, const void* A, int64_t lda,
                      const void* dUws, void* dX, int64_t lddx, hipStream_t s) {
  if (is_bf16) {
    EpiStore<bf16> ex{(bf16*)dX, lddx, M, h};
    return gemm_bf16<true, true>(pick_tile(M, h), (const bf16*)dUws, f, (const bf16*)A, lda, M, h, f, ex,
                                 s);
  }
  EpiStore<float> ex{(float*)dX, lddx, M, h};
  return launch_gemm_f32<true, true>((const float*)dUws, f, (const float*)A, lda, M, h, f, ex, s);
}

hipError_t mlp_bwd_dw(bool is_bf16, int M, int h, int f, const void* X, int64_t ldx,
                      const void* dZ, int64_t lddz, const void* Yws, const void* dUws, void* dA,
                      int64_t ldda, void* dB, int64_t lddb, hipStream_t s) {
  const int64_t ldw = f;
  if (is_bf16) {
    const bf16 *x = (const bf16*)X, *dz = (const bf16*)dZ, *y = (const bf16*)Yws, *du = (const bf16*)dUws;
    EpiStore<bf16> eb{(bf16*)dB, lddb, f, h};
    EpiStore<bf16> ea{(bf16*)dA, ldda, h, f};
    if (f >= 256 && h >= 256 && M >= 256)
      return launch_gemm_pp_group2(pp_problem<256, 256, false, false>(y, ldw, dz, lddz, f, h, M, eb),
                                   pp_problem<256, 256, false, false>(x, ldx, du, ldw, h, f, M, ea), s);
    return launch_gemm_pp_group2(pp_problem<128, 128, false, false>(y, ldw, dz, lddz, f, h, M, eb),
                                 pp_problem<128, 128, false, false>(x, ldx, du, ldw, h, f, M, ea), s);
  }
  const float *x = (const float*)X, *dz = (const float*)dZ, *y = (const float*)Yws, *du = (const float*)dUws;
  EpiStore<float> eb{(float*)dB, lddb, f, h};
  hipError_t e = launch_gemm_f32<false, false>(y, ldw, dz, lddz, f, h, M, eb, s);
  if (e != hipSuccess) return e;
  EpiStore<float> ea{(float*)dA, ldda, h, f};
  return launch_gemm_f32<false, false>(x, ldx, du, ldw, h, f, M, ea, s);
}

int num_tiles() { return kNumTiles; }

bool tile_shape(int tile, int* bm, int* bn) {
  if (tile < 0 || tile >= kNumTiles) return false;
  *bm = kTileShapes[tile].bm;
  *bn = kTileShapes[tile].bn;
  return true;
}

int picked_tile(int M, int N) { return pick_tile(M, N); }

hipError_t gemm_store_bf16(int tile, bool a_kmajor, bool b_kmajor, int M, int N, int K,
                           const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                           int64_t ldc, hipStream_t s) {
  const TileId t = tile < 0 ? pick_tile(M, N) : (TileId)tile;
  EpiStore<bf16> e{(bf16*)C, ldc, M, N};
  const bf16 *a = (const bf16*)A, *b = (const bf16*)B;
  if (a_kmajor && !b_kmajor) return gemm_bf16<true, false>(t, a, lda, b, ldb, M, N, K, e, s);
  if (a_kmajor && b_kmajor) return gemm_bf16<true, true>(t, a, lda, b, ldb, M, N, K, e, s);
  if (!a_kmajor && !b_kmajor) return gemm_bf16<false, false>(t, a, lda, b, ldb, M, N, K, e, s);
  return hipErrorInvalidValue;
}

}  // namespace lgs
