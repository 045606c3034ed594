// Tile-shape choice for the bf16 GEMM core and the launch switch over the
// instantiated shapes.
#pragma once

#include "gemm_bf16.hpp"

namespace lgs {

enum TileId : int { T256x256 = 0, T256x224, T256x192, T256x160, T128x128, kNumTiles };

struct TileShape {
  int bm, bn, wgm;  // block tile and the waves' grid (wgm x 4/wgm)
  float eff;        // relative per-CU efficiency (bigger tiles reuse each LDS byte more)
};

constexpr TileShape kTileShapes[kNumTiles] = {{256, 256, 2, 1.00f},
                                              {256, 224, 4, 0.97f},
                                              {256, 192, 2, 0.96f},
                                              {256, 160, 4, 0.92f},
                                              {128, 128, 2, 0.75f}};

// The chip runs one 256x* block per compute unit at a time (the double
// buffered tiles use 96-128 KB of the 160 KB LDS), so a launch proceeds in
// "waves" of 256 blocks.  Pick the shape minimising waves x tile area / eff:
// e.g. a 4096 x 3584 output is 224 blocks of 256x256 (1/8 of the chip idle)
// but exactly 256 blocks of 256x224.
inline TileId pick_tile(int M, int N) {
  constexpr int kCUs = 256;
  TileId best = T256x256;
  double best_cost = 1e300;
  for (int t = 0; t < kNumTiles; ++t) {
    const TileShape& s = kTileShapes[t];
    const long tiles = (long)((M + s.bm - 1) / s.bm) * ((N + s.bn - 1) / s.bn);
    const long waves = (tiles + kCUs - 1) / kCUs;
    const double cost = (double)waves * s.bm * s.bn / s.eff;
    if (cost < best_cost * 0.999) { best_cost = cost; best = (TileId)t; }
  }
  return best;
}

inline int tile_bn(TileId t) { return kTileShapes[t].bn; }
inline int tile_wn(TileId t) { return kTileShapes[t].bn * kTileShapes[t].wgm / 4; }

template <int BM, int BN, int WGM, bool AK, bool BK, class Epi>
inline GemmProblem<BM, BN, WGM, AK, BK, Epi> problem(const bf16* A, int64_t lda, const bf16* B,
                                                     int64_t ldb, int M, int N, int K,
                                                     const Epi& epi) {
  return GemmProblem<BM, BN, WGM, AK, BK, Epi>{A, lda, B, ldb, M, N, K, epi};
}

template <bool AK, bool BK, class Epi>
inline hipError_t gemm_bf16(TileId t, const bf16* A, int64_t lda, const bf16* B, int64_t ldb,
                            int M, int N, int K, const Epi& epi, hipStream_t s) {
  switch (t) {
    case T256x256: return launch_gemm(problem<256, 256, 2, AK, BK>(A, lda, B, ldb, M, N, K, epi), s);
    case T256x224: return launch_gemm(problem<256, 224, 4, AK, BK>(A, lda, B, ldb, M, N, K, epi), s);
    case T256x192: return launch_gemm(problem<256, 192, 2, AK, BK>(A, lda, B, ldb, M, N, K, epi), s);
    case T256x160: return launch_gemm(problem<256, 160, 4, AK, BK>(A, lda, B, ldb, M, N, K, epi), s);
    case T128x128: return launch_gemm(problem<128, 128, 2, AK, BK>(A, lda, B, ldb, M, N, K, epi), s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lgs
