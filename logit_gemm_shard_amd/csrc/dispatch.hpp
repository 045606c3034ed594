// Tile-shape choice for the bf16 GEMM cores and the launch switch over the
// instantiated shapes: 256x256, 256x320, 256x192 and 128x128 tiles run on the 8-wave
// ping-pong core (gemm_pp.hpp), 256x224 and 256x160 (whose widths do not
// split into two 32-multiple column halves) on the 4-wave core.
#pragma once

#include "gemm_bf16.hpp"
#include "gemm_pp.hpp"

namespace lgs {

enum TileId : int { T256x256 = 0, T256x224, T256x192, T256x160, T128x128, T256x320, kNumTiles };

struct TileShape {
  int bm, bn;
  int wn;     // width of a wave's tile (one CE slab)
  float eff;  // relative per-CU throughput, from sweeps of both cores
};

constexpr TileShape kTileShapes[kNumTiles] = {{256, 256, 128, 1.00f},   // ping-pong
                                              {256, 224, 224, 0.87f},   // 4-wave, 4x1
                                              {256, 192, 96, 0.85f},    // ping-pong
                                              {256, 160, 160, 0.72f},   // 4-wave, 4x1
                                              {128, 128, 64, 0.55f},    // ping-pong
                                              {256, 320, 160, 1.02f}};  // ping-pong

// One 256x* block per compute unit at a time (the LDS rings use 120-160 KB
// of the 160 KB), so a launch proceeds in rounds of 256 blocks.  Pick the
// shape minimising rounds x tile area / eff: e.g. an 8192 x 6400 output is
// 640 blocks of 256x320 (two and a half rounds) but 800 of 256x256 (the
// fourth round one eighth full).
//
// `allowed` is a bit mask over TileId (every mask includes 256x256).
constexpr unsigned kAllTiles = (1u << kNumTiles) - 1;
// ping-pong tiles whose wave width is a multiple of 64 (whole pairs of
// 32-column groups per wave, for paired epilogues)
constexpr unsigned kPairedTiles = (1u << T256x256) | (1u << T128x128);
// the ping-pong tiles
constexpr unsigned kPPTiles = (1u << T256x256) | (1u << T256x192) | (1u << T128x128) | (1u << T256x320);

inline TileId pick_tile(int M, int N, unsigned allowed = kAllTiles) {
  constexpr int kCUs = 256;
  TileId best = T256x256;
  double best_cost = 1e300;
  for (int t = 0; t < kNumTiles; ++t) {
    if (!(allowed & (1u << t))) continue;
    const TileShape& s = kTileShapes[t];
    const long tiles = (long)((M + s.bm - 1) / s.bm) * ((N + s.bn - 1) / s.bn);
    const long waves = (tiles + kCUs - 1) / kCUs;
    const double cost = (double)waves * s.bm * s.bn / s.eff;
    if (cost < best_cost * 0.999) { best_cost = cost; best = (TileId)t; }
  }
  return best;
}

inline double tile_cost(TileId t, int M, int N) {
  constexpr int kCUs = 256;
  const TileShape& s = kTileShapes[t];
  const long tiles = (long)((M + s.bm - 1) / s.bm) * ((N + s.bn - 1) / s.bn);
  return (double)((tiles + kCUs - 1) / kCUs) * s.bm * s.bn / s.eff;
}

// A launch plan over columns: the picked tile on columns [0, c1), then (if
// c1 < N) a second launch with another tile on [c1, N).  Splitting pays when
// the picked tile leaves a partly filled last round that smaller tiles on the
// remaining columns fill: e.g. 8192 x 6400 is 640 blocks of 256x320 (2.5
// rounds, cost 3 rounds of 256x320), but 256 of them on the first 2560
// columns (one full round) and 480 blocks of 256x256 on the other 3840 (two
// rounds of smaller tiles) cost about 2.6.  Both launches' tiles must share
// `wn` (the caller's slab numbering) when the caller needs it; `same_wn`
// enforces that.
struct ColumnPlan {
  TileId main;
  int c1;  // columns of the first launch (a multiple of its tile width), N if not split
  TileId tail;
};

inline ColumnPlan plan_columns(int M, int N, bool same_wn, unsigned allowed = kAllTiles) {
  const TileId t = pick_tile(M, N, allowed);
  ColumnPlan best{t, N, t};
  double best_cost = tile_cost(t, M, N);
  const int bn = kTileShapes[t].bn;
  for (int c1 = bn; c1 < N; c1 += bn)
    for (int u = 0; u < kNumTiles; ++u) {
      if (!(allowed & (1u << u))) continue;
      if (same_wn && kTileShapes[u].wn != kTileShapes[t].wn) continue;
      const double c = tile_cost(t, M, c1) + tile_cost((TileId)u, M, N - c1);
      if (c < best_cost * 0.97) {  // a second launch costs a few microseconds
        best_cost = c;
        best = ColumnPlan{t, c1, (TileId)u};
      }
    }
  return best;
}

inline int tile_bn(TileId t) { return kTileShapes[t].bn; }
inline int tile_wn(TileId t) { return kTileShapes[t].wn; }

template <int BM, int BN, int WGM, bool AK, bool BK, class Epi>
inline GemmProblem<BM, BN, WGM, AK, BK, Epi> problem(const bf16* A, int64_t lda, const bf16* B,
                                                     int64_t ldb, int M, int N, int K,
                                                     const Epi& epi) {
  return GemmProblem<BM, BN, WGM, AK, BK, Epi>{A, lda, B, ldb, M, N, K, epi};
}

// Launch on tile t; only the shapes in kMask are instantiated (others fail).
template <bool AK, bool BK, unsigned kMask = kAllTiles, class Epi>
inline hipError_t gemm_bf16(TileId t, const bf16* A, int64_t lda, const bf16* B, int64_t ldb,
                            int M, int N, int K, const Epi& epi, hipStream_t s) {
  if (!(kMask & (1u << t))) return hipErrorInvalidValue;
  switch (t) {
    case T256x256:
      if constexpr (kMask & (1u << T256x256))
        return launch_gemm_pp(pp_problem<256, 256, AK, BK>(A, lda, B, ldb, M, N, K, epi), s);
      break;
    case T256x224:
      if constexpr (kMask & (1u << T256x224))
        return launch_gemm(problem<256, 224, 4, AK, BK>(A, lda, B, ldb, M, N, K, epi), s);
      break;
    case T256x192:
      if constexpr (kMask & (1u << T256x192))
        return launch_gemm_pp(pp_problem<256, 192, AK, BK>(A, lda, B, ldb, M, N, K, epi), s);
      break;
    case T256x160:
      if constexpr (kMask & (1u << T256x160))
        return launch_gemm(problem<256, 160, 4, AK, BK>(A, lda, B, ldb, M, N, K, epi), s);
      break;
    case T128x128:
      if constexpr (kMask & (1u << T128x128))
        return launch_gemm_pp(pp_problem<128, 128, AK, BK>(A, lda, B, ldb, M, N, K, epi), s);
      break;
    case T256x320:
      if constexpr (kMask & (1u << T256x320))
        return launch_gemm_pp(pp_problem<256, 320, AK, BK>(A, lda, B, ldb, M, N, K, epi), s);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace lgs
