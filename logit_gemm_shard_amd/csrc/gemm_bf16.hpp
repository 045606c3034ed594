// bf16 GEMM core for gfx950 (CDNA4): C[M,N] = sum_k A(m,k) B(k,n), fp32
// accumulation on the 32x32x16 bf16 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Block: 256 threads = 4 wave64s (one per SIMD) in a WGM x WGN grid (2x2 or
// 4x1); block tile BM x BN; K tiles of 32 (two 16-wide MFMA sub-steps).
//
// Operand tiles go global -> LDS with direct-to-LDS buffer loads (each wave
// instruction moves 64 x 16 B into 1 KB of LDS; the hardware range check
// returns zeros past an operand's end, so ragged edges need no branches).
// A ring of 3-5 LDS stages (as many as fit in 160 KB) gives the loads of a K
// tile several steps to land; one barrier per K tile.
//
// LDS layout per operand and stage:
//  * K-contiguous operand (element (r,k) at base[r*ld + k]): R rows of 32 k =
//    64 B; 16-B chunk c of row r sits at slot c ^ swz(r), swz(r) =
//    (r >> 2) & 3.  Fragment reads (32 consecutive rows, one chunk column per
//    half-wave) touch distinct banks, and since the swizzle of a row only
//    depends on r & 31, every fragment of a wave is one per-lane address plus
//    an immediate offset.
//  * M/N-contiguous operand (element (r,k) at base[k*ld + r]): 32 k-rows of R
//    values, kept in that orientation, in groups of four k-rows whose 64-byte
//    blocks (32 values) alternate, so no padding is needed for conflict-free
//    reads.  Fragments come from two ds_read_b64_tr_b16 (LDS transpose reads:
//    within each 16-lane group, lanes 4j..4j+3 address row j of a 4 x 16
//    block and lane i receives column i), so no register transposes are needed.
//
// MFMA operand roles are swapped (the B tile feeds the instruction's first
// operand) so each lane ends with runs of four consecutive output columns:
// lane l, accumulator element r of 32x32 tile (i, j) is
// C[32i + l%32][32j + 8(r/4) + 4(l/32) + r%4].
#pragma once

#include <type_traits>

#include "common.hpp"

namespace lgs {

#define LGS_AS3 __attribute__((address_space(3)))
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBK = 32;           // K per pipeline stage (two 16-wide MFMA sub-steps)
constexpr int kLdsMax = 160 * 1024;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).  The direct-to-LDS
// loads are waited for explicitly: a barrier alone does not wait for them.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(63 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0) only
}

template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// f(integral_constant<int, i>) for i = 0 .. n-1, unrolled at compile time.
template <int n, class F, int i = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (i < n) {
    f(std::integral_constant<int, i>{});
    static_for<n, F, i + 1>(static_cast<F&&>(f));
  }
}

// Per-lane parts of the loads and fragment reads are computed once per tile;
// inside the K loop an operand only moves its buffer resource forward by one
// K tile (scalar arithmetic), and every fragment read is one per-lane
// register plus a compile-time offset.
template <int R, bool KMAJ, int KT = kBK>
struct OpLayout;

// K-contiguous operand, KT (32 or 64) k values per stage: tile row r's 2 KT
// bytes form one LDS row of KT / 8 16-byte chunks.  A chunk's slot in its row
// is swizzled by the row so that the 16 rows a fragment read touches per
// 16-lane group land in distinct 16-byte slots of 256 bytes (no bank
// conflict): with 64-byte rows, rows in groups of four ((r >> 2) & 3); with
// 128-byte rows, rows in pairs ((r >> 1) & 7).  A 1 KB load fills 1024 / (2 KT)
// whole rows, each group of KT / 8 lanes reading one row's 2 KT contiguous
// bytes: 64-wide stages read whole 128-byte lines.
template <int R, int KT>
struct OpLayout<R, true, KT> {
  static_assert(R % 32 == 0, "tile rows must be a multiple of 32");
  static_assert(KT == 32 || KT == 64, "stages of 32 or 64 k");
  static constexpr int kRowBytes = 2 * KT;
  static constexpr int kChunks = KT / 8;  // 16-byte chunks per row
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;
  static constexpr int kBytes = R * kRowBytes;
  static constexpr int kInstr = kBytes / 1024;  // 1 KB loads per stage
  static constexpr uint32_t kColBytes = kRowBytes;  // LDS bytes per tile row
  __device__ __forceinline__ static int swzk(int row) { return KT == 32 ? (row >> 2) & 3 : (row >> 1) & 7; }
  // byte offset (from the tile's first row, k0 = 0) that lane `lane` of load
  // n reads; out of range past the operand's last row
  __device__ __forceinline__ static uint32_t src_off(int n, int lane, int64_t ld, int rows_left) {
    const int row = kRowsPerLoad * n + lane / kChunks;
    return row < rows_left ? (uint32_t)(row * ld + kcol(n, lane)) * 2u : kOutOfRange;
  }
  // k (within the stage) of the 8 elements that lane reads in load n
  __device__ __forceinline__ static int kcol(int n, int lane) {
    return ((lane % kChunks) ^ swzk(kRowsPerLoad * n + lane / kChunks)) * 8;
  }
  // Fragment of rows row0 + lane%32 (row0 a multiple of 32), k = 16 q +
  // 8 (lane/32) .. +7 of the stage: the swizzle only depends on lane%32, so
  // the address is lane_off(q) + kRowBytes row0.
  __device__ __forceinline__ static uint32_t lane_off(int q, int lane) {
    const int r = lane & 31;
    return (uint32_t)(r * kRowBytes + (((2 * q) ^ (lane >> 5) ^ swzk(r)) << 4));
  }
  template <int kRow0>
  __device__ __forceinline__ static bf16x8 frag(const char* p) {  // p = base + wave part + lane_off(q)
    return *reinterpret_cast<const bf16x8*>(p + kRow0 * kRowBytes);
  }
};

template <int R, int KT>
struct OpLayout<R, false, KT> {
  // Layout in LDS: k-rows in groups of four; within a group the 64-byte
  // blocks (32 columns) of the four rows alternate: columns 32 b .. 32 b + 31
  // of k-row 4g + r sit at byte 8R g + 256 b + 64 r.  A transposing fragment
  // read takes four consecutive k-rows of 32 columns per half-wave, which
  // this puts in 256 consecutive bytes (all 64 banks, no conflict) without
  // padding, so a stage holds exactly the tile's 2 KT R bytes.  Each group of
  // four lanes of a load still reads 64 contiguous bytes of one row.
  static_assert(R % 32 == 0, "tile rows must be a multiple of 32");
  static constexpr int kGroupBytes = 8 * R;     // four k-rows
  static constexpr int kGroupChunks = R / 2;    // 16-B chunks per group
  static constexpr int kBytes = KT * 2 * R;
  static constexpr int kInstr = kBytes / 1024;  // 1 KB loads per stage
  static constexpr uint32_t kColBytes = 8;      // LDS bytes per column, for column offsets that are multiples of 8
  // k-row and first column of the chunk that lane `lane` of load n fills
  __device__ __forceinline__ static void chunk_of(int n, int lane, int& krow, int& col) {
    const int p = n * 64 + lane;
    const int g = p / kGroupChunks, w = p - g * kGroupChunks;
    krow = 4 * g + ((w >> 2) & 3);
    col = 32 * (w >> 4) + 8 * (w & 3);
  }
  // byte offset (from the tile's first column, k0 = 0); out of range past the
  // operand's last column.  Rows past K fall outside the buffer resource,
  // which ends at the operand's last row.
  __device__ __forceinline__ static uint32_t src_off(int n, int lane, int64_t ld, int rows_left) {
    int krow, col;
    chunk_of(n, lane, krow, col);
    return col < rows_left ? (uint32_t)(krow * ld + col) * 2u : kOutOfRange;
  }
  __device__ __forceinline__ static int kcol(int n, int lane) {
    int krow, col;
    chunk_of(n, lane, krow, col);
    return krow;
  }
  // The same load with the tile's columns taken from two blocks of the
  // operand in alternating 32-column groups: tile column c holds column
  // (c / 64) 32 + c % 32 of the first block (c / 32 even) or of the second
  // block, `half` columns to the right (c / 32 odd).  cols_left bounds the
  // column within a block.  Tiles start at multiples of 64 columns, so a
  // tile column's group parity is that of its global column.
  __device__ __forceinline__ static uint32_t src_off_paired(int n, int lane, int64_t ld, int cols_left,
                                                           int half) {
    static_assert(R % 64 == 0, "paired tiles hold whole pairs of 32-column groups");
    int krow, c;
    chunk_of(n, lane, krow, c);
    const int col = ((c >> 6) << 5) + (c & 31);
    return col < cols_left ? (uint32_t)(krow * ld + col + ((c >> 5) & 1) * half) * 2u : kOutOfRange;
  }
  // Two ds_read_b64_tr_b16 per fragment (columns row0 .. row0+31 of the
  // wave's part, k = 16 s + 8 (lane/32) .. +7): lanes 4j..4j+3 of each
  // 16-lane group address k-row j of a 4 x 16 block.  The per-lane part:
  __device__ __forceinline__ static uint32_t lane_off(int, int lane) {
    const int g = lane >> 4, i16 = lane & 15;
    const int col = 16 * (g & 1) + 4 * (i16 & 3);  // < 32: within one 64-byte block
    return (uint32_t)(2 * (g >> 1) * kGroupBytes + (i16 >> 2) * 64 + col * 2);
  }
  // Issued as inline assembly: the compiler would otherwise treat them as
  // possibly aliasing the direct-to-LDS loads in flight and wait for all of
  // those first.  Results are only valid after an explicit lgkmcnt wait.
  // k-rows 16 kS + 4 h + ... are group 4 kS + h; column row0 (a multiple of
  // 32) starts block row0 / 32, 256 bytes each.
  template <int kS, int kRow0>
  __device__ __forceinline__ static bf16x8 frag_tr(uint32_t a) {  // a = base + wave part + lane_off
    s16x4 lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(a), "i"(4 * kS * kGroupBytes + 8 * kRow0));
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(a), "i"((4 * kS + 1) * kGroupBytes + 8 * kRow0));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// Resource covering an operand from element (row0, k0) of its tile
// (K-contiguous) or (k0, row0) (M/N-contiguous) to the operand's last element;
// empty once k0 is past K.
template <bool KMAJ>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const bf16* base, int64_t ld, int row0,
                                                           int rows, int K, int k0) {
  const int64_t first = KMAJ ? (int64_t)row0 * ld + k0 : (int64_t)k0 * ld + row0;
  const int64_t last = KMAJ ? (int64_t)(rows - 1) * ld + K : (int64_t)(K - 1) * ld + rows;  // one past
  const int64_t bytes = k0 < K ? (last - first) * 2 : 0;
  return make_rsrc(base + first, (uint32_t)bytes);
}

// Block index -> output tile.  The hardware deals consecutive workgroup ids
// round-robin over the 8 XCDs (each with its own L2); renumber so that every
// XCD owns a contiguous run of ids, then walk tiles in groups of kGroupM tile
// rows so that a run shares a few A row-panels and B column-panels in its L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

__device__ __forceinline__ void tile_of_block(int pid, int nblk, int tiles_m, int tiles_n,
                                              int& tm, int& tn) {
  if (nblk % kXcds == 0) {
    const int per = nblk / kXcds;
    pid = (pid % kXcds) * per + pid / kXcds;
  }
  const int width = kGroupM * tiles_n;
  const int group = pid / width;
  const int first = group * kGroupM;
  const int gsz = min(tiles_m - first, kGroupM);
  const int in = pid - group * width;
  tm = first + in % gsz;
  tn = in / gsz;
}

// An epilogue with kPaired = true takes the B operand as two column blocks
// read in alternating 32-column groups (OpLayout::src_off_paired), so that
// each wave's accumulator tiles come in pairs (2q, 2q+1) over the same output
// columns; only the ping-pong core (gemm_pp.hpp) builds it.
template <class E, class = void>
struct PairedEpi : std::false_type {};
template <class E>
struct PairedEpi<E, std::void_t<decltype(E::kPaired)>> : std::bool_constant<E::kPaired> {};

template <int BM, int BN, int WGM, bool AK, bool BK>
struct Tile {
  static constexpr int WGN = 4 / WGM;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  using LA = OpLayout<BM, AK>;
  using LB = OpLayout<BN, BK>;
  static constexpr int kStage = LA::kBytes + LB::kBytes;
  static constexpr int kStages = kLdsMax / kStage < 5 ? kLdsMax / kStage : 5;
  static_assert(kStages >= 3, "need at least three stages");
  static constexpr int kLdsBytes = kStages * kStage;
};

// Elementwise epilogues: each wave stages 32-row slices of its accumulators
// through its own region of LDS (free once the K loop has passed its last
// barrier) and reads each slice back as 8-column chunks: chunk c of a slice is
// row c / (WN/8), columns 8 (c % (WN/8)) .. +7, and lane l takes chunks l,
// l + 64, ...  Stores of 16 bytes per lane are then contiguous along rows.
// Only the wave itself touches its region, so a slice needs no block barrier:
// LDS requests of one wave complete in order, and the waits below make the
// staged values visible to the other lanes before they are read.
// Epilogues with an input of the output's shape (Epi::kLoads) get the chunk's
// 8 input values loaded one slice ahead, so that their memory latency overlaps
// the staging and math of the slice before.
template <int WN, int ROWS>
struct SliceShape {
  static constexpr int kCpr = WN / 8;          // chunks per row
  static constexpr int kChunks = ROWS * kCpr;  // chunks per slice
  static constexpr int kPerLane = kChunks / 64;
  static_assert(kChunks % 64 == 0, "wave tile width must be a multiple of 32");
};

__device__ __forceinline__ void wave_lds_sync() {
  wait_lgkm0();
  __builtin_amdgcn_wave_barrier();
}

// Slices are ROWS = 32 rows (one MFMA row tile), or 16 (half a row tile,
// written by the lanes holding those rows) where a wave's 32 x (WN+4) floats
// times the block's waves would not fit in the LDS ring.
template <int TM, int TN, int WN, int ROWS, class Epi>
__device__ __forceinline__ void staged_epilogue(const f32x16 (&acc)[TM][TN], char* smem, int wave,
                                                int lane, int mb, int nb, const Epi& epi) {
  static_assert(ROWS == 32 || ROWS == 16, "slice rows");
  using SS = SliceShape<WN, ROWS>;
  using In = std::decay_t<decltype(epi.load8(0, 0))>;  // the chunk's input values
  constexpr int LD = WN + 4;  // floats per staged row
  constexpr int kHalves = 32 / ROWS;
  float* st = reinterpret_cast<float*>(smem) + wave * ROWS * LD;
  In in[2][SS::kPerLane];
  auto prefetch = [&](int sl, In(&dst)[SS::kPerLane]) {
#pragma unroll
    for (int k = 0; k < SS::kPerLane; ++k) {
      const int c = lane + 64 * k, r = c / SS::kCpr, q = c - r * SS::kCpr;
      dst[k] = epi.load8(mb + ROWS * sl + r, nb + 8 * q);
    }
  };
  if constexpr (Epi::kLoads) prefetch(0, in[0]);
  const int lrow = lane & 31;
#pragma unroll
  for (int sl = 0; sl < TM * kHalves; ++sl) {
    const int i = sl / kHalves, h = sl % kHalves;
    if constexpr (Epi::kLoads)
      if (sl + 1 < TM * kHalves) prefetch(sl + 1, in[(sl + 1) & 1]);
    if (kHalves == 1 || (lrow >> 4) == h) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4*>(st + (lrow - ROWS * h) * LD + j * 32 + 8 * q + 4 * (lane >> 5)) =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    }
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < SS::kPerLane; ++k) {
      const int c = lane + 64 * k, r = c / SS::kCpr, q = c - r * SS::kCpr;
      float v[8];
      const f32x4 lo = *reinterpret_cast<const f32x4*>(st + r * LD + q * 8);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(st + r * LD + q * 8 + 4);
      v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
      v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
      epi.apply8(mb + ROWS * sl + r, nb + 8 * q, v, in[sl & 1][k]);
    }
    wave_lds_sync();
  }
}

// Rows per staged slice for `waves` waves of width WN in `lds` bytes.
template <int WN>
constexpr int stage_rows(int waves, int lds) {
  return waves * 32 * (WN + 4) * 4 <= lds ? 32 : 16;
}

// An epilogue with a large per-chunk input may cap the slice height
// (Epi::kMaxRows = 16), which halves the registers its prefetched inputs take.
template <class E, class = void>
struct EpiMaxRows : std::integral_constant<int, 32> {};
template <class E>
struct EpiMaxRows<E, std::void_t<decltype(E::kMaxRows)>> : std::integral_constant<int, E::kMaxRows> {};

template <class Epi, int WN>
constexpr int slice_rows(int waves, int lds) {
  return stage_rows<WN>(waves, lds) < EpiMaxRows<Epi>::value ? stage_rows<WN>(waves, lds)
                                                               : EpiMaxRows<Epi>::value;
}

// One GEMM of the core: C[M, N] = A B with its epilogue, block tile BM x BN.
template <int BM_, int BN_, int WGM_, bool AK_, bool BK_, class Epi_>
struct GemmProblem {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_;
  static constexpr bool AK = AK_, BK = BK_;
  using Epi = Epi_;
  using T = Tile<BM, BN, WGM, AK, BK>;
  const bf16* A;
  int64_t lda;
  const bf16* B;
  int64_t ldb;
  int M, N, K;
  Epi epi;
  __host__ __device__ int tiles_m() const { return (M + BM - 1) / BM; }
  __host__ __device__ int tiles_n() const { return (N + BN - 1) / BN; }
  __host__ __device__ int tiles() const { return tiles_m() * tiles_n(); }
};

// Debug builds: every span problem p's blocks touch (both operands up to
// their last element, and each buffer of the epilogue) lies inside a buffer
// the entry point validated, and the tiles cover the output.
template <class P>
inline void debug_problem(const P& p) {
  LGS_CHECK(p.M > 0 && p.N > 0 && p.K > 0);
  LGS_CHECK((int64_t)p.tiles_m() * P::BM >= p.M && (int64_t)p.tiles_n() * P::BN >= p.N);
  LGS_NEED(p.A, P::AK ? debug::mat_bytes(p.M, p.lda, p.K, 2) : debug::mat_bytes(p.K, p.lda, p.M, 2),
           "GEMM operand A");
  LGS_NEED(p.B, P::BK ? debug::mat_bytes(p.N, p.ldb, p.K, 2) : debug::mat_bytes(p.K, p.ldb, p.N, 2),
           "GEMM operand B");
  p.epi.debug_spans(P::BN);
}

// The block's work on output tile (tmi, tni) of problem p.
template <class P>
__device__ __forceinline__ void gemm_tile(const P& p, char* smem, int tmi, int tni) {
  using T = typename P::T;
  using LA = typename T::LA;
  using LB = typename T::LB;
  static_assert(!PairedEpi<typename P::Epi>::value, "paired epilogues run on the ping-pong core");
  constexpr int TM = T::TM, TN = T::TN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WGN, wn = wave % T::WGN;
  const int M = p.M, N = p.N, K = p.K;
  const int m0 = tmi * P::BM, n0 = tni * P::BN;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + kBK - 1) / kBK;
  constexpr int IA = (LA::kInstr + 3) / 4, IB = (LB::kInstr + 3) / 4;
  constexpr int kPer = IA + IB;  // loads per tile per wave

  // Direct-to-LDS loads.  Load n of an operand fills bytes [1024 n, 1024 n +
  // 1024) of its region in a stage; waves take every 4th load (a duplicate of
  // the last load where the count is not a multiple of four: the same bytes
  // written twice with the same values).  The per-lane source offsets are
  // fixed for the tile; each K tile moves the buffer resources instead.  A
  // K-contiguous operand's last, partial K tile masks its lanes past K.
  uint32_t offa[IA], offb[IB];
  int kca[IA], kcb[IB];
#pragma unroll
  for (int t = 0; t < IA; ++t) {
    const int n = min(wave + 4 * t, LA::kInstr - 1);
    offa[t] = LA::src_off(n, lane, p.lda, M - m0);
    kca[t] = LA::kcol(n, lane);
  }
#pragma unroll
  for (int t = 0; t < IB; ++t) {
    const int n = min(wave + 4 * t, LB::kInstr - 1);
    offb[t] = LB::src_off(n, lane, p.ldb, N - n0);
    kcb[t] = LB::kcol(n, lane);
  }
  __amdgpu_buffer_rsrc_t ra, rb;
  bool kfull = true;
  auto load_prep = [&](int kt) {
    const int k0 = kt * kBK;
    ra = tile_rsrc<P::AK>(p.A, p.lda, m0, M, K, k0);
    rb = tile_rsrc<P::BK>(p.B, p.ldb, n0, N, K, k0);
    kfull = k0 + kBK <= K;
  };
  auto load_one = [&](int st, int u, int kt) {
    char* base = smem + st * T::kStage;
    if (u < IA) {
      const int n = min(wave + 4 * u, LA::kInstr - 1);
      uint32_t off = offa[u];
      if (P::AK && !kfull) off = kt * kBK + kca[u] < K ? off : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LGS_AS3 void*)(base + n * 1024), 16, (int)off, 0, 0, 0);
    } else {
      const int t = u - IA, n = min(wave + 4 * t, LB::kInstr - 1);
      uint32_t off = offb[t];
      if (P::BK && !kfull) off = kt * kBK + kcb[t] < K ? off : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (LGS_AS3 void*)(base + LA::kBytes + n * 1024), 16, (int)off, 0, 0, 0);
    }
  };

  // Fragment reads: one per-lane register per operand and sub-step, plus the
  // stage and a compile-time offset per fragment.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LGS_AS3 char*)smem;
  const uint32_t fa_lane[2] = {LA::lane_off(0, lane) + (uint32_t)(wm * T::WM) * LA::kColBytes,
                               LA::lane_off(1, lane) + (uint32_t)(wm * T::WM) * LA::kColBytes};
  const uint32_t fb_lane[2] = {LB::lane_off(0, lane) + (uint32_t)(wn * T::WN) * LB::kColBytes + LA::kBytes,
                               LB::lane_off(1, lane) + (uint32_t)(wn * T::WN) * LB::kColBytes + LA::kBytes};
  bf16x8 fa[2][TM], fb[2][TN];
  // fragments of sub-step s of the tile in stage st into buffer d
  auto read_frags = [&](int st, auto s_c, int d) {
    constexpr int s = decltype(s_c)::value;
    const uint32_t sb = (uint32_t)(st * T::kStage);
    if constexpr (P::AK) {
      const char* pa = smem + sb + fa_lane[s];
      static_for<TM>([&](auto i) { fa[d][i] = LA::template frag<32 * decltype(i)::value>(pa); });
    } else {
      const uint32_t a = lds0 + sb + fa_lane[0];
      static_for<TM>([&](auto i) { fa[d][i] = LA::template frag_tr<s, 32 * decltype(i)::value>(a); });
    }
    if constexpr (P::BK) {
      const char* pb = smem + sb + fb_lane[s];
      static_for<TN>([&](auto j) { fb[d][j] = LB::template frag<32 * decltype(j)::value>(pb); });
    } else {
      const uint32_t b = lds0 + sb + fb_lane[0];
      static_for<TN>([&](auto j) { fb[d][j] = LB::template frag_tr<s, 32 * decltype(j)::value>(b); });
    }
  };
  auto mma = [&](int d) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[d][j], fa[d][i], acc[i][j], 0, 0, 0);
  };

  // Ring of S stages of 32-wide K tiles.  Step kt (tile kt in stage kt % S):
  // read the fragments of its second 16-wide sub-step, MFMAs on the first;
  // wait for this wave's loads of tile kt+1, barrier (tile kt+1 visible to all
  // waves; every read of tile kt-1's stage retired), start loading tile
  // kt+S-1 into that stage; read tile kt+1's first fragments, MFMAs on the
  // second sub-step.  Loads thus have S-2 steps to land.  Tiles past the end
  // load zeros (empty resources), so the loop body has no data branches.
  constexpr int S = T::kStages;
#pragma unroll
  for (int t = 0; t < S - 1; ++t) {
    load_prep(t);
#pragma unroll
    for (int u = 0; u < kPer; ++u) load_one(t, u, t);
  }
  wait_vmcnt<(S - 2) * kPer>();  // this wave's loads of tile 0 done
  __syncthreads();
  read_frags(0, std::integral_constant<int, 0>{}, 0);
  wait_lgkm0();
  int st_cur = 0;
  constexpr int kMfma = TM * TN;
  for (int kt = 0; kt < nk; ++kt) {
    const int st_nxt = st_cur + 1 == S ? 0 : st_cur + 1;
    const int st_free = st_cur == 0 ? S - 1 : st_cur - 1;
    // first sub-step: issue the second sub-step's fragment reads, then the
    // first sub-step's MFMAs (and the resources of the next loads)
    read_frags(st_cur, std::integral_constant<int, 1>{}, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(0);
    load_prep(kt + S - 1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(S - 3) * kPer>();  // this wave's loads of tile kt+1 done
    __syncthreads();
    wait_lgkm0();                  // second sub-step's fragments in registers
    // second sub-step: tile kt+1's first fragment reads, then its MFMAs with
    // the loads of tile kt+S-1 issued between them
    read_frags(st_nxt, std::integral_constant<int, 0>{}, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kPer; ++u) load_one(st_free, u, kt + S - 1);
    mma(1);
#pragma unroll
    for (int q = 0; q < kMfma; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // 1 MFMA
      if (q < kPer) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 direct-to-LDS load
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm0();                  // tile kt+1's first fragments in registers
    st_cur = st_nxt;
  }
  wait_vmcnt<0>();  // the (zero) loads past the end must land before LDS is reused

  const int mb = m0 + wm * T::WM, nb = n0 + wn * T::WN;
  if constexpr (P::Epi::kDirect) {
    // The epilogue reads the accumulators in their MFMA lane layout.
    p.epi.template direct<TM, TN, T::WN>(acc, mb, nb, lane);
  } else {
    __syncthreads();  // every wave is past its last read of the LDS ring
    constexpr int R = slice_rows<typename P::Epi, T::WN>(4, T::kLdsBytes);
    static_assert(4 * R * (T::WN + 4) * 4 <= T::kLdsBytes, "staging does not fit the LDS tiles");
    staged_epilogue<TM, TN, T::WN, R>(acc, smem, wave, lane, mb, nb, p.epi);
  }
}

template <class P>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(P p) {
  __shared__ __attribute__((aligned(1024))) char smem[P::T::kLdsBytes];
  int tmi, tni;
  tile_of_block(blockIdx.x, gridDim.x, p.tiles_m(), p.tiles_n(), tmi, tni);
  gemm_tile(p, smem, tmi, tni);
}

// Several independent GEMMs in one launch: blocks [0, p0.tiles()) work on p0,
// the next p1.tiles() on p1, the rest on p2.  Put the longest-K problems
// first: blocks start in index order, so the short tiles of the later
// problems fill the compute units the long ones leave free.
template <class P0, class P1, class P2>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_group3_kernel(P0 p0, P1 p1, P2 p2) {
  constexpr int kL0 = P0::T::kLdsBytes, kL1 = P1::T::kLdsBytes, kL2 = P2::T::kLdsBytes;
  constexpr int kL = kL0 > kL1 ? (kL0 > kL2 ? kL0 : kL2) : (kL1 > kL2 ? kL1 : kL2);
  __shared__ __attribute__((aligned(1024))) char smem[kL];
  int pid = blockIdx.x, tmi, tni;
  const int t0 = p0.tiles(), t1 = p1.tiles();
  if (pid < t0) {
    tile_of_block(pid, t0, p0.tiles_m(), p0.tiles_n(), tmi, tni);
    gemm_tile(p0, smem, tmi, tni);
  } else if ((pid -= t0) < t1) {
    tile_of_block(pid, t1, p1.tiles_m(), p1.tiles_n(), tmi, tni);
    gemm_tile(p1, smem, tmi, tni);
  } else {
    pid -= t1;
    tile_of_block(pid, p2.tiles(), p2.tiles_m(), p2.tiles_n(), tmi, tni);
    gemm_tile(p2, smem, tmi, tni);
  }
}

template <class P>
inline hipError_t launch_gemm(const P& p, hipStream_t stream) {
  debug_problem(p);
  LGS_LAUNCH((gemm_bf16_kernel<P>), dim3(p.tiles()), dim3(kThreads), 0, stream, p);
  return LGS_LAUNCH_STATUS();
}

template <class P0, class P1, class P2>
inline hipError_t launch_gemm_group3(const P0& p0, const P1& p1, const P2& p2, hipStream_t stream) {
  debug_problem(p0);
  debug_problem(p1);
  debug_problem(p2);
  LGS_LAUNCH((gemm_bf16_group3_kernel<P0, P1, P2>), dim3(p0.tiles() + p1.tiles() + p2.tiles()), dim3(kThreads),
             0, stream, p0, p1, p2);
  return LGS_LAUNCH_STATUS();
}

}  // namespace lgs
