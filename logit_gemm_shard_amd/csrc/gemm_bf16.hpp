// bf16 GEMM core for gfx950: C[M,N] = sum_k A(m,k) B(k,n), fp32 accumulate,
// on the 16x16x32 bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Block: 256 threads = 4 wave64s in a 2x2 grid; block tile BM x BN, K step 64.
// Each wave owns a (BM/2) x (BN/2) tile of 16x16 accumulators.
//
// Data path per K step:
//   global --(16 B per lane, vector loads into registers)--> registers
//          --(ds_write_b128)--> LDS, double buffered, one barrier per step
//          --(ds_read_b128)--> MFMA operands.
// The next step's global loads are issued before the current step's MFMAs so
// their latency hides behind the math.
//
// LDS holds every tile "K-contiguous": row r (an m or an n) is 64 bf16 =
// 128 B = eight 16-byte chunks, chunk c stored at slot c ^ swz(r) so that
// both the fragment reads (16 consecutive rows, one chunk) and the transposed
// stores (rows 8 apart) spread over all banks.  An operand whose memory is
// K-contiguous is copied chunk by chunk; an operand whose memory is
// M/N-contiguous is loaded as 8x8 bf16 blocks (8 k-rows of 16 B) and
// transposed in registers with byte permutes before the LDS store.  After
// staging, all operand layouts run the same MFMA loop.
//
// MFMA operand roles are swapped (the B tile feeds the instruction's first
// operand) so that each lane ends with four consecutive output columns of
// one row: lane l of 16x16 tile (i, j) holds C[16i + l%16][16j + 4(l/16) + 0..3].
#pragma once

#include "common.hpp"

namespace lgs {

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kRowBytes = kBK * 2;  // 128 B per LDS row

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

// Operand tiles are read with buffer loads: the resource covers the operand
// from the tile's first row / column to its end, and the hardware range check
// returns zeros for any offset past that, so ragged edges need no branches.
// Offsets are 32-bit (operands are limited to 2 GiB, checked on the host).
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Stage R rows of a K-contiguous operand: element (r, k) at base[r * ld + k],
// `base` already offset to the tile's first row.
template <int R, bool KMAJ>
struct Stage;

template <int R>
struct Stage<R, true> {
  static_assert((R * 8) % kThreads == 0, "tile rows must be a multiple of 32");
  static constexpr int kN = R * 8 / kThreads;
  static constexpr int kSpareRows = 0;
  uint4 v[kN];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int64_t ld, int rows_left, int k0,
                                       int K, int tid) {
#pragma unroll
    for (int j = 0; j < kN; ++j) {
      const int q = tid + j * kThreads;
      const int r = q >> 3, gk = k0 + (q & 7) * 8;
      const uint32_t off = (r < rows_left && gk < K) ? (uint32_t)(r * ld + gk) * 2u : kOutOfRange;
      v[j] = buffer_load16(rs, off);
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < kN; ++j) {
      const int q = tid + j * kThreads;
      *reinterpret_cast<uint4*>(lds + lds_off(q >> 3, q & 7)) = v[j];
    }
  }
};

// Stage R rows of an M/N-contiguous operand: element (r, k) at base[k * ld + r],
// `base` already offset to the tile's first column.  Unit u covers rows
// 8q..8q+7 and k-block kb (8 k values): eight 16-byte loads, one per k, then
// an in-register 8x8 transpose.
template <int R>
struct Stage<R, false> {
  static_assert(R % 8 == 0, "tile rows must be a multiple of 8");
  static constexpr int kUnits = (R / 8) * (kBK / 8);
  static constexpr int kNU = (kUnits + kThreads - 1) / kThreads;
  // Threads past the last unit still run the same code (no divergent branch
  // around the loads): they read out of range (zeros) and write to spare rows.
  static constexpr int kSpareRows = (kUnits % kThreads) ? 8 : 0;
  uint4 v[kNU][8];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int64_t ld, int rows_left, int k0,
                                       int K, int tid) {
#pragma unroll
    for (int u = 0; u < kNU; ++u) {
      const int unit = tid + u * kThreads;
      const bool active = kSpareRows == 0 || unit < kUnits;
      const int q = unit % (R / 8), kb = unit / (R / 8);
      const bool rv = active && q * 8 < rows_left;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gk = k0 + kb * 8 + j;
        const uint32_t off = (rv && gk < K) ? (uint32_t)(gk * ld + q * 8) * 2u : kOutOfRange;
        v[u][j] = buffer_load16(rs, off);
      }
    }
  }
  __device__ __forceinline__ static unsigned word(const uint4& x, int d) {
    return d == 0 ? x.x : d == 1 ? x.y : d == 2 ? x.z : x.w;
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < kNU; ++u) {
      const int unit = tid + u * kThreads;
      const bool active = kSpareRows == 0 || unit < kUnits;
      const int q = unit % (R / 8), kb = unit / (R / 8);
      const int row0 = active ? q * 8 : R;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // output row 8q+i gathers element i of the eight k-rows; element i of a
        // row lives in 32-bit word i/2, low half for even i, high half for odd i.
        // v_perm_b32 byte selectors: 0-3 pick from the second source, 4-7 from the first.
        const unsigned sel = (i & 1) ? 0x07060302u : 0x05040100u;
        const int d = i >> 1;
        uint4 o;
        o.x = __builtin_amdgcn_perm(word(v[u][1], d), word(v[u][0], d), sel);
        o.y = __builtin_amdgcn_perm(word(v[u][3], d), word(v[u][2], d), sel);
        o.z = __builtin_amdgcn_perm(word(v[u][5], d), word(v[u][4], d), sel);
        o.w = __builtin_amdgcn_perm(word(v[u][7], d), word(v[u][6], d), sel);
        *reinterpret_cast<uint4*>(lds + lds_off(row0 + i, kb & 7)) = o;
      }
    }
  }
};

// Resource covering an operand from its tile's first row (K-contiguous) or
// first column (M/N-contiguous) to the operand's last element.
template <bool KMAJ>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const bf16* base, int64_t ld, int row0,
                                                           int rows, int K) {
  if (KMAJ)
    return make_rsrc(base + (int64_t)row0 * ld, (uint32_t)(((int64_t)(rows - 1 - row0) * ld + K) * 2));
  return make_rsrc(base + row0, (uint32_t)(((int64_t)(K - 1) * ld + (rows - row0)) * 2));
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

template <int BM, int BN, bool AK, bool BK>
struct Tile {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
  // one LDS buffer: A rows (+ spare rows), then B rows (+ spare rows)
  static constexpr int kARows = BM + Stage<BM, AK>::kSpareRows;
  static constexpr int kBufRows = kARows + BN + Stage<BN, BK>::kSpareRows;
  static constexpr int kLdsBytes = 2 * kBufRows * kRowBytes;
};

// Epilogue: each wave stages 16-row slices of its accumulators through LDS
// (free once the K loop has passed its last barrier) and hands each slice to
// the epilogue, which reads it back in whatever lane mapping suits it.  Global
// stores become 16-byte and coalesced, and the epilogue math is one compact
// loop body instead of being unrolled over every accumulator.
template <int TM, int TN, int WN, class Epi>
__device__ __forceinline__ void staged_epilogue(const f32x4 (&acc)[TM][TN], char* smem, int wave,
                                                int lane, int mb, int nb, const Epi& epi) {
  constexpr int LD = WN + 4;  // floats per staged row
  float* st = reinterpret_cast<float*>(smem) + wave * 16 * LD;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
      *reinterpret_cast<f32x4*>(st + (lane & 15) * LD + j * 16 + 4 * (lane >> 4)) = acc[i][j];
    __syncthreads();
    epi.template slice<WN, LD>(st, mb + i * 16, nb, lane);
    __syncthreads();
  }
}

// Elementwise epilogues: lane c takes row c / (WN/8), columns 8*(c % (WN/8))..+7.
template <int WN, int LD, class Epi>
__device__ __forceinline__ void elementwise_slice(const Epi& epi, const float* st, int m0, int nb,
                                                  int lane) {
  constexpr int CHUNKS = 16 * WN / 8;
#pragma unroll 1
  for (int c = lane; c < CHUNKS; c += 64) {
    const int r = c / (WN / 8), q = c - r * (WN / 8);
    float v[8];
    const f32x4 lo = *reinterpret_cast<const f32x4*>(st + r * LD + q * 8);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(st + r * LD + q * 8 + 4);
    v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
    v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
    epi.template apply<8>(m0 + r, nb + q * 8, v);
  }
}

// One GEMM of the core: C[M, N] = A B with its epilogue, block tile BM x BN.
template <int BM_, int BN_, bool AK_, bool BK_, class Epi_>
struct GemmProblem {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr bool AK = AK_, BK = BK_;
  using Epi = Epi_;
  using T = Tile<BM, BN, AK, BK>;
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

// The block's work on output tile (tmi, tni) of problem p.
template <class P>
__device__ __forceinline__ void gemm_tile(const P& p, char* smem, int tmi, int tni) {
  using T = typename P::T;
  constexpr int BM = P::BM, BN = P::BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int M = p.M, N = p.N, K = p.K;
  const int m0 = tmi * BM, n0 = tni * BN;

  f32x4 acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  Stage<BM, P::AK> sa;
  Stage<BN, P::BK> sb;
  const __amdgpu_buffer_rsrc_t ra = tile_rsrc<P::AK>(p.A, p.lda, m0, M, K);
  const __amdgpu_buffer_rsrc_t rb = tile_rsrc<P::BK>(p.B, p.ldb, n0, N, K);
  char* const buf0 = smem;
  char* const buf1 = smem + T::kBufRows * kRowBytes;
  const int nk = (K + kBK - 1) / kBK;

  sa.load(ra, p.lda, M - m0, 0, K, tid);
  sb.load(rb, p.ldb, N - n0, 0, K, tid);
  sa.store(buf0, tid);
  sb.store(buf0 + T::kARows * kRowBytes, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const char* As = (kt & 1) ? buf1 : buf0;
    const char* Bs = As + T::kARows * kRowBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      sa.load(ra, p.lda, M - m0, (kt + 1) * kBK, K, tid);
      sb.load(rb, p.ldb, N - n0, (kt + 1) * kBK, K, tid);
    }
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      bf16x8 a[T::TM], b[T::TN];
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(As + lds_off(wm * T::WM + i * 16 + (lane & 15), c));
#pragma unroll
      for (int j = 0; j < T::TN; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(Bs + lds_off(wn * T::WN + j * 16 + (lane & 15), c));
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      char* nxt = (kt & 1) ? buf0 : buf1;
      sa.store(nxt, tid);
      sb.store(nxt + T::kARows * kRowBytes, tid);
    }
    __syncthreads();
  }

  const int mb = m0 + wm * T::WM, nb = n0 + wn * T::WN;
  static_assert(4 * 16 * (T::WN + 4) * 4 <= T::kLdsBytes, "staging does not fit the LDS tiles");
  staged_epilogue<T::TM, T::TN, T::WN>(acc, smem, wave, lane, mb, nb, p.epi);
}

template <class P>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(P p) {
  __shared__ __attribute__((aligned(16))) char smem[P::T::kLdsBytes];
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
  __shared__ __attribute__((aligned(16))) char smem[kL];
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
  hipLaunchKernelGGL((gemm_bf16_kernel<P>), dim3(p.tiles()), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <class P0, class P1, class P2>
inline hipError_t launch_gemm_group3(const P0& p0, const P1& p1, const P2& p2, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_bf16_group3_kernel<P0, P1, P2>), dim3(p0.tiles() + p1.tiles() + p2.tiles()),
                     dim3(kThreads), 0, stream, p0, p1, p2);
  return hipGetLastError();
}

}  // namespace lgs
