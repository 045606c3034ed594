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

// Stage R rows of a K-contiguous operand: element (r, k) at base[r * ld + k].
template <int R, bool KMAJ>
struct Stage;

template <int R>
struct Stage<R, true> {
  static_assert((R * 8) % kThreads == 0, "tile rows must be a multiple of 32");
  static constexpr int kN = R * 8 / kThreads;
  uint4 v[kN];
  __device__ __forceinline__ void load(const bf16* __restrict__ base, int64_t ld, int row0,
                                       int rows, int k0, int K, int tid) {
#pragma unroll
    for (int j = 0; j < kN; ++j) {
      const int q = tid + j * kThreads;
      const int r = q >> 3, c = q & 7;
      const int gr = row0 + r, gk = k0 + c * 8;
      if (gr < rows && gk < K)
        v[j] = *reinterpret_cast<const uint4*>(base + (int64_t)gr * ld + gk);
      else
        v[j] = make_uint4(0u, 0u, 0u, 0u);
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

// Stage R rows of an M/N-contiguous operand: element (r, k) at base[k * ld + r].
// Unit u covers rows 8q..8q+7 and k-block kb (8 k values): eight 16-byte
// loads, one per k, then an in-register 8x8 transpose.
template <int R>
struct Stage<R, false> {
  static_assert(R % 8 == 0, "tile rows must be a multiple of 8");
  static constexpr int kUnits = (R / 8) * (kBK / 8);
  static constexpr int kNU = (kUnits + kThreads - 1) / kThreads;
  uint4 v[kNU][8];
  __device__ __forceinline__ void load(const bf16* __restrict__ base, int64_t ld, int row0,
                                       int rows, int k0, int K, int tid) {
#pragma unroll
    for (int u = 0; u < kNU; ++u) {
      const int unit = tid + u * kThreads;
      if ((kUnits % kThreads) != 0 && unit >= kUnits) continue;
      const int q = unit % (R / 8), kb = unit / (R / 8);
      const int gr = row0 + q * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gk = k0 + kb * 8 + j;
        if (gr < rows && gk < K)
          v[u][j] = *reinterpret_cast<const uint4*>(base + (int64_t)gk * ld + gr);
        else
          v[u][j] = make_uint4(0u, 0u, 0u, 0u);
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
      if ((kUnits % kThreads) != 0 && unit >= kUnits) continue;
      const int q = unit % (R / 8), kb = unit / (R / 8);
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
        *reinterpret_cast<uint4*>(lds + lds_off(q * 8 + i, kb)) = o;
      }
    }
  }
};

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

template <int BM, int BN>
struct Tile {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
  static constexpr int kLdsBytes = 2 * (BM + BN) * kRowBytes;
};

// Hand every quad of a wave's accumulators to epi.quad(m, n, values).
template <int TM, int TN, class Epi>
__device__ __forceinline__ void for_quads(const f32x4 (&acc)[TM][TN], int mb, int nb, int lane,
                                          const Epi& epi) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      epi.quad(mb + i * 16 + (lane & 15), nb + j * 16 + 4 * (lane >> 4), acc[i][j]);
}

template <int BM, int BN, bool AK, bool BK, class Epi>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const bf16* __restrict__ A, int64_t lda, const bf16* __restrict__ B,
                      int64_t ldb, int M, int N, int K, Epi epi) {
  using T = Tile<BM, BN>;
  __shared__ __attribute__((aligned(16))) char smem[T::kLdsBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tmi, tni;
  tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, tmi, tni);
  const int m0 = tmi * BM, n0 = tni * BN;

  f32x4 acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  Stage<BM, AK> sa;
  Stage<BN, BK> sb;
  char* const buf0 = smem;
  char* const buf1 = smem + (BM + BN) * kRowBytes;
  const int nk = (K + kBK - 1) / kBK;

  sa.load(A, lda, m0, M, 0, K, tid);
  sb.load(B, ldb, n0, N, 0, K, tid);
  sa.store(buf0, tid);
  sb.store(buf0 + BM * kRowBytes, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const char* As = (kt & 1) ? buf1 : buf0;
    const char* Bs = As + BM * kRowBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      sa.load(A, lda, m0, M, (kt + 1) * kBK, K, tid);
      sb.load(B, ldb, n0, N, (kt + 1) * kBK, K, tid);
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
      sb.store(nxt + BM * kRowBytes, tid);
    }
    __syncthreads();
  }

  const int mb = m0 + wm * T::WM, nb = n0 + wn * T::WN;
  // Quad-wise epilogues get their quads; whole-tile epilogues (the CE
  // partials) reduce across the wave's accumulators themselves.
  if constexpr (Epi::kWholeTile)
    epi.template tile<T::TM, T::TN>(acc, mb, nb, lane);
  else
    for_quads(acc, mb, nb, lane, epi);
}

// Host-side launch of one (BM, BN) instantiation; returns the grid size.
template <int BM, int BN, bool AK, bool BK, class Epi>
inline hipError_t launch_gemm_bf16(const bf16* A, int64_t lda, const bf16* B, int64_t ldb, int M,
                                   int N, int K, const Epi& epi, hipStream_t stream) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, AK, BK, Epi>), dim3(tiles), dim3(kThreads), 0,
                     stream, A, lda, B, ldb, M, N, K, epi);
  return hipGetLastError();
}

}  // namespace lgs
