// 8-wave "ping-pong" variant of the bf16 GEMM core (the LDS layouts of
// gemm_bf16.hpp with 64-wide stages; the same epilogues).
//
// Why: on gfx950 the data an LDS read returns to a wave costs that wave's
// own MFMA issue about 25 cycles per KB, while reads returning to ANOTHER
// wave on the same SIMD cost the MFMA wave nothing (measured).  With one wave
// per SIMD the fragment traffic of a 128x128 wave tile (16 KB per 32-wide K
// tile) therefore adds ~40% to its 1024 MFMA cycles.  Here each SIMD runs two
// waves, one from each of two groups (waves w and w+4 share a SIMD), and the
// groups alternate between phases, separated by block barriers: while one
// group multiplies the K half whose fragments it holds in registers, the
// other reads its fragments of that half from LDS.  The matrix cores of a
// SIMD then see back-to-back MFMAs of one wave or the other.
//
// Block: 512 threads; block tile BM x BN, wave w owns rows (w & 3) BM/4 and
// columns (w >> 2) BN/2 (group g = w >> 2 owns one column half), or, for
// 256x256 tiles with a K-contiguous A and an N-contiguous B, rows g BM/2 and
// columns (w & 3) BN/4 (group g owns one row half; PPTile::kRowGroups).
// The LDS ring holds two stages of 64 k; each stage is two 32-wide halves,
// and half kt is read by group 0 in phase 2kt and by group 1 in phase 2kt+1,
// and computed by each in its next phase.  The stage bookkeeping is at the
// K loop.
#pragma once

#include "gemm_bf16.hpp"

namespace lgs {

constexpr int kPPWaves = 8;

// s_barrier without the memory fence of __syncthreads(): that fence makes the
// compiler wait for every direct-to-LDS load in flight (vmcnt(0)) before the
// barrier, which would drain the load pipeline at every phase.  The waits the
// pipeline needs are explicit (vmcnt for this wave's loads, lgkmcnt for its
// fragment reads); the empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
constexpr int kPPThreads = 64 * kPPWaves;
template <int BM, int BN, bool AK, bool BK>
struct PPTile {
  // 256x256 tiles with a K-contiguous A and an N-contiguous B: waves in a
  // 2 x 4 grid (each group owns a row half), so the B fragments, read with
  // the slower transposing reads, are read twice per K tile instead of four
  // times (and A's 128-bit reads four times instead of twice).
  static constexpr bool kRowGroups = BM == 256 && BN == 256 && AK && !BK;
  static constexpr int WM = kRowGroups ? BM / 2 : BM / 4, WN = kRowGroups ? BN / 4 : BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  // A K-contiguous A is staged 64 k at a time: its LDS rows are then 128
  // bytes and every load reads whole cache lines (with 32 k each 1 KB load
  // touches 16 half lines, and a K tile's loads with both operands
  // K-contiguous took longer than its MFMAs).  Its ring holds three such
  // stages, so a stage is loaded six phases or more before it is read (with
  // two, about four: measured much slower).  Every other operand is staged
  // 32 k at a time in a ring of up to four (four measured faster than five:
  // fewer loads in flight, less congestion).  Each operand has its own LDS
  // region.
  static constexpr bool kAPairs = AK;
  using LA = OpLayout<BM, AK, kAPairs ? 64 : 32>;
  using LB = OpLayout<BN, BK, 32>;
  static constexpr int kAStages = kAPairs ? 3 : 4;
  static constexpr int kABytes = kAStages * LA::kBytes;
  static constexpr int kBFit = (kLdsMax - kABytes) / LB::kBytes;
  static constexpr int kBStages = kBFit < 4 ? kBFit : 4;
  static_assert(kBStages >= 3, "B needs a ring of at least three stages");
  static constexpr int kLdsBytes = kABytes + kBStages * LB::kBytes;
  // loads per stage per wave (every 8th load; a count that is not a
  // multiple of 8 duplicates the last load in some waves)
  static constexpr int IA = (LA::kInstr + kPPWaves - 1) / kPPWaves;
  static constexpr int IB = (LB::kInstr + kPPWaves - 1) / kPPWaves;
  // A 64-k A stage's loads are split over the two read phases of the
  // stage before it (IA / 2 per wave in each), so that every read phase
  // issues the same number of loads.
  static_assert(!kAPairs || IA % 2 == 0, "a 64-k A stage splits its loads evenly over two halves");
  static constexpr int kAPerHalf = kAPairs ? IA / 2 : IA;
};

// A wave's load sequence, simulated at compile time.  The prologue issues
// A's stages 0 .. kAStages-2 and B's tiles 0 .. kBStages-2 in the order the
// halves need them (A's stage first on a tie).  The read phase of half j
// then issues A's part (64-k stages: loads [0, IA/2) of stage j/2 +
// kAStages - 1 for even j, loads [IA/2, IA) of it for odd j; 32-k stages:
// tile j + kAStages - 1) and B's tile j + kBStages - 1, A's part first if
// a_first.  pp_after(h) counts the loads issued after the last one that
// half h reads, when the wave has issued everything up to the read phase of
// half h - 1 (h = 0: the prologue alone).  A phase that ends with vmcnt <= n
// (and a block barrier) guarantees every load of the next half when
// n <= pp_after(h).
template <class T>
constexpr int pp_after(int h, bool a_first) {
  int issued = 0, needed_end = 0;
  const int need_a = T::kAPairs ? h / 2 : h, need_b = h;
  auto note = [&](bool ok) {
    if (ok && issued > needed_end) needed_end = issued;
  };
  // prologue, by the half that first reads each stage
  const int last = 2 * (T::kAStages + T::kBStages);
  for (int half = 0; half < last; ++half) {
    const int sa = T::kAPairs ? half / 2 : half;
    const bool a_now = sa < T::kAStages - 1 && (T::kAPairs ? half % 2 == 0 : true);
    if (a_now) {
      issued += T::IA;
      note(sa == need_a);
    }
    if (half < T::kBStages - 1) {
      issued += T::IB;
      note(half == need_b);
    }
  }
  for (int j = 0; j < h; ++j) {
    const int sa = T::kAPairs ? j / 2 + T::kAStages - 1 : j + T::kAStages - 1, tb = j + T::kBStages - 1;
    // a 64-k stage is complete after its odd half's part
    const bool a_done = !T::kAPairs || j % 2 == 1;
    for (int o = 0; o < 2; ++o) {
      if ((o == 0) == a_first) {
        issued += T::kAPerHalf;
        note(a_done && sa == need_a);
      } else {
        issued += T::IB;
        note(tb == need_b);
      }
    }
  }
  return issued - needed_end;
}

// The in-loop wait: the smallest pp_after over the halves from the first on.
template <class T>
constexpr int pp_wait_count(bool a_first) {
  int n = 1 << 30;
  for (int h = 1; h < 64; ++h) n = pp_after<T>(h, a_first) < n ? pp_after<T>(h, a_first) : n;
  return n;
}

template <int BM_, int BN_, bool AK_, bool BK_, class Epi_>
struct PPProblem {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr bool AK = AK_, BK = BK_;
  using Epi = Epi_;
  using T = PPTile<BM, BN, AK, BK>;
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

// No in-launch reduction: the tile's accumulators go straight to its epilogue.
struct NoFix {
  static constexpr bool kActive = false;
};

// In-launch reduction of a tile whose K range is split into `parts` blocks of
// the same launch.  Every part writes its fp32 accumulators to its slot of the
// tile's partial buffer (in the accumulator lane layout: one 16-byte vector
// per lane per 4 values, so every access is a contiguous 1 KB per wave) and
// counts itself in the tile's counter.  The part that arrives last adds all
// slots in part order, which makes the sum independent of the arrival order,
// and continues to the epilogue; the others end.  No part waits for another.
//
// The parts may run on different XCDs, each with its own L2.  The slots are
// written and read with device-scope accesses (sc1: written through to, and
// read from, the memory side), and each wave's slot stores have completed
// (vmcnt 0) before the block counts itself, so the last part reads every
// slot whole.  No L2-wide fence is needed: one (write back and invalidate the
// XCD's whole L2) costs the other tiles streaming through that L2 their
// cached operand panels.  The counter must be 0 at launch; the last part
// sets it back to 0.
struct KPartFix {
  static constexpr bool kActive = true;
  static constexpr int kDeviceScope = 16;  // buffer cache policy: sc1
  float* part;  // this tile's slots: [parts][kPPWaves][TM][TN][4][64] f32x4
  int* count;   // this tile's arrival counter
  int s, parts;
  template <int TM, int TN>
  __device__ __forceinline__ bool reduce(f32x16 (&acc)[TM][TN], char* smem, int wave, int lane) const {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    constexpr int kWaveBytes = TM * TN * 4 * 64 * 16;
    constexpr int kPartBytes = kPPWaves * kWaveBytes;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(part, (uint32_t)(parts * kPartBytes));
    const int base = wave * kWaveBytes + lane * 16;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs,
                                                 s * kPartBytes + base + ((i * TN + j) * 4 + q) * 1024, 0,
                                                 kDeviceScope);
        }
    wait_vmcnt<0>();  // this wave's slot stores are complete
    __syncthreads();
    int* flag = reinterpret_cast<int*>(smem);  // the LDS ring is free: every wave is past the K loop
    if (threadIdx.x == 0) {
      const int last = atomicAdd(count, 1) == parts - 1;
      if (last) atomicExch(count, 0);
      *flag = last;
    }
    __syncthreads();
    const bool last = *flag != 0;
    __syncthreads();
    if (!last) return false;
    // Slot 0, then slots 1, 2, ... added in order; each slot's loads are
    // issued together.
    for (int u = 0; u < parts; ++u) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 t = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, u * kPartBytes + base + ((i * TN + j) * 4 + q) * 1024,
                                                             0, kDeviceScope));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = u ? acc[i][j][4 * q + e] + t[e] : t[e];
          }
    }
    return true;
  }
};

template <class P, class Fix = NoFix>
__device__ __forceinline__ void gemm_tile_pp(const P& p, char* smem, int tmi, int tni, const Fix& fix = Fix{}) {
  using T = typename P::T;
  using LA = typename T::LA;
  using LB = typename T::LB;
  constexpr int TM = T::TM, TN = T::TN;
  constexpr bool kPaired = PairedEpi<typename P::Epi>::value;
  static_assert(!kPaired || (!P::BK && TN % 2 == 0),
                "paired tiles: an N-contiguous B and whole pairs of 32-column groups per wave");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wm = T::kRowGroups ? grp : wave & 3, wn = T::kRowGroups ? wave & 3 : grp;
  const int M = p.M, N = p.N, K = p.K;
  const int m0 = tmi * P::BM, n0 = tni * P::BN;
  // B columns the tile reads: BN of them from n0, or for a paired epilogue
  // BN / 2 from each of the two blocks (the second `half` columns on).
  int bcol0 = n0, bcols = N;
  if constexpr (kPaired) {
    bcol0 = tni * (P::BN / 2);
    bcols = 2 * p.epi.half;
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + kBK - 1) / kBK;  // 32-wide halves (one phase each)
  constexpr int IA = T::IA, IB = T::IB;
  constexpr int KA = T::kAPairs ? 64 : 32;  // k per A stage
  // A's part of a read phase first, or B's tile: whichever lets the phase
  // ends leave more loads in flight.
  constexpr bool kAF = pp_wait_count<T>(true) >= pp_wait_count<T>(false);

  // Direct-to-LDS loads: load n of an operand's stage fills bytes
  // [1024 n, +1024) of the stage; waves take every 8th load (duplicating the
  // last one where the count is not a multiple of eight).  Offsets fixed per
  // tile; the buffer resources move per stage; a K-contiguous operand's
  // partial last stage masks its lanes past K.  A K-contiguous operand's k
  // (within the stage) of a lane's 8 elements is the same in all of a wave's
  // loads: with 64-byte rows it depends on the lane only, with 128-byte rows
  // also on the parity of the load index, which is the wave's for loads
  // n = wave + 8t (a 64-k A stage holds a multiple of 8 loads).
  static_assert(!T::kAPairs || LA::kInstr % kPPWaves == 0, "whole loads per wave in a 64-k stage");
  uint32_t offa[IA], offb[IB];
  const int kca = LA::kcol(wave, lane), kcb = LB::kcol(wave, lane);
#pragma unroll
  for (int t = 0; t < IA; ++t) offa[t] = LA::src_off(min(wave + kPPWaves * t, LA::kInstr - 1), lane, p.lda, M - m0);
#pragma unroll
  for (int t = 0; t < IB; ++t) {
    const int n = min(wave + kPPWaves * t, LB::kInstr - 1);
    if constexpr (kPaired)
      offb[t] = LB::src_off_paired(n, lane, p.ldb, p.epi.half - bcol0, p.epi.half);
    else
      offb[t] = LB::src_off(n, lane, p.ldb, N - n0);
  }
  // A's stage st (k from st KA) into slot st % kAStages of A's region, B's
  // tile tl (k from 32 tl) into slot tl % kBStages of B's region.  Stages
  // past K load nothing (empty resource: zeros), which keeps every wave's
  // load count per half fixed for the vmcnt waits.
  // loads [T0, T1) of the wave's share of A's stage st
  auto load_a = [&](int st, auto t0_c, auto t1_c) {
    constexpr int T0 = decltype(t0_c)::value, T1 = decltype(t1_c)::value;
    const int k0 = st * KA;
    const __amdgpu_buffer_rsrc_t ra = tile_rsrc<P::AK>(p.A, p.lda, m0, M, K, k0);
    const bool kfull = k0 + KA <= K;
    char* base = smem + (st % T::kAStages) * LA::kBytes;
#pragma unroll
    for (int t = T0; t < T1; ++t) {
      const int n = min(wave + kPPWaves * t, LA::kInstr - 1);
      uint32_t off = offa[t];
      if (P::AK && !kfull) off = k0 + kca < K ? off : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LGS_AS3 void*)(base + n * 1024), 16, (int)off, 0, 0, 0);
    }
  };
  auto load_b = [&](int tl) {
    const int k0 = tl * kBK;
    const __amdgpu_buffer_rsrc_t rb = tile_rsrc<P::BK>(p.B, p.ldb, bcol0, bcols, K, k0);
    const bool kfull = k0 + kBK <= K;
    char* base = smem + T::kABytes + (tl % T::kBStages) * LB::kBytes;
#pragma unroll
    for (int t = 0; t < IB; ++t) {
      const int n = min(wave + kPPWaves * t, LB::kInstr - 1);
      uint32_t off = offb[t];
      if (P::BK && !kfull) off = k0 + kcb < K ? off : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (LGS_AS3 void*)(base + n * 1024), 16, (int)off, 0, 0, 0);
    }
  };

  // Fragments of both 16-wide sub-steps of half kt.  A transposing read's
  // per-lane offset does not depend on the sub-step (it goes into the
  // instruction's offset).  A K-contiguous operand's does, through the chunk
  // swizzle only: in sub-step q of its stage the chunk bits of the byte
  // offset are (2q) ^ (lane / 32) ^ swizzle(row), so the offset is that of
  // sub-step 0 with 32 q xor-ed in (every other part of the address is a
  // multiple of 2 KT bytes).  For a 64-k A stage, half kt is sub-steps
  // 2 (kt % 2) and 2 (kt % 2) + 1.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LGS_AS3 char*)smem;
  const uint32_t fa_lane = LA::lane_off(0, lane) + (uint32_t)(wm * T::WM) * LA::kColBytes;
  const uint32_t fb_lane = LB::lane_off(0, lane) + (uint32_t)(wn * T::WN) * LB::kColBytes + T::kABytes;
  bf16x8 fa[2][TM], fb[2][TN];
  auto read_sub = [&](uint32_t ab, uint32_t bb, auto qa_c, auto s_c) {
    constexpr int qa = decltype(qa_c)::value, s = decltype(s_c)::value;
    if constexpr (P::AK) {
      const char* pa = smem + ((ab + fa_lane) ^ (32u * qa));
      static_for<TM>([&](auto i) { fa[s][i] = LA::template frag<32 * decltype(i)::value>(pa); });
    } else {
      const uint32_t a = lds0 + ab + fa_lane;
      static_for<TM>([&](auto i) { fa[s][i] = LA::template frag_tr<qa, 32 * decltype(i)::value>(a); });
    }
    if constexpr (P::BK) {
      const char* pb = smem + ((bb + fb_lane) ^ (32u * s));
      static_for<TN>([&](auto j) { fb[s][j] = LB::template frag<32 * decltype(j)::value>(pb); });
    } else {
      const uint32_t b = lds0 + bb + fb_lane;
      static_for<TN>([&](auto j) { fb[s][j] = LB::template frag_tr<s, 32 * decltype(j)::value>(b); });
    }
  };
  // Read phase of half kt: this wave's fragments, then its loads of the
  // stages that enter the rings now (A's stage kt/2 + kAStages - 1 for even
  // kt with 64-k stages, else kt + kAStages - 1; B's tile kt + kBStages - 1),
  // then wait for the fragments.  The fragment reads overwrite registers that
  // this wave's previous MFMAs read as sources: on gfx950 an MFMA reads its A
  // and B operands at issue, so overwriting them afterwards needs no wait
  // states (the compiler's own hazard model inserts none for a DS or VALU
  // write there).  Only the compiler barrier below is needed.
  auto read_phase = [&](int kt, auto half_c) {
    constexpr int half = decltype(half_c)::value;
    asm volatile("" ::: "memory");
    const uint32_t ab = (uint32_t)(((T::kAPairs ? kt >> 1 : kt) % T::kAStages) * LA::kBytes);
    const uint32_t bb = (uint32_t)((kt % T::kBStages) * LB::kBytes);
    constexpr int q0 = T::kAPairs ? 2 * half : 0;
    read_sub(ab, bb, std::integral_constant<int, q0>{}, std::integral_constant<int, 0>{});
    read_sub(ab, bb, std::integral_constant<int, q0 + 1>{}, std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
    // A's part: half `half` of the loads of 64-k stage kt/2 + kAStages - 1,
    // or all of 32-k tile kt + kAStages - 1
    auto a_part = [&]() {
      if constexpr (T::kAPairs)
        load_a((kt >> 1) + T::kAStages - 1, std::integral_constant<int, half * T::kAPerHalf>{},
               std::integral_constant<int, (half + 1) * T::kAPerHalf>{});
      else
        load_a(kt + T::kAStages - 1, std::integral_constant<int, 0>{}, std::integral_constant<int, IA>{});
    };
    if constexpr (kAF) {
      a_part();
      load_b(kt + T::kBStages - 1);
    } else {
      load_b(kt + T::kBStages - 1);
      a_part();
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm0();
  };
  auto compute_phase = [&]() {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s][j], fa[s][i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // End of a phase: this wave's loads that the next half reads have landed
  // (pp_after: past the prologue the same count of later loads for every
  // half), then barrier.
  constexpr int kWait = pp_wait_count<T>(kAF);
  static_assert(kWait >= 0 && kWait < 64 && pp_after<T>(8, kAF) == kWait && pp_after<T>(9, kAF) == kWait,
                "the prologue must not leave fewer loads in flight than the steady state");
  auto phase_end = [&]() {
    wait_vmcnt<kWait>();
    block_barrier();
  };

  // Phases: in phase 2kt group 0 reads half kt and group 1 computes half
  // kt - 1; in phase 2kt + 1 group 0 computes half kt and group 1 reads it.
  // A ring slot is reloaded in a read phase only after both groups have read
  // its previous stage: B's tile kt + kBStages - 1 goes into the slot of tile
  // kt - 1, which group 1 read in phase 2kt - 1; A's 64-k stage kt/2 + 2
  // (even kt) into the slot of stage kt/2 - 1, whose last half group 1 read
  // in phase 2kt - 1.  Group 1 starts one barrier later (block barriers
  // count arrivals, not program points), and group 0 ends with one extra
  // barrier to match.
  // Prologue, in the order pp_after simulates: each stage by the first half
  // that reads it, A's first on a tie.
  static_for<2 * (T::kAStages + T::kBStages)>([&](auto h_c) {
    constexpr int h = decltype(h_c)::value;
    constexpr int sa = T::kAPairs ? h / 2 : h;
    if constexpr (sa < T::kAStages - 1 && (!T::kAPairs || h % 2 == 0))
      load_a(sa, std::integral_constant<int, 0>{}, std::integral_constant<int, IA>{});
    if constexpr (h < T::kBStages - 1) load_b(h);
  });
  wait_vmcnt<pp_after<T>(0, kAF)>();  // half 0's stages have landed
  block_barrier();
  if (grp == 1) block_barrier();
  for (int kt = 0; kt < nk; kt += 2) {
    read_phase(kt, std::integral_constant<int, 0>{});
    phase_end();
    compute_phase();
    phase_end();
    if (kt + 1 < nk) {
      read_phase(kt + 1, std::integral_constant<int, 1>{});
      phase_end();
      compute_phase();
      phase_end();
    }
  }
  if (grp == 0) block_barrier();
  wait_vmcnt<0>();  // the (zero) loads past the end must land before LDS is reused
  if constexpr (Fix::kActive) {
    __syncthreads();  // every wave is past its last read of the LDS ring
    if (!fix.template reduce<TM, TN>(acc, smem, wave, lane)) return;
  }

  const int mb = m0 + wm * T::WM, nb = n0 + wn * T::WN;
  if constexpr (P::Epi::kDirect) {
    p.epi.template direct<TM, TN, T::WN>(acc, mb, nb, lane);
  } else {
    __syncthreads();  // every wave is past its last read of the LDS ring
    constexpr int R = slice_rows<typename P::Epi, T::WN>(kPPWaves, T::kLdsBytes);
    static_assert(kPPWaves * R * (T::WN + 4) * 4 <= T::kLdsBytes, "staging does not fit the LDS tiles");
    if constexpr (kPaired) {
      // The pairs as computed (if kept), then their combination, which is
      // WN / 2 columns wide starting at output column nb / 2.  The second
      // staging lays the waves' LDS regions out with a narrower row, so one
      // wave's region there overlaps others' regions of the first: a block
      // barrier separates them (each wave has drained its LDS reads at the
      // end of a staging).
      if (p.epi.keeps_pairs()) {
        staged_epilogue<TM, TN, T::WN, R>(acc, smem, wave, lane, mb, nb, p.epi.pairs);
        block_barrier();
      }
      f32x16 out[TM][TN / 2];
      p.epi.template combine<TM, TN>(acc, out);
      constexpr int R2 = slice_rows<decltype(p.epi.out), T::WN / 2>(kPPWaves, T::kLdsBytes);
      staged_epilogue<TM, TN / 2, T::WN / 2, R2>(out, smem, wave, lane, mb, nb / 2, p.epi.out);
    } else {
      staged_epilogue<TM, TN, T::WN, R>(acc, smem, wave, lane, mb, nb, p.epi);
    }
  }
}

template <class P>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pp_kernel(P p) {
  __shared__ __attribute__((aligned(1024))) char smem[P::T::kLdsBytes];
  int tmi, tni;
  tile_of_block(blockIdx.x, gridDim.x, p.tiles_m(), p.tiles_n(), tmi, tni);
  gemm_tile_pp(p, smem, tmi, tni);
}

// Three independent GEMMs in one launch (blocks [0, p0.tiles()) on p0, then
// p1, then p2; longest-K problems first so the short tiles of the later ones
// fill the compute units the long ones leave free).
template <class P0, class P1, class P2>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pp_group3_kernel(P0 p0, P1 p1, P2 p2) {
  constexpr int kL0 = P0::T::kLdsBytes, kL1 = P1::T::kLdsBytes, kL2 = P2::T::kLdsBytes;
  constexpr int kL = kL0 > kL1 ? (kL0 > kL2 ? kL0 : kL2) : (kL1 > kL2 ? kL1 : kL2);
  __shared__ __attribute__((aligned(1024))) char smem[kL];
  int pid = blockIdx.x, tmi, tni;
  const int t0 = p0.tiles(), t1 = p1.tiles();
  if (pid < t0) {
    tile_of_block(pid, t0, p0.tiles_m(), p0.tiles_n(), tmi, tni);
    gemm_tile_pp(p0, smem, tmi, tni);
  } else if ((pid -= t0) < t1) {
    tile_of_block(pid, t1, p1.tiles_m(), p1.tiles_n(), tmi, tni);
    gemm_tile_pp(p1, smem, tmi, tni);
  } else {
    pid -= t1;
    tile_of_block(pid, p2.tiles(), p2.tiles_m(), p2.tiles_n(), tmi, tni);
    gemm_tile_pp(p2, smem, tmi, tni);
  }
}

// The problem restricted to K range [k0, k0 + kc): both operands move to the
// range's first K row or column, so the range is an ordinary GEMM.
template <class P>
__device__ __forceinline__ P k_range(const P& p, int k0, int kc) {
  P q = p;
  q.A = P::AK ? p.A + k0 : p.A + (int64_t)k0 * p.lda;
  q.B = P::BK ? p.B + k0 : p.B + (int64_t)k0 * p.ldb;
  q.K = min(kc, p.K - k0);
  return q;
}

// Partial buffers and counters of the K-split problems of one grouped launch.
struct KSplit {
  float* part;  // [tiles of p0, then of p1][parts][BM * BN] fp32
  int* count;   // [tiles of p0, then of p1]
  int parts, kchunk;
};

template <class P>
__device__ __forceinline__ void run_k_part(const P& p, const KSplit& k, int tile0, int b, char* smem) {
  const int tiles = p.tiles(), s = b / tiles, t = b - s * tiles;
  int tmi, tni;
  tile_of_block(t, tiles, p.tiles_m(), p.tiles_n(), tmi, tni);
  const int64_t slot = (int64_t)P::BM * P::BN;
  const KPartFix fix{k.part + (int64_t)(tile0 + t) * k.parts * slot, k.count + tile0 + t, s, k.parts};
  gemm_tile_pp(k_range(p, s * k.kchunk, k.kchunk), smem, tmi, tni, fix);
}

// gemm_pp_group3_kernel with p0 and p1 split over K into k.parts parts each,
// reduced inside the launch (KPartFix).  Blocks: p0's parts (part-major),
// then p1's, then p2's tiles.
template <class P0, class P1, class P2>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pp_group3_ksplit_kernel(P0 p0, P1 p1, P2 p2, KSplit k) {
  constexpr int kL0 = P0::T::kLdsBytes, kL1 = P1::T::kLdsBytes, kL2 = P2::T::kLdsBytes;
  constexpr int kL = kL0 > kL1 ? (kL0 > kL2 ? kL0 : kL2) : (kL1 > kL2 ? kL1 : kL2);
  __shared__ __attribute__((aligned(1024))) char smem[kL];
  int pid = blockIdx.x;
  const int t0 = p0.tiles(), t1 = p1.tiles();
  if (pid < t0 * k.parts) {
    run_k_part(p0, k, 0, pid, smem);
  } else if ((pid -= t0 * k.parts) < t1 * k.parts) {
    run_k_part(p1, k, t0, pid, smem);
  } else {
    pid -= t1 * k.parts;
    int tmi, tni;
    tile_of_block(pid, p2.tiles(), p2.tiles_m(), p2.tiles_n(), tmi, tni);
    gemm_tile_pp(p2, smem, tmi, tni);
  }
}

// gemm_pp_group3_kernel with only the last `tail` tiles of p1 (in its block
// order) split over K into k.parts parts, launched after p2's tiles: the
// launch's unsplit blocks fill whole rounds of the compute units and the
// split tiles' shorter parts make the last round.  Blocks: p0's tiles,
// p1's first tiles, p2's tiles, then the tail's parts (part-major).  Slot
// and counter j belong to tail tile j.
template <class P0, class P1, class P2>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pp_group3_tail_kernel(P0 p0, P1 p1, P2 p2, KSplit k, int tail) {
  constexpr int kL0 = P0::T::kLdsBytes, kL1 = P1::T::kLdsBytes, kL2 = P2::T::kLdsBytes;
  constexpr int kL = kL0 > kL1 ? (kL0 > kL2 ? kL0 : kL2) : (kL1 > kL2 ? kL1 : kL2);
  __shared__ __attribute__((aligned(1024))) char smem[kL];
  int pid = blockIdx.x, tmi, tni;
  const int t0 = p0.tiles(), t1 = p1.tiles(), head = t1 - tail, t2 = p2.tiles();
  if (pid < t0) {
    tile_of_block(pid, t0, p0.tiles_m(), p0.tiles_n(), tmi, tni);
    gemm_tile_pp(p0, smem, tmi, tni);
  } else if ((pid -= t0) < head) {
    tile_of_block(pid, t1, p1.tiles_m(), p1.tiles_n(), tmi, tni);
    gemm_tile_pp(p1, smem, tmi, tni);
  } else if ((pid -= head) < t2) {
    tile_of_block(pid, t2, p2.tiles_m(), p2.tiles_n(), tmi, tni);
    gemm_tile_pp(p2, smem, tmi, tni);
  } else {
    pid -= t2;
    const int s = pid / tail, j = pid - s * tail;
    tile_of_block(head + j, t1, p1.tiles_m(), p1.tiles_n(), tmi, tni);
    const KPartFix fix{k.part + (int64_t)j * k.parts * P1::BM * P1::BN, k.count + j, s, k.parts};
    gemm_tile_pp(k_range(p1, s * k.kchunk, k.kchunk), smem, tmi, tni, fix);
  }
}

static __global__ __launch_bounds__(256) void zero_i32_kernel(int* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <class P0, class P1, class P2>
inline hipError_t launch_gemm_pp_group3_ksplit(const P0& p0, const P1& p1, const P2& p2, const KSplit& k,
                                               hipStream_t stream) {
  const int counters = p0.tiles() + p1.tiles();
  debug_problem(p0);
  debug_problem(p1);
  debug_problem(p2);
  static_assert(P0::BM * P0::BN == P1::BM * P1::BN, "one slot size for both split problems");
  LGS_CHECK(k.parts >= 2 && k.kchunk % kBK == 0 && (int64_t)(k.parts - 1) * k.kchunk < p0.K &&
            (int64_t)k.parts * k.kchunk >= p0.K && p0.K == p1.K);
  LGS_NEED(k.part, (size_t)counters * k.parts * P0::BM * P0::BN * 4, "K-split partial slots");
  LGS_NEED(k.count, (size_t)counters * 4, "K-split counters");
  LGS_LAUNCH(zero_i32_kernel, dim3((counters + 255) / 256), dim3(256), 0, stream, k.count, counters);
  LGS_LAUNCH((gemm_pp_group3_ksplit_kernel<P0, P1, P2>), dim3((p0.tiles() + p1.tiles()) * k.parts + p2.tiles()),
             dim3(kPPThreads), 0, stream, p0, p1, p2, k);
  return LGS_LAUNCH_STATUS();
}

template <class P0, class P1, class P2>
inline hipError_t launch_gemm_pp_group3_tail(const P0& p0, const P1& p1, const P2& p2, const KSplit& k,
                                             int tail, hipStream_t stream) {
  debug_problem(p0);
  debug_problem(p1);
  debug_problem(p2);
  LGS_CHECK(tail >= 1 && tail <= p1.tiles() && k.parts >= 2 && k.kchunk % kBK == 0 &&
            (int64_t)(k.parts - 1) * k.kchunk < p1.K && (int64_t)k.parts * k.kchunk >= p1.K);
  LGS_NEED(k.part, (size_t)tail * k.parts * P1::BM * P1::BN * 4, "K-split partial slots");
  LGS_NEED(k.count, (size_t)tail * 4, "K-split counters");
  LGS_LAUNCH(zero_i32_kernel, dim3((tail + 255) / 256), dim3(256), 0, stream, k.count, tail);
  LGS_LAUNCH((gemm_pp_group3_tail_kernel<P0, P1, P2>),
             dim3(p0.tiles() + p1.tiles() - tail + p2.tiles() + tail * k.parts), dim3(kPPThreads), 0, stream, p0,
             p1, p2, k, tail);
  return LGS_LAUNCH_STATUS();
}

// Every tile of p split over K into k.parts parts (blocks part-major),
// reduced inside the launch (KPartFix): slot and counter t belong to tile t.
template <class P>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pp_ksplit_kernel(P p, KSplit k) {
  __shared__ __attribute__((aligned(1024))) char smem[P::T::kLdsBytes];
  run_k_part(p, k, 0, blockIdx.x, smem);
}

template <class P>
inline hipError_t launch_gemm_pp_ksplit(const P& p, const KSplit& k, hipStream_t stream) {
  const int tiles = p.tiles();
  debug_problem(p);
  LGS_CHECK(k.parts >= 2 && k.kchunk % kBK == 0 && (int64_t)(k.parts - 1) * k.kchunk < p.K &&
            (int64_t)k.parts * k.kchunk >= p.K);
  LGS_NEED(k.part, (size_t)tiles * k.parts * P::BM * P::BN * 4, "K-split partial slots");
  LGS_NEED(k.count, (size_t)tiles * 4, "K-split counters");
  LGS_LAUNCH(zero_i32_kernel, dim3((tiles + 255) / 256), dim3(256), 0, stream, k.count, tiles);
  LGS_LAUNCH((gemm_pp_ksplit_kernel<P>), dim3(tiles * k.parts), dim3(kPPThreads), 0, stream, p, k);
  return LGS_LAUNCH_STATUS();
}

// Two GEMMs in one launch, every tile of p0 split over K (part-major blocks
// first), p1's tiles unsplit after them.
template <class P0, class P1>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pp_group2_ksplit_kernel(P0 p0, P1 p1, KSplit k) {
  constexpr int kL = P0::T::kLdsBytes > P1::T::kLdsBytes ? P0::T::kLdsBytes : P1::T::kLdsBytes;
  __shared__ __attribute__((aligned(1024))) char smem[kL];
  int pid = blockIdx.x;
  const int t0 = p0.tiles();
  if (pid < t0 * k.parts) {
    run_k_part(p0, k, 0, pid, smem);
  } else {
    pid -= t0 * k.parts;
    int tmi, tni;
    tile_of_block(pid, p1.tiles(), p1.tiles_m(), p1.tiles_n(), tmi, tni);
    gemm_tile_pp(p1, smem, tmi, tni);
  }
}

template <class P0, class P1>
inline hipError_t launch_gemm_pp_group2_ksplit(const P0& p0, const P1& p1, const KSplit& k, hipStream_t stream) {
  const int tiles = p0.tiles();
  debug_problem(p0);
  debug_problem(p1);
  LGS_CHECK(k.parts >= 2 && k.kchunk % kBK == 0 && (int64_t)(k.parts - 1) * k.kchunk < p0.K &&
            (int64_t)k.parts * k.kchunk >= p0.K);
  LGS_NEED(k.part, (size_t)tiles * k.parts * P0::BM * P0::BN * 4, "K-split partial slots");
  LGS_NEED(k.count, (size_t)tiles * 4, "K-split counters");
  LGS_LAUNCH(zero_i32_kernel, dim3((tiles + 255) / 256), dim3(256), 0, stream, k.count, tiles);
  LGS_LAUNCH((gemm_pp_group2_ksplit_kernel<P0, P1>), dim3(tiles * k.parts + p1.tiles()), dim3(kPPThreads), 0,
             stream, p0, p1, k);
  return LGS_LAUNCH_STATUS();
}

// Two independent GEMMs in one launch (p0 first).
template <class P0, class P1>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pp_group2_kernel(P0 p0, P1 p1) {
  constexpr int kL = P0::T::kLdsBytes > P1::T::kLdsBytes ? P0::T::kLdsBytes : P1::T::kLdsBytes;
  __shared__ __attribute__((aligned(1024))) char smem[kL];
  int pid = blockIdx.x, tmi, tni;
  const int t0 = p0.tiles();
  if (pid < t0) {
    tile_of_block(pid, t0, p0.tiles_m(), p0.tiles_n(), tmi, tni);
    gemm_tile_pp(p0, smem, tmi, tni);
  } else {
    pid -= t0;
    tile_of_block(pid, p1.tiles(), p1.tiles_m(), p1.tiles_n(), tmi, tni);
    gemm_tile_pp(p1, smem, tmi, tni);
  }
}

template <class P0, class P1>
inline hipError_t launch_gemm_pp_group2(const P0& p0, const P1& p1, hipStream_t stream) {
  debug_problem(p0);
  debug_problem(p1);
  LGS_LAUNCH((gemm_pp_group2_kernel<P0, P1>), dim3(p0.tiles() + p1.tiles()), dim3(kPPThreads), 0, stream, p0,
             p1);
  return LGS_LAUNCH_STATUS();
}

template <class P0, class P1, class P2>
inline hipError_t launch_gemm_pp_group3(const P0& p0, const P1& p1, const P2& p2, hipStream_t stream) {
  debug_problem(p0);
  debug_problem(p1);
  debug_problem(p2);
  LGS_LAUNCH((gemm_pp_group3_kernel<P0, P1, P2>), dim3(p0.tiles() + p1.tiles() + p2.tiles()), dim3(kPPThreads),
             0, stream, p0, p1, p2);
  return LGS_LAUNCH_STATUS();
}

template <class P>
inline hipError_t launch_gemm_pp(const P& p, hipStream_t stream) {
  debug_problem(p);
  LGS_LAUNCH((gemm_pp_kernel<P>), dim3(p.tiles()), dim3(kPPThreads), 0, stream, p);
  return LGS_LAUNCH_STATUS();
}

template <int BM, int BN, bool AK, bool BK, class Epi>
inline PPProblem<BM, BN, AK, BK, Epi> pp_problem(const bf16* A, int64_t lda, const bf16* B,
                                                 int64_t ldb, int M, int N, int K, const Epi& epi) {
  return PPProblem<BM, BN, AK, BK, Epi>{A, lda, B, ldb, M, N, K, epi};
}

}  // namespace lgs
