// The matrix cores' bf16 rate on this part with nothing but MFMAs to run: the
// ceiling that the GEMM kernels' fractions of the spec peak are read against
// (declared in include/lgs_testing.h; not part of the method's interface).
//
// Every wave holds kOps pairs of 32x16 / 16x32 bf16 operands in registers and
// runs kChains independent accumulator chains of v_mfma_f32_32x32x16_bf16.
// The operand pairs rotate between consecutive instructions (chain c in step
// j takes A[(c + j) % kOps] and B[c]), so the multipliers see changing data as
// in a GEMM; the part's power limit makes the rate depend on that data.  No
// memory traffic between the first operand load and the final store.
//
// After iters8 passes of kOps steps, chain c holds iters8 * (sum_k A_k) B_c,
// exact in fp32 for small-integer operands (the GPU test's check of the
// instruction's lane layout).  Each wave also records its elapsed shader
// clocks (s_memtime) and 100 MHz reference ticks (s_memrealtime) around the
// loop: their ratio is the clock the matrix cores actually ran at.
#include "common.hpp"
#include "internal.hpp"

namespace lgs {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kOps = 8;     // operand pairs per lane
constexpr int kChains = 8;  // independent accumulators per wave

__global__ __launch_bounds__(512) void mfma_rate_kernel(const bf16x8* __restrict__ ops, int iters8,
                                                        float* __restrict__ out,
                                                        uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  bf16x8 a[kOps], b[kOps];
#pragma unroll
  for (int k = 0; k < kOps; ++k) {
    a[k] = ops[(2 * k) * 64 + lane];
    b[k] = ops[(2 * k + 1) * 64 + lane];
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  // One step is kChains independent MFMAs; the scheduling barrier keeps the
  // compiler from interleaving steps, which would put dependent MFMAs of one
  // chain back to back.
  for (int i = 0; i < iters8; ++i)
#pragma unroll
    for (int j = 0; j < kOps; ++j) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(c + j) % kOps], b[c], acc[c], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float* o = out + w * (kChains * 16 * 64);
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[(c * 16 + r) * 64 + lane] = acc[c][r];
  if (lane == 0) {
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

}  // namespace

size_t mfma_rate_out_floats(int blocks, int waves) { return (size_t)blocks * waves * kChains * 16 * 64; }

hipError_t mfma_rate(int blocks, int waves, int iters8, const void* ops, float* out, uint64_t* clocks,
                     hipStream_t s) {
  LGS_CHECK(blocks >= 1 && waves >= 1 && waves <= 8 && iters8 >= 0);
  LGS_NEED(ops, (size_t)2 * kOps * 64 * 16, "operands");
  LGS_NEED(out, mfma_rate_out_floats(blocks, waves) * 4, "accumulators");
  LGS_NEED(clocks, (size_t)blocks * waves * 16, "clock counts");
  LGS_LAUNCH(mfma_rate_kernel, dim3(blocks), dim3(64 * waves), 0, s, (const bf16x8*)ops, iters8, out, clocks);
  return LGS_LAUNCH_STATUS();
}

}  // namespace lgs
