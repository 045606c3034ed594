// Vocab-parallel cross-entropy forward for one rank's slice: the fused logit
// GEMM (partials per wave column-slab, see xent.hpp) and the slab merge.
//
// Rank r owns vocabulary rows [vocab_start, vocab_start + Vr).  Per token it
// produces the slice max m_r, the sum of exp(z - m_r) over the slice l_r, the
// target logit T_r (exactly +0 when the target id is outside the slice) and
// the global id of the slice's first maximum.  Ranks then exchange those
// numbers instead of logits ("LIT-022: Megatron-LM ...", "Key takeaways").
#include <mutex>

#include "dispatch.hpp"
#include "internal.hpp"
#include "xent.hpp"

namespace lgs {

// The launch plan: the slice's columns in one launch, or two (plan_columns),
// on the ping-pong tiles (e.g. 8192 x 6400: the first 2560 columns on
// 256x320, the other 3840 on 256x256).  Each launch numbers its slabs from
// where the previous one ended, with its own wave width.
static ColumnPlan xent_plan(int M, int Vr) { return plan_columns(M, Vr, false, kPPTiles); }

// Slabs the launch plan writes: every wave column of every tile writes one
// slab (a wave column wholly past the slice end writes -inf / 0 partials that
// the merge never reads), so a launch of `cols` columns on tile t writes
// ceil(cols / BN) * BN / WN of them.  The merge reads the first
// ceil(Vr / WN) (one launch) or c1 / WN + ceil((Vr - c1) / WN_tail) (two).
static int slabs_written(const ColumnPlan& plan, int Vr) {
  const int bn = tile_bn(plan.main);
  int n = (plan.c1 + bn - 1) / bn * bn / tile_wn(plan.main);
  if (plan.c1 < Vr) {
    const int bt = tile_bn(plan.tail);
    n += (Vr - plan.c1 + bt - 1) / bt * bt / tile_wn(plan.tail);
  }
  return n;
}

size_t xent_scratch_bytes(int M, int Vr) {
  return (size_t)slabs_written(xent_plan(M, Vr), Vr) * (size_t)M * 16u;
}

// Eight lanes per token fold the slabs into the rank's partials, each lane
// walking every eighth slab (independent loads in flight), then combining with
// lane shuffles.  Ties on the maximum go to the lowest column, i.e. the first
// maximum of the slice.
__global__ __launch_bounds__(256) void xent_merge_kernel(XentSlabs s, int nslabs, int M,
                                                         int vocab_start, float* m_r, float* l_r,
                                                         float* t_r, int32_t* argmax_r,
                                                         float* loss) {
  constexpr int kLanes = 8;
  const int m = blockIdx.x * (256 / kLanes) + threadIdx.x / kLanes, part = threadIdx.x % kLanes;
  const bool valid = m < M;
  const int mm = valid ? m : 0;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  if (s.idx) {
#pragma unroll 4
    for (int k = part; k < nslabs; k += kLanes) {
      const float v = s.m[(int64_t)k * M + mm];
      const int i = s.idx[(int64_t)k * M + mm];
      if (v > best || (v == best && i < bi)) { best = v; bi = i; }
    }
  } else {
#pragma unroll 4
    for (int k = part; k < nslabs; k += kLanes) best = fmaxf(best, s.m[(int64_t)k * M + mm]);
  }
#pragma unroll
  for (int off = 1; off < kLanes; off <<= 1) {
    const float ob = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  }
  float L = 0.f, T = 0.f;
#pragma unroll 4
  for (int k = part; k < nslabs; k += kLanes) {
    const int64_t o = (int64_t)k * M + mm;
    L += s.l[o] * fast_exp(s.m[o] - best);
    T += s.t[o];
  }
#pragma unroll
  for (int off = 1; off < kLanes; off <<= 1) {
    L += __shfl_xor(L, off);
    T += __shfl_xor(T, off);
  }
  if (!valid || part != 0) return;
  m_r[m] = best;
  l_r[m] = L;
  t_r[m] = T;
  if (argmax_r) argmax_r[m] = bi == 0x7fffffff ? -1 : vocab_start + bi;
  if (loss) loss[m] = best + logf(L) - T;
}

hipError_t xent_fwd(int M, int h, int Vr, int vocab_start, const void* H, int64_t ldh,
                    const void* E, int64_t lde, const int32_t* targets, float* m_r, float* l_r,
                    float* t_r, int32_t* argmax_r, float* loss, void* scratch, hipStream_t s) {
  const ColumnPlan plan = xent_plan(M, Vr);
  const int WN = tile_wn(plan.main);
  const size_t slab_elems = (size_t)slabs_written(plan, Vr) * M;
  XentSlabs sl;
  sl.m = (float*)scratch;
  sl.l = sl.m + slab_elems;
  sl.t = sl.l + slab_elems;
  sl.idx = argmax_r ? (int32_t*)(sl.t + slab_elems) : nullptr;  // argmax only when asked for
  const bf16 *hh = (const bf16*)H, *e = (const bf16*)E;
  const EpiXent e1{sl, targets, vocab_start, M, plan.c1, WN, 0, 0};
  hipError_t err = gemm_bf16<true, true>(plan.main, hh, ldh, e, lde, M, plan.c1, h, e1, s);
  if (err != hipSuccess) return err;
  int nslabs = plan.c1 / WN;
  if (plan.c1 < Vr) {
    const int rest = Vr - plan.c1, WNt = tile_wn(plan.tail);
    const EpiXent e2{sl, targets, vocab_start + plan.c1, M, rest, WNt, plan.c1, nslabs};
    err = gemm_bf16<true, true>(plan.tail, hh, ldh, e + (int64_t)plan.c1 * lde, lde, M, rest, h, e2, s);
    if (err != hipSuccess) return err;
    nslabs += (rest + WNt - 1) / WNt;
  } else {
    nslabs = (Vr + WN - 1) / WN;
  }
  // the merge reads the first nslabs slabs of every plane, all written above
  LGS_CHECK(nslabs <= slabs_written(plan, Vr));
  LGS_NEED(sl.m, (size_t)nslabs * M * 4, "slab maxima read by the merge");
  LGS_NEED(sl.l, (size_t)nslabs * M * 4, "slab sums read by the merge");
  LGS_NEED(sl.t, (size_t)nslabs * M * 4, "slab targets read by the merge");
  if (sl.idx) LGS_NEED(sl.idx, (size_t)nslabs * M * 4, "slab argmax read by the merge");
  LGS_NEED(m_r, (size_t)M * 4, "m_r");
  LGS_NEED(l_r, (size_t)M * 4, "l_r");
  LGS_NEED(t_r, (size_t)M * 4, "tgt_r");
  if (argmax_r) LGS_NEED(argmax_r, (size_t)M * 4, "argmax_r");
  if (loss) LGS_NEED(loss, (size_t)M * 4, "loss");
  LGS_LAUNCH(xent_merge_kernel, dim3((M + 31) / 32), dim3(256), 0, s, sl, nslabs, M, vocab_start, m_r, l_r, t_r,
             argmax_r, loss);
  return LGS_LAUNCH_STATUS();
}

// ---------------------------------------------------------------------------
// The slab partials of the allocation-free entry point live in one file-scope
// device array.  Each device that loads the library holds its own copy until
// the process ends; its address differs per device and is only known to the
// runtime, so it is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept.  Host code never passes the array's name to a
// kernel: on the host that name is a stand-in, not a device address.  The
// fused CE writes every slab entry the merge reads before the merge runs, so
// nothing in the array needs clearing between calls; calls that overlap on
// one device share the array and race.
static __device__ __align__(256) unsigned char scratch[kXentStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t xent_static_scratch(hipStream_t s, void** out) {
  if (debug::dry_run()) {  // debug builds without a GPU: a stand-in address, never dereferenced
    *out = (void*)((uintptr_t)1 << 46);
    debug::allow(*out, kXentStaticScratchBytes);
    return hipSuccess;
  }
  int dev = -1;
  hipError_t e = hipStreamGetDevice(s, &dev);  // the device the stream's work runs on
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  debug::allow(*out, kXentStaticScratchBytes);
  return hipSuccess;
}

}  // namespace lgs
