// One launch for a flat step that holds both prefill rows and decode rows.
//
// The flat batch puts every kind of request into one step ("Model
// execution", section "Flattening a step"); its prefill rows are bound by the
// matrix cores and its decode rows by HBM ("Inside the engine: kernels, CUDA
// graphs and the life of a request", section "Prefill has a full grid; decode
// at batch 1 has almost none").  Run back to back, the matrix cores idle
// through the decode and HBM through the prefill.  Run as two kernels on two
// streams, the decode's tens of thousands of small work-groups keep every
// compute unit partly occupied, so a prefill work-group (which needs a whole
// CU: 92 KB of LDS and every VGPR of two waves per SIMD) is only placed once
// the decode grid drains.
//
// Here one persistent work-group per compute unit (eight waves; the LDS is
// the union of the two bodies' buffers) takes work units from two device
// counters: the matrix-core kernel's (work item, KV head) units, heavy
// first, and the decode kernel's (KV head, request rank, split) units,
// longest request first.  A quarter of the work-groups start on the prefill
// units and the rest on the decode units; each moves to the other list when
// its own runs dry, so the launch ends when both are done, whichever way the
// work is split.  Both bodies are the ones the separate kernels run (the
// decode body in its two-fragment-set form, which keeps as many loads in
// flight at eight waves per CU as the many-work-group form does at sixteen),
// so every unit's result is bit-for-bit that of the separate launches.
#include "decode_body.h"
#include "prefill_body.h"

namespace pa {
namespace {

constexpr int kMixedWaves = 8;
// one work-group in this many starts on the prefill units
#ifndef PA_MIXED_PREFILL_SHARE
#define PA_MIXED_PREFILL_SHARE 4
#endif
static_assert(PA_PREFILL_WAVES == kMixedWaves && PA_PREFILL_ROW_GROUPS == 1,
              "the mixed kernel runs the prefill body at eight waves, one row group");

template <int D>
union MixedSmem {
  PrefillSmem<D, PA_PREFILL_KEYS> p;
  DecodeSmem<D, kMixedWaves, 2> d;
};

template <int D, int G, bool F8, int NTP>
__global__ __launch_bounds__(64 * kMixedWaves, 1) void mixed_kernel(PrefillParams pp,
                                                                    DecodeParams dp,
                                                                    int32_t* __restrict__ claim,
                                                                    int32_t prefill_first,
                                                                    int32_t decode_x,
                                                                    int32_t decode_units) {
  __shared__ __align__(16) MixedSmem<D> sm;
  __shared__ int s_unit[2];
  const int prefill_units = pp.plan[0] * pp.hkv;
  bool on_prefill = (int)blockIdx.x < prefill_first;
  for (;;) {
    if (threadIdx.x == 0) {
      // the list this work-group is on first, then the other one
      int kind = -1, u = 0;
      for (int t = 0; t < 2 && kind < 0; ++t) {
        if ((t == 0) == on_prefill) {
          const int v = atomicAdd(&claim[0], 1);
          if (v < prefill_units) kind = 0, u = v;
        } else {
          const int v = atomicAdd(&claim[1], 1);
          if (v < decode_units) kind = 1, u = v;
        }
      }
      s_unit[0] = kind;
      s_unit[1] = u;
    }
    __syncthreads();
    const int kind = s_unit[0], u = s_unit[1];
    __syncthreads();  // s_unit is rewritten by the next claim
    if (kind < 0) break;  // both lists are exhausted
    on_prefill = kind == 0;
    // the thread index as a fresh value each pass, so that the compiler
    // keeps each unit's per-thread arithmetic inside the unit
    const int tid = unit_tid();
    if (kind == 0)
      prefill_unit<D, G, kMixedWaves, 1, PA_PREFILL_KEYS, F8, false>(pp, u, sm.p, tid);
    else
      decode_unit<D, G, kMixedWaves, 2, F8, NTP>(dp, u % decode_x, u / decode_x, sm.d, tid);
    __syncthreads();  // the next unit reuses the shared memory
  }
}

template <int D, int G, bool F8>
void launch_dg(const AttnArgs& a, hipStream_t stream) {
  const PrefillParams pp = make_prefill_params(a);
  const DecodeParams dp = make_decode_params(a);
  const int32_t decode_x = a.num_seqs * a.hkv;
  const int32_t decode_units = decode_x * a.splits;
  const int32_t wgs = a.num_cus;
  const int32_t prefill_first = (wgs + PA_MIXED_PREFILL_SHARE - 1) / PA_MIXED_PREFILL_SHARE;
  trace_before(K_MIXED, stream);
  // V streamed non-temporally when the call's blocks are unshared, or per
  // request as the decode order marks it (as in the many-work-group decode
  // kernel)
  if (a.unshared)
    hipLaunchKernelGGL((mixed_kernel<D, G, F8, kNtV>), dim3(wgs), dim3(64 * kMixedWaves), 0,
                       stream, pp, dp, a.claim, prefill_first, decode_x, decode_units);
  else if (a.detect_sharing)
    hipLaunchKernelGGL((mixed_kernel<D, G, F8, kNtAuto>), dim3(wgs), dim3(64 * kMixedWaves), 0,
                       stream, pp, dp, a.claim, prefill_first, decode_x, decode_units);
  else
    hipLaunchKernelGGL((mixed_kernel<D, G, F8, 0>), dim3(wgs), dim3(64 * kMixedWaves), 0,
                       stream, pp, dp, a.claim, prefill_first, decode_x, decode_units);
  trace_after(stream);
}

template <int D, bool F8>
void launch_d(const AttnArgs& a, hipStream_t stream) {
  switch (a.hq / a.hkv) {
    case 1: launch_dg<D, 1, F8>(a, stream); break;
    case 2: launch_dg<D, 2, F8>(a, stream); break;
    case 4: launch_dg<D, 4, F8>(a, stream); break;
    case 8: launch_dg<D, 8, F8>(a, stream); break;
    default: launch_dg<D, 16, F8>(a, stream); break;
  }
}

}  // namespace

hipError_t launch_mixed_bf16(const AttnArgs& a0, hipStream_t stream) {
  // the work list and the decode order come from one launch
  hipError_t e = launch_prefill_plan(a0, stream, true);
  if (e != hipSuccess) return e;
  AttnArgs a = a0;
  a.order_ready = 1;
  if (a.cache_fp8) {
    if (a.d == 64) launch_d<64, true>(a, stream);
    else launch_d<128, true>(a, stream);
  } else {
    if (a.d == 64) launch_d<64, false>(a, stream);
    else launch_d<128, false>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace pa
