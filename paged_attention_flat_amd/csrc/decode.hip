// Decode attention (bf16 cache, fp32 accumulation) for requests with few new
// tokens, with an optional split of the key axis.
//
// Method: "Inside the engine: kernels, CUDA graphs and the life of a request",
// sections "Never materialise the T x T matrix" (online softmax: running max m
// and denominator l, accumulator rescaled by e^(m_old - m_new)), "Prefill has a
// full grid; decode at batch 1 has almost none" (split-KV partials over block
// ranges, merged in a second reduction -- here by the last split of each
// request and KV head to finish, inside this launch) and "Attention over a
// block table, not a contiguous tensor" (keys and values gathered through the
// block table).  The cache holds bf16, or E4M3 codes with per-KV-head scales
// (converted to bf16 exactly in registers; K's scale folds into the score
// scale, V's into the output).
//
// MI355X design.  One work-group = (KV head, request, split); its waves
// walk disjoint pairs of 16-token blocks of the split's range and each keeps
// its own (m, l, acc) state, merged lane by lane through LDS at the end.  All
// query heads of the KV head (group size G) and up to 16 / G new tokens are
// packed as the 16 columns of a 16x16x32 bf16 MFMA, so every K/V byte is read
// from HBM once per step:
//   S^T[key][col] = K[key][:] . Q[col][:]    A = K rows (16-byte loads),
//                                            B = Q (held in registers)
//   O^T[d][col]  += V^T[d][keys] P[keys][col] A = V (dim-major cache block:
//                                            16-byte loads of 8 keys),
//                                            B = P straight from the S^T
//                                            accumulator, no shuffles.
// A pair of blocks gives the 32-key contraction of the P.V product; the rows
// of the two S^T products are assigned to keys so that each lane's P values
// are 8 consecutive keys of one block, matching one 16-byte V load.  Block
// ids come 64 at a time from one coalesced table load and are picked with
// readlane.  With many units, sixteen waves per CU (four 4-wave work-groups
// at 118 VGPRs) keep enough loads in flight to cover HBM latency; with few,
// eight waves per CU each keep the next pair's loads in flight while they
// compute the current one (two fragment sets).  Row maxima use two
// cross-lane exchanges; exponentials are base 2 on log2(e)-prescaled scores.
//
// Work order: work-group index = KV head fastest, then request rank.  For
// batches with more work than compute units the ranks come from a device-side
// counting sort of the decode requests by block count, longest first, so the
// long requests start early and short ones fill the tail.
#include "decode_body.h"

namespace pa {
namespace {

// Counting sort of the decode requests by block count, with the sharing
// test when `tables` is given (decode_order_block).
__global__ __launch_bounds__(1024) void decode_order_kernel(const int32_t* __restrict__ qsl,
                                                            const int32_t* __restrict__ seq_lens,
                                                            const int32_t* __restrict__ tables,
                                                            int32_t table_stride,
                                                            int32_t num_seqs, int32_t dq,
                                                            int32_t shift,
                                                            int32_t* __restrict__ order) {
  __shared__ OrderSmem sm;
  __shared__ ShareSmem share;
  decode_order_block(qsl, seq_lens, tables, table_stride, num_seqs, dq, shift, order, sm,
                     &share);
}

// NTP: the loads that take the non-temporal policy.  The long-context shape
// streams K and V that way with a bf16 cache (measured 9-10 % faster from
// 16K keys on, equal below).  The many-work-group shape streams V only, and
// only for requests whose blocks are their own (kNtV for every request when
// the call says so, kNtAuto per request as the decode order marks it): 8 %
// (bf16) and 9 % (E4M3) faster on 256 unshared requests, 25 % slower where
// all of them re-read one long prefix, which cached loads serve from
// L2/MALL; non-temporal K loads (64 bytes of 16 rows each) were slower there
// in either case.
//
// Waves per SIMD the register allocation must allow: two for the two-
// fragment-set shape at four waves; four for the bf16 one-pair shape at four
// waves (118 VGPRs, four work-groups per CU; left free, the compiler takes
// 115 VGPRs + 32 AGPRs and only three fit, which measured 1 % slower on 256
// unshared requests and 3 % on the shared-prefix decode); one otherwise (the
// E4M3 one-pair shape held to four waves measured 0.5 % slower than at three,
// and five waves of either dtype spill).
constexpr int decode_min_waves(int nw, int pipe, bool f8) {
  return pipe == 2 ? (nw < 8 ? 8 / nw : 1) : (nw == 4 && !f8 ? 4 : 1);
}

template <int D, int G, int NW, int PIPE, bool F8, int NTP>
__global__ __launch_bounds__(64 * NW, decode_min_waves(NW, PIPE, F8)) void decode_kernel(
    DecodeParams p) {
  __shared__ DecodeSmem<D, NW, PIPE> sm;
  decode_unit<D, G, NW, PIPE, F8, NTP>(p, blockIdx.x, blockIdx.y, sm, threadIdx.x);
}

// the counting sort of the decode requests, when the launch ranks them
template <int G>
void order_dg(const AttnArgs& a, hipStream_t stream) {
  // (the shared-prefix setup kernel may already have built it)
  if (a.decode_order == nullptr || a.order_ready) return;
  trace_before(K_DECODE_ORDER, stream);
  hipLaunchKernelGGL(decode_order_kernel, dim3(1), dim3(1024), 0, stream, a.qsl, a.seq_lens,
                     a.detect_sharing ? a.tables : nullptr, a.table_stride, a.num_seqs, 16 / G,
                     decode_order_shift(a.max_seq_len), a.decode_order);
  trace_after(stream);
}

template <int D, int G, bool F8>
void launch_dg(const AttnArgs& a, hipStream_t stream) {
  const DecodeParams p = make_decode_params(a);
  order_dg<G>(a, stream);
  dim3 grid(a.num_seqs * a.hkv, a.splits);
  const int64_t units = (int64_t)a.num_seqs * a.hkv * a.splits;
  trace_before(a.splits > 1 ? K_DECODE_SPLIT : K_DECODE, stream);
  if (units <= 2 * (int64_t)a.num_cus) {
    constexpr int NW = PA_DECODE_WAVES_PIPE;
    hipLaunchKernelGGL((decode_kernel<D, G, NW, 2, F8, kNtK | kNtV>), grid, dim3(64 * NW), 0,
                       stream, p);
  } else if (a.unshared) {
    constexpr int NW = PA_DECODE_WAVES_WIDE;
    hipLaunchKernelGGL((decode_kernel<D, G, NW, 1, F8, kNtV>), grid, dim3(64 * NW), 0, stream, p);
  } else if (a.detect_sharing) {
    constexpr int NW = PA_DECODE_WAVES_WIDE;
    hipLaunchKernelGGL((decode_kernel<D, G, NW, 1, F8, kNtAuto>), grid, dim3(64 * NW), 0, stream,
                       p);
  } else {
    constexpr int NW = PA_DECODE_WAVES_WIDE;
    hipLaunchKernelGGL((decode_kernel<D, G, NW, 1, F8, 0>), grid, dim3(64 * NW), 0, stream, p);
  }
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

hipError_t launch_decode_bf16(const AttnArgs& a, hipStream_t stream) {
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
