// Prefill / chunked-prefill attention on bf16 matrix cores (fp32 accumulate).
//
// Method: "Inside the engine: kernels, CUDA graphs and the life of a request",
// section "Never materialise the T x T matrix": a tile of query rows stays on
// chip while K/V tiles stream past it; the softmax is kept incrementally with
// a running max m and denominator l, the accumulator rescaled by
// e^(m_old - m_new), so only O(T d) bytes move.  Keys and values are gathered
// through the block table ("Attention over a block table, not a contiguous
// tensor").  Rows of a request are causal with prior context: row i of a
// request with q_len new tokens sees positions 0 .. seq_len - q_len + i.
//
// MI355X design.  A work-group owns 256 query rows = (256 / G) tokens x the G
// query heads of one KV head (token-major), so each K/V tile staged in LDS
// serves every head that reads it.  Each of its eight waves (two per SIMD)
// owns 32 rows and runs 32x32x16 bf16 MFMAs:
//   S^T[key][row] = K[key][:] . Q[row][:]   A = K tile rows from LDS (16-byte
//                                          reads), B = Q in registers
//   O^T[d][row]  += V^T[d][keys] P[keys][row]  A = V^T tile (the cache block
//                                          is dim-major, so it lands in LDS
//                                          without a transpose), B = P taken
//                                          directly from the S^T accumulator
// With the S^T orientation a lane holds 16 keys of one query row, so the row
// max needs one cross-lane exchange per 32-key half.  Within each 16-key
// group the V^T tile stores keys in the order 0-3, 8-11, 4-7, 12-15, which is
// the order a lane's P operand carries them in, so one 16-byte LDS read gives
// the matching V operand.
//
// Key tiles are 64 keys (four cache blocks); K is double-buffered in LDS and
// V^T triple-buffered: the global loads of tile k+1 are issued before the
// MFMAs of tile k and written to LDS afterwards, one barrier per tile, and
// the P.V MFMAs of tile k-1 are spread through the softmax of tile k (whose
// exponentials would otherwise run with the matrix core idle).  The running max is
// only moved when a row's tile max exceeds it by more than 2^8 (base 2): the
// stale max keeps P <= 256, exact after the final division, and the
// accumulator rescale is skipped on almost every tile.
//
// A device-built work list, sorted by key count (longest first), holds one
// entry per (request, query tile) of requests with more new tokens than the
// decode kernel packs, so mixed batches launch without a host read of the
// metadata.  Work-group index = KV head fastest: the tiles of one (request, KV
// head) land on the same XCD (round-robin dispatch over 8 XCDs) and share its
// L2 copy of that head's K/V.
#include "decode_body.h"
#include "kv_write_body.h"
#include "prefill_body.h"

namespace pa {
namespace {

constexpr int kPlanBuckets = 4096;

// Work list: plan[0] = item count, then (request, query tile) pairs sorted by
// the number of keys the tile's last row sees, largest first.  `tmp` holds
// the unsorted list (2 ints per item).  Work-group 0 builds it; a second
// work-group, when launched, ranks the decode requests into `order` (the
// decode order of the same step, built beside the plan instead of in a
// launch of its own).
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ qsl,
                                                    const int32_t* __restrict__ seq_lens,
                                                    int32_t num_seqs, int32_t dq, int32_t tq,
                                                    int32_t shift, int32_t* __restrict__ plan,
                                                    int32_t* __restrict__ tmp, int32_t cap,
                                                    int32_t* __restrict__ claim,
                                                    int32_t* __restrict__ order,
                                                    int32_t order_shift,
                                                    const int32_t* __restrict__ tables,
                                                    int32_t table_stride) {
  __shared__ OrderSmem osm;
  __shared__ ShareSmem share;
  static_assert(kPlanBuckets == kBuckets, "the plan uses the decode order's histogram");
  if (blockIdx.x == 1) {
    decode_order_block(qsl, seq_lens, tables, table_stride, num_seqs, dq, order_shift, order,
                       osm, &share);
    return;
  }
  int* const s_scan = osm.part;
  int* const hist = osm.hist;
  const int tid = threadIdx.x;
  // the mixed kernel's work counters start from zero every call
  if (claim != nullptr && tid < 2) claim[tid] = 0;
  for (int i = tid; i < kPlanBuckets; i += 1024) hist[i] = 0;
  __syncthreads();
  // 1. enumerate items (request, tile) into tmp, histogram of weights; `run`
  // (the same in every thread) counts the items of earlier chunks
  int run = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += 1024) {
    const int b = c0 + tid;
    int n = 0, ql = 0, ctx = 0;
    if (b < num_seqs) {
      ql = qsl[b + 1] - qsl[b];
      ctx = seq_lens[b] - ql;
      if (ql > dq) n = (ql + tq - 1) / tq;
    }
    int chunk_items;
    const int base = run + block_scan<1024>(n, s_scan, chunk_items) - n;
    for (int k = 0; k < n; ++k) {
      const int idx = base + k;
      if (idx < cap) {
        tmp[2 * idx] = b;
        tmp[2 * idx + 1] = k;
        const int keys = ctx + min((k + 1) * tq, ql);
        atomicAdd(&hist[kPlanBuckets - 1 - min(keys >> shift, kPlanBuckets - 1)], 1);
      }
    }
    run += chunk_items;
  }
  __syncthreads();  // the histogram is complete
  const int count = min(run, cap);
  // 2. exclusive scan of the histogram (4 buckets per thread)
  int loc[4], s = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    loc[k] = s;
    s += hist[tid * 4 + k];
  }
  int all_items;
  const int base = block_scan<1024>(s, s_scan, all_items) - s;
#pragma unroll
  for (int k = 0; k < 4; ++k) hist[tid * 4 + k] = base + loc[k];
  __syncthreads();
  // 3. scatter in weight order
  for (int i = tid; i < count; i += 1024) {
    const int b = tmp[2 * i], k = tmp[2 * i + 1];
    const int ql = qsl[b + 1] - qsl[b];
    const int keys = seq_lens[b] - ql + min((k + 1) * tq, ql);
    const int pos = atomicAdd(&hist[kPlanBuckets - 1 - min(keys >> shift, kPlanBuckets - 1)], 1);
    plan[1 + 2 * pos] = b;
    plan[2 + 2 * pos] = k;
  }
  if (tid == 0) plan[0] = count;
}

template <int D, int G, int NW, int RG, int kBK, bool F8, bool CASC>
__global__ __launch_bounds__(64 * NW, 1) void prefill_kernel(PrefillParams p) {
  __shared__ __align__(16) PrefillSmem<D, kBK> sm;
  prefill_unit<D, G, NW, RG, kBK, F8, CASC>(p, blockIdx.x, sm, threadIdx.x);
}

// The work list (plan kernel; it also zeroes a.claim, and with_order: ranks
// the decode requests in a second work-group unless that order is already
// built) and, when the call writes the step's tokens, the write of the
// prefill rows' tokens (the decode kernel writes its own rows').
template <int G>
hipError_t plan_dg(const AttnArgs& a, hipStream_t stream, bool with_order) {
  int shift = 0;
  while ((a.max_seq_len >> shift) >= kPlanBuckets) ++shift;
  const bool order = with_order && a.decode_order != nullptr && !a.order_ready;
  trace_before(K_PLAN, stream);
  hipLaunchKernelGGL(plan_kernel, dim3(order ? 2 : 1), dim3(1024), 0, stream, a.qsl, a.seq_lens,
                     a.num_seqs, decode_max_q(G), prefill_tile_tokens(G), shift, a.plan,
                     a.plan_tmp, a.plan_cap, a.claim, order ? a.decode_order : nullptr,
                     decode_order_shift(a.max_seq_len), a.detect_sharing ? a.tables : nullptr,
                     a.table_stride);
  trace_after(stream);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && a.knew != nullptr) e = launch_kv_write_plan(a, prefill_tile_tokens(G), stream);
  return e;
}

template <int D, int G, bool F8>
void launch_dg(const AttnArgs& a, hipStream_t stream) {
  constexpr int NW = PA_PREFILL_WAVES;
  constexpr int RG = PA_PREFILL_ROW_GROUPS;
  constexpr int BK = PA_PREFILL_KEYS;
  const PrefillParams p = make_prefill_params(a);
  if (plan_dg<G>(a, stream, false) != hipSuccess) return;
  trace_before(K_PREFILL, stream);
  hipLaunchKernelGGL((prefill_kernel<D, G, NW, RG, BK, F8, false>), dim3(a.plan_cap * a.hkv),
                     dim3(64 * NW), 0, stream, p);
  trace_after(stream);
}

// Gathered decode rows of the sharers of a shared prefix: pre_index[b] = first
// gathered row of request b (or -1), vtok / vpos = flat token and position of
// every gathered row, count in casc_count[0].  Requests whose rows the decode
// kernel handles (0 < q_len <= dq, dq also bounded by the host's
// max_query_len, which sized the gathered-row buffers) take part; others keep
// pre_index = -1 and read the prefix themselves.  The decode order of the
// step (order nullable) is built in the same launch by a second work-group:
// one kernel boundary fewer on the step's serial path, and the two parts'
// memory round trips overlap.  cascade_setup_block<NT>(part) is called by
// every thread of an NT-thread work-group: part 0 gathers, part 1 ranks;
// sm is its LDS.
struct CascadeSetupArgs {
  const int32_t* sharers;
  int32_t num_sharers;
  const int32_t* qsl;
  const int32_t* seq_lens;
  int32_t num_seqs, dq;
  int32_t* pre_index;
  int32_t* vtok;
  int32_t* vpos;
  int32_t* count;
  int32_t* order;
  int32_t order_dq, order_shift;
};

typedef OrderSmem CascadeSetupSmem;

template <int NT>
__device__ __forceinline__ void cascade_setup_block(const CascadeSetupArgs& c,
                                                    CascadeSetupSmem& sm, int part) {
  if (part == 1) {
    // (no sharing test: the shared-prefix call streams every decode unit's V)
    decode_order_block<NT>(c.qsl, c.seq_lens, nullptr, 0, c.num_seqs, c.order_dq,
                           c.order_shift, c.order, sm, nullptr);
    return;
  }
  const int tid = threadIdx.x;
  for (int b = tid; b < c.num_seqs; b += NT) c.pre_index[b] = -1;
  // the sharers' pre_index entries are written after every -1 above
  __syncthreads();
  int run = 0;  // gathered rows of earlier chunks (the same in every thread)
  for (int c0 = 0; c0 < c.num_sharers; c0 += NT) {
    const int i = c0 + tid;
    int b = -1, ql = 0;
    if (i < c.num_sharers) {
      b = c.sharers[i];
      if (b >= 0 && b < c.num_seqs) {
        ql = c.qsl[b + 1] - c.qsl[b];
        if (ql <= 0 || ql > c.dq) ql = 0;
      }
    }
    int chunk_rows;
    const int v0 = run + block_scan<NT>(ql, sm.part, chunk_rows) - ql;
    if (ql > 0) {
      c.pre_index[b] = v0;
      const int ctx = c.seq_lens[b] - ql;
      for (int j = 0; j < ql; ++j) {
        c.vtok[v0 + j] = c.qsl[b] + j;
        c.vpos[v0 + j] = ctx + j;
      }
    }
    run += chunk_rows;
  }
  if (tid == 0) c.count[0] = run;
}

// work-groups of the setup: the gather, and the ranking when it is asked for
inline int cascade_setup_groups(const CascadeSetupArgs& c) { return c.order != nullptr ? 2 : 1; }

__global__ __launch_bounds__(1024) void cascade_setup_kernel(CascadeSetupArgs c) {
  __shared__ CascadeSetupSmem sm;
  cascade_setup_block<1024>(c, sm, blockIdx.x);
}

// The first launch of the one-call shared-prefix step: the first one or two
// work-groups run the setup above (at 256 threads), the others write the
// step's new tokens exactly as pa_kv_write does (16 flat tokens of one KV
// head each).  The two are independent (the setup reads only metadata), so
// the setup's latency hides under the write, and both are done before the
// prefix stage reads the cache.
__global__ __launch_bounds__(256) void cascade_write_setup_kernel(
    CascadeSetupArgs c, const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, const int64_t* __restrict__ slots,
    int32_t nt, int32_t hkv, int32_t d, int64_t num_slots, int32_t setup_groups) {
  __shared__ __align__(16) union {
    CascadeSetupSmem setup;
    WriteStage<uint16_t> write;
  } sm;
  if ((int)blockIdx.x < setup_groups) {
    cascade_setup_block<256>(c, sm.setup, blockIdx.x);
    return;
  }
  const int w = blockIdx.x - setup_groups;
  const int t0 = (w / hkv) * kWriteTokens;
  write_tokens<uint16_t>(key, value, kc, vc, slots, t0, min(kWriteTokens, nt - t0), w % hkv, hkv,
                         d, num_slots, sm.write.vrow, sm.write.slot, threadIdx.x);
}

template <int G>
CascadeSetupArgs cascade_setup_args(const AttnArgs& a) {
  CascadeSetupArgs c;
  c.sharers = a.sharers;
  c.num_sharers = a.num_sharers;
  c.qsl = a.qsl;
  c.seq_lens = a.seq_lens;
  c.num_seqs = a.num_seqs;
  c.dq = min(decode_max_q(G), a.max_query_len);
  c.pre_index = a.pre_index;
  c.vtok = a.vtok;
  c.vpos = a.vpos;
  c.count = a.casc_count;
  c.order = a.decode_order;
  c.order_dq = decode_max_q(G);
  c.order_shift = decode_order_shift(a.max_seq_len);
  return c;
}

template <int G>
void cascade_write_setup_g(const AttnArgs& a, hipStream_t stream) {
  const int64_t groups = ((int64_t)a.num_tokens + kWriteTokens - 1) / kWriteTokens;
  const CascadeSetupArgs c = cascade_setup_args<G>(a);
  const int setup_groups = cascade_setup_groups(c);
  trace_before(K_CASCADE_WRITE_SETUP, stream);
  hipLaunchKernelGGL(cascade_write_setup_kernel, dim3((unsigned)(setup_groups + groups * a.hkv)),
                     dim3(256), 0, stream, c, (const uint16_t*)a.knew, (const uint16_t*)a.vnew,
                     (uint16_t*)a.kc, (uint16_t*)a.vc, a.slots, a.num_tokens, a.hkv, a.d,
                     a.num_blocks * kWriteTokens, setup_groups);
  trace_after(stream);
}

template <int D, int G>
void launch_cascade_dg(const AttnArgs& a, hipStream_t stream) {
  constexpr int NW = PA_PREFILL_WAVES;
  constexpr int RG = PA_PREFILL_ROW_GROUPS;
  constexpr int BK = PA_PREFILL_KEYS;
  constexpr int TQ = 32 * RG * NW / G;
  PrefillParams p = {};
  p.q = (const uint16_t*)a.q;
  p.kc = a.kc;
  p.vc = a.vc;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.scale_log2 = a.scale * kLog2e;
  p.casc_count = a.casc_count;
  p.vtok = a.vtok;
  p.vpos = a.vpos;
  p.pre_blocks = a.pre_blocks;
  p.pre_tokens = 16 * a.num_pre_blocks;
  p.pre_splits = a.casc_ksplits;
  p.pre_chunk = a.casc_kchunk;
  p.pre_rows = a.casc_rows_max;
  p.pre_out = a.pre_out;
  p.pre_lse = a.pre_lse;
  if (!a.casc_setup_ready) {
    trace_before(K_CASCADE_SETUP, stream);
    const CascadeSetupArgs c = cascade_setup_args<G>(a);
    hipLaunchKernelGGL(cascade_setup_kernel, dim3(cascade_setup_groups(c)), dim3(1024), 0,
                       stream, c);
    trace_after(stream);
  }
  const int tiles = (a.casc_rows_max + TQ - 1) / TQ;
  trace_before(K_CASCADE_PREFIX, stream);
  hipLaunchKernelGGL((prefill_kernel<D, G, NW, RG, BK, false, true>),
                     dim3(tiles * a.casc_ksplits * a.hkv), dim3(64 * NW), 0, stream, p);
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

hipError_t launch_cascade_prefix(const AttnArgs& a, hipStream_t stream) {
  if (a.d == 64) {
    switch (a.hq / a.hkv) {
      case 1: launch_cascade_dg<64, 1>(a, stream); break;
      case 2: launch_cascade_dg<64, 2>(a, stream); break;
      case 4: launch_cascade_dg<64, 4>(a, stream); break;
      case 8: launch_cascade_dg<64, 8>(a, stream); break;
      default: launch_cascade_dg<64, 16>(a, stream); break;
    }
  } else {
    switch (a.hq / a.hkv) {
      case 1: launch_cascade_dg<128, 1>(a, stream); break;
      case 2: launch_cascade_dg<128, 2>(a, stream); break;
      case 4: launch_cascade_dg<128, 4>(a, stream); break;
      case 8: launch_cascade_dg<128, 8>(a, stream); break;
      default: launch_cascade_dg<128, 16>(a, stream); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_cascade_write_setup(const AttnArgs& a, hipStream_t stream) {
  switch (a.hq / a.hkv) {
    case 1: cascade_write_setup_g<1>(a, stream); break;
    case 2: cascade_write_setup_g<2>(a, stream); break;
    case 4: cascade_write_setup_g<4>(a, stream); break;
    case 8: cascade_write_setup_g<8>(a, stream); break;
    default: cascade_write_setup_g<16>(a, stream); break;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_plan(const AttnArgs& a, hipStream_t stream, bool with_order) {
  switch (a.hq / a.hkv) {
    case 1: return plan_dg<1>(a, stream, with_order);
    case 2: return plan_dg<2>(a, stream, with_order);
    case 4: return plan_dg<4>(a, stream, with_order);
    case 8: return plan_dg<8>(a, stream, with_order);
    default: return plan_dg<16>(a, stream, with_order);
  }
}

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t stream) {
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
