// Internal declarations shared by the host API and the kernel translation
// units of the paged-attention library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

// ---- kernel ids for tracing -------------------------------------------------
enum KernelId : int32_t {
  K_KV_WRITE = 0,
  K_DECODE = 1,
  K_DECODE_SPLIT = 2,
  K_COMBINE = 3,
  K_PLAN = 4,
  K_PREFILL = 5,
  K_F32_ATTN = 6,
  K_F32_ATTN_SPLIT = 7,
  K_DECODE_ORDER = 8,
  K_ZERO = 9,
  K_KV_WRITE_FP8 = 10,
  K_ROPE_KV_WRITE = 11,
  K_CASCADE_SETUP = 12,
  K_CASCADE_PREFIX = 13,
  K_MIXED = 14,
  K_CASCADE_WRITE_SETUP = 15,
  K_COUNT = 16
};

// Tracing hooks (pa_api.cpp).  trace_before/after bracket one launch.
void trace_before(int32_t kernel_id, hipStream_t stream);
void trace_after(hipStream_t stream);

// ---- launchers (each enqueues on `stream` and returns hipGetLastError) ------
hipError_t launch_kv_write(const void* key, const void* value, void* kc, void* vc,
                           const int64_t* slots, int32_t nt, int32_t hkv,
                           int32_t d, int32_t esize, int64_t num_blocks,
                           hipStream_t stream);
// Quantising write into an E4M3 cache (one byte per element), per-KV-head
// float scales: code = e4m3(clamp(x / scale[h], -448, 448)), ties to even.
// Rotary embedding of Q (in place) and the new K, fused with the KV write.
hipError_t launch_rope_kv_write(void* query, const void* key, const void* value, void* kc,
                                void* vc, const int64_t* slots, const int64_t* positions,
                                const float* cos_sin, int32_t max_position, int32_t nt,
                                int32_t hq, int32_t hkv, int32_t d, int32_t esize,
                                int64_t num_blocks, hipStream_t stream);
hipError_t launch_kv_write_fp8(const void* key, const void* value, void* kc, void* vc,
                               const int64_t* slots, const float* k_scale,
                               const float* v_scale, int32_t nt, int32_t hkv, int32_t d,
                               int32_t esize, int64_t num_blocks, hipStream_t stream);

struct AttnArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* tables;
  int32_t num_seqs, num_tokens, max_query_len, max_seq_len;
  int32_t hq, hkv, d, table_stride;
  float scale;
  int32_t splits;
  void* out;
  float* lse;
  float* part_out;      // [splits][nt][hq][d] when splits > 1
  float* part_lse;      // [splits][nt][hq]
  int32_t* plan;        // work list of the matrix-core kernel: count + 2 ints/item
  int32_t* plan_tmp;    // unsorted work list (2 ints/item)
  int32_t plan_cap;     // capacity of the work list (items)
  int32_t* decode_order;  // nullable: count + ranked decode requests
  int32_t* claim;         // [2] work counters of the mixed kernel (prefill, decode)
  int32_t order_ready;    // 1: decode_order was already built this call
  int32_t casc_setup_ready;  // 1: the shared-prefix setup already ran this call
  int32_t unshared;       // 1: no cache block is read by two requests of the step
                          //    (the many-unit decode then streams V non-temporally)
  int32_t detect_sharing; // 1: the decode order marks the requests whose first block
                          //    no other request has, and the many-unit decode streams
                          //    their V non-temporally
  int32_t num_cus;        // compute units of the current device
  int32_t* sem;           // nullable: zeroed arrival counters, one per (request, KV head)
  int32_t cache_fp8;      // 1: kc / vc hold E4M3 codes (query and out bf16)
  const float* k_scale;   // [hkv] when cache_fp8: a cached K value is code * k_scale[h]
  const float* v_scale;   // [hkv] when cache_fp8
  // shared-prefix (cascade) attention; sharers == nullptr: none
  const int32_t* sharers;     // [num_sharers] request indices
  int32_t num_sharers;
  const int32_t* pre_blocks;  // [num_pre_blocks] the shared prefix's blocks
  int32_t num_pre_blocks;
  int32_t casc_rows_max;      // bound on gathered rows (grid of the prefix stage)
  int32_t casc_ksplits;       // key ranges of the prefix stage (partials per row)
  int32_t casc_kchunk;        // keys per range, a multiple of 64
  int32_t* pre_index;         // [num_seqs] first gathered row of each request, or -1
  int32_t* vtok;              // [casc_rows_max]
  int32_t* vpos;              // [casc_rows_max]
  int32_t* casc_count;        // [1]
  float* pre_out;             // [casc_ksplits][casc_rows_max][hq][d]
  float* pre_lse;             // [casc_ksplits][casc_rows_max][hq]
  // fused decode step (bf16): new K/V and slots written by the decode kernel
  const void* knew;           // nullable
  const void* vnew;
  const int64_t* slots;
  int64_t num_blocks;
};

// Largest number of new tokens per request that the decode kernel packs.
inline int32_t decode_max_q(int32_t group) { return 16 / group; }
// Prefill work-group shape: PA_PREFILL_WAVES waves, each owning
// PA_PREFILL_ROW_GROUPS groups of 32 query rows.
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
#ifndef PA_PREFILL_ROW_GROUPS
#define PA_PREFILL_ROW_GROUPS 1
#endif
// Query tokens per work-group of the prefill kernel.
inline int32_t prefill_tile_tokens(int32_t group) {
  return 32 * PA_PREFILL_ROW_GROUPS * PA_PREFILL_WAVES / group;
}

// KV write of the tokens of the matrix-core kernel's work list (a.plan, built
// on the same stream first): a.knew / a.vnew / a.slots into a.kc / a.vc, bf16
// or quantised to E4M3 (a.cache_fp8), tq tokens per work item.
hipError_t launch_kv_write_plan(const AttnArgs& a, int32_t tq, hipStream_t stream);
hipError_t launch_decode_bf16(const AttnArgs& a, hipStream_t stream);
// The pieces of a step with prefill rows, run as one persistent launch:
// the matrix-core kernel's work list (a.claim zeroed; with_order: the decode
// order built beside it; with a.knew, then the write of its tokens), then
// the mixed kernel whose work-groups take prefill units and decode units
// from two counters.
hipError_t launch_prefill_plan(const AttnArgs& a, hipStream_t stream, bool with_order);
hipError_t launch_mixed_bf16(const AttnArgs& a, hipStream_t stream);
hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t stream);
// shared-prefix stage: gather the sharers' decode rows (unless
// a.casc_setup_ready), attend them to the shared blocks (partials in pre_out
// / pre_lse); the decode kernel merges
hipError_t launch_cascade_prefix(const AttnArgs& a, hipStream_t stream);
// one launch: the shared-prefix setup (gathered rows and decode order) beside
// the KV write of all a.num_tokens tokens (a.knew / a.vnew / a.slots, bf16)
hipError_t launch_cascade_write_setup(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream);
hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t stream);
hipError_t launch_combine(const float* po, const float* pl, int32_t splits,
                          int32_t nt, int32_t hq, int32_t d, void* out, float* lse,
                          int32_t out_bf16, const int32_t* qsl, int32_t num_seqs,
                          int32_t decode_max_q, hipStream_t stream);

// pa_decode_step (shared with the no-alloc entry point, which passes the
// library's own workspace).
pa_status decode_step_impl(const void* key, const void* value, void* key_cache,
                           void* value_cache, const int64_t* slot_mapping, const void* query,
                           const int32_t* query_start_loc, const int32_t* seq_lens,
                           const int32_t* block_tables, int32_t num_seqs, int32_t num_tokens,
                           int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t block_table_stride, int64_t num_blocks, float scale,
                           int32_t num_splits, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, pa_dtype dtype, void* stream);

}  // namespace pa
