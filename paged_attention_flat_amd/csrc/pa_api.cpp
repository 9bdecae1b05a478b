// Host side of the C ABI declared in include/pa.h: argument validation, the
// launch plan of one flat step, the split / no-split crossover and the
// optional kernel tracing.  No entry point synchronises or reads device
// memory; grids are sized from host scalars only.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace pa {
namespace {

// ---- tracing ----------------------------------------------------------------
struct TraceState {
  std::mutex mu;
  bool active = false;
  int32_t capacity = 0;
  int32_t used = 0;
  std::vector<hipEvent_t> start, stop;
  std::vector<int32_t> ids;
};

TraceState& trace() {
  static TraceState* s = new TraceState();  // never destroyed: safe at exit
  return *s;
}

thread_local int32_t g_pending = -1;

void destroy_events(TraceState& t) {
  for (auto e : t.start) hipEventDestroy(e);
  for (auto e : t.stop) hipEventDestroy(e);
  t.start.clear();
  t.stop.clear();
  t.ids.clear();
  t.capacity = 0;
  t.used = 0;
}

int32_t device_cu_count() {
  static std::atomic<int32_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64) {
    const int32_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool is_pow2_group(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t plan_capacity(int32_t num_seqs, int32_t num_tokens) {
  // items <= sum over prefill requests of ceil(q_len / TQ) <= num_tokens / TQ
  // + (number of such requests); TQ >= 8 and at most min(num_seqs,
  // num_tokens / 2) requests qualify (they have >= 2 tokens)
  const size_t by_tokens = (size_t)num_tokens / 8 + 1;
  const size_t reqs = std::min<size_t>((size_t)num_seqs, (size_t)num_tokens / 2 + 1);
  return by_tokens + reqs;
}

// Workspace layout (each region 256-byte aligned):
//   [split-merge counters: num_seqs * hq ints, zero between calls]
//   [plan: 1 + 2 * cap ints][plan_tmp: 2 * cap ints][decode order: 1 + num_seqs ints]
//   [mixed kernel's work counters: 2 ints, zeroed by the plan kernel]
//   [partial out: splits * nt * hq * d floats][partial lse: splits * nt * hq floats]
struct WsLayout {
  size_t sem, plan, plan_tmp, order, claim, part_out, part_lse;
  size_t pre_index, vtok, vpos, casc_count, pre_out, pre_lse;  // cascade only
  size_t total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// casc_rows > 0: room for the shared-prefix stage (gathered rows, their
// partials) and split partials even at one split (sharers always merge).
WsLayout ws_layout(int32_t num_seqs, int32_t num_tokens, int32_t hq, int32_t d, int32_t splits,
                   int64_t casc_rows = 0, int32_t casc_ksplits = 1) {
  WsLayout w = {};
  const size_t cap = plan_capacity(num_seqs, num_tokens);
  // arrival counters of the split merge, one per (request, KV head <= Hq);
  // must be zero on entry and are left zero by every call
  w.sem = 0;
  w.plan = align256((size_t)num_seqs * hq * sizeof(int32_t));
  w.plan_tmp = align256(w.plan + (1 + 2 * cap) * sizeof(int32_t));
  w.order = align256(w.plan_tmp + 2 * cap * sizeof(int32_t));
  w.claim = align256(w.order + (1 + (size_t)num_seqs) * sizeof(int32_t));
  w.part_out = align256(w.claim + 2 * sizeof(int32_t));
  w.part_lse = w.part_out;
  w.total = w.part_out;
  if (splits > 1 || casc_rows > 0) {
    const size_t rows = (size_t)splits * num_tokens * hq;
    w.part_lse = align256(w.part_out + rows * d * sizeof(float));
    w.total = align256(w.part_lse + rows * sizeof(float));
  }
  if (casc_rows > 0) {
    const size_t R = (size_t)casc_rows;
    w.pre_index = w.total;
    w.vtok = align256(w.pre_index + (size_t)num_seqs * sizeof(int32_t));
    w.vpos = align256(w.vtok + R * sizeof(int32_t));
    w.casc_count = align256(w.vpos + R * sizeof(int32_t));
    const size_t KR = (size_t)casc_ksplits * R;
    w.pre_out = align256(w.casc_count + sizeof(int32_t));
    w.pre_lse = align256(w.pre_out + KR * hq * d * sizeof(float));
    w.total = align256(w.pre_lse + KR * hq * sizeof(float));
  }
  return w;
}

// Key ranges of the shared-prefix stage: enough work-groups for one per
// compute unit (the matrix-core kernel's LDS admits one per CU, so a second
// round only adds start-up, partial stores and partials for the decode
// kernel to merge), each range a whole number of 64-key tiles.
void cascade_key_split(int32_t num_pre_blocks, int64_t casc_rows, int32_t group, int32_t hkv,
                       int32_t num_cus, int32_t* ksplits, int32_t* kchunk) {
  const int64_t tq = prefill_tile_tokens(group);
  const int64_t tiles = std::max<int64_t>(1, (casc_rows + tq - 1) / tq);
  const int64_t units = tiles * hkv;
  const int64_t ktiles = std::max<int64_t>(1, (num_pre_blocks + 3) / 4);  // 64-key tiles
  int64_t ks = std::max<int64_t>(1, ((int64_t)num_cus + units - 1) / units);
  ks = std::min<int64_t>(ks, std::min<int64_t>(ktiles, 64));
  const int64_t per = (ktiles + ks - 1) / ks;                  // tiles per range
  *ksplits = (int32_t)((ktiles + per - 1) / per);              // no empty range
  *kchunk = (int32_t)(per * 64);
}

size_t workspace_bytes_for(int32_t num_seqs, int32_t num_tokens, int32_t hq, int32_t d,
                           int32_t splits) {
  return ws_layout(num_seqs, num_tokens, hq, d, splits).total;
}


}  // namespace

void trace_before(int32_t kernel_id, hipStream_t stream) {
  TraceState& t = trace();
  std::lock_guard<std::mutex> lk(t.mu);
  g_pending = -1;
  if (!t.active || t.used >= t.capacity) return;
  g_pending = t.used++;
  t.ids[g_pending] = kernel_id;
  hipEventRecord(t.start[g_pending], stream);
}

void trace_after(hipStream_t stream) {
  if (g_pending < 0) return;
  TraceState& t = trace();
  std::lock_guard<std::mutex> lk(t.mu);
  hipEventRecord(t.stop[g_pending], stream);
  g_pending = -1;
}

}  // namespace pa

using namespace pa;

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t pa_version(void) { return 100; }  // 0.1.0

namespace {
std::atomic<int32_t> g_unshared{0};  // pa_set_unshared_blocks: 1, 0 (automatic) or -1
}  // namespace

int32_t pa_set_unshared_blocks(int32_t mode) {
  return g_unshared.exchange(mode > 0 ? 1 : (mode < 0 ? -1 : 0));
}

const char* pa_kernel_name(int32_t id) {
  switch (id) {
    case K_KV_WRITE: return "kv_write";
    case K_DECODE: return "decode";
    case K_DECODE_SPLIT: return "decode_split_partial";
    case K_COMBINE: return "split_combine";
    case K_PLAN: return "prefill_plan";
    case K_PREFILL: return "prefill_mfma";
    case K_F32_ATTN: return "attn_f32";
    case K_F32_ATTN_SPLIT: return "attn_f32_split_partial";
    case K_DECODE_ORDER: return "decode_order";
    case K_ZERO: return "workspace_zero";
    case K_KV_WRITE_FP8: return "kv_write_fp8";
    case K_ROPE_KV_WRITE: return "rope_kv_write";
    case K_CASCADE_SETUP: return "cascade_setup";
    case K_CASCADE_PREFIX: return "cascade_prefix";
    case K_MIXED: return "mixed_prefill_decode";
    case K_CASCADE_WRITE_SETUP: return "cascade_write_setup";
  }
  return "unknown";
}

pa_status pa_trace_begin(int32_t capacity) {
  if (capacity <= 0 || capacity > (1 << 20)) return PA_ERR_INVALID;
  TraceState& t = trace();
  std::lock_guard<std::mutex> lk(t.mu);
  destroy_events(t);
  t.start.resize(capacity);
  t.stop.resize(capacity);
  t.ids.assign(capacity, -1);
  for (int32_t i = 0; i < capacity; ++i) {
    if (hipEventCreate(&t.start[i]) != hipSuccess || hipEventCreate(&t.stop[i]) != hipSuccess) {
      t.start.resize(i);
      t.stop.resize(i);
      destroy_events(t);
      return PA_ERR_HIP;
    }
  }
  t.capacity = capacity;
  t.used = 0;
  t.active = true;
  return PA_OK;
}

pa_status pa_trace_end(void) {
  TraceState& t = trace();
  std::lock_guard<std::mutex> lk(t.mu);
  t.active = false;
  return PA_OK;
}

int32_t pa_trace_read(int32_t* kernel_ids, float* ms, int32_t capacity) {
  if (kernel_ids == nullptr || ms == nullptr || capacity < 0) return -1;
  TraceState& t = trace();
  std::lock_guard<std::mutex> lk(t.mu);
  const int32_t n = std::min(capacity, t.used);
  for (int32_t i = 0; i < n; ++i) {
    float v = -1.f;
    if (hipEventElapsedTime(&v, t.start[i], t.stop[i]) != hipSuccess) v = -1.f;
    kernel_ids[i] = t.ids[i];
    ms[i] = v;
  }
  return n;
}

size_t pa_attention_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                   int32_t head_dim, int32_t num_splits) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits < 1)
    return 0;
  return workspace_bytes_for(num_seqs, num_tokens, num_q_heads, head_dim, num_splits);
}

static constexpr int64_t kMaxHeuristicSplits = 64;

int32_t pa_choose_num_splits(int32_t num_seqs, int32_t max_query_len, int32_t max_seq_len,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t num_cus) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 || max_seq_len <= 0) return 1;
  const int32_t group = num_q_heads / num_kv_heads;
  if (group <= 0 || group > 16) return 1;
  if (max_query_len > decode_max_q(group)) return 1;  // prefill rows present
  if (num_cus <= 0) num_cus = device_cu_count();
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  if (units >= num_cus) return 1;
  // one split work-group per CU: each split adds a partial to merge, and a
  // second resident work-group per CU gains less than that costs
  const int64_t want = ((int64_t)num_cus + units - 1) / units;
  const int64_t blocks = (max_seq_len + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE;
  const int64_t by_blocks = std::max<int64_t>(1, blocks / 8);  // >= 8 blocks per split
  int64_t s = std::min<int64_t>(want, by_blocks);
  // the last split of a (request, KV head) merges every partial of its rows;
  // past 64 partials that merge needs several dependent rounds of loads and
  // costs more than the extra work-groups gain (one request of 32768 keys on
  // one KV head: 256 splits 26.1 us, 128: 18.4, 64: 17.7, 32: 22.4)
  s = std::min<int64_t>(s, kMaxHeuristicSplits);
  s = std::min<int64_t>(s, PA_MAX_SPLITS);
  return (int32_t)std::max<int64_t>(1, s);
}

int32_t pa_capture_size(int32_t num_tokens, int32_t max_size) {
  if (num_tokens < 1 || num_tokens > max_size) return -1;
  int32_t size;
  if (num_tokens <= 2) size = num_tokens;
  else if (num_tokens <= 4) size = 4;
  else if (num_tokens < 256) size = (num_tokens + 7) & ~7;
  else size = (num_tokens + 15) & ~15;
  return size <= max_size ? size : -1;
}

pa_status pa_kv_write(const void* key, const void* value, void* key_cache, void* value_cache,
                      const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                      void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID;
  if (block_size != PA_BLOCK_SIZE) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return PA_ERR_INVALID;
  const int32_t esize = dtype == PA_BF16 ? 2 : 4;
  hipError_t e = launch_kv_write(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                 num_kv_heads, head_dim, esize, num_blocks, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_attention_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return PA_OK;
  if (workspace == nullptr) return PA_ERR_NULL;
  if (!aligned16(workspace)) return PA_ERR_INVALID;
  hipError_t e = launch_zero(workspace, workspace_bytes, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_split_combine(const float* partial_out, const float* partial_lse,
                           int32_t num_splits, int32_t num_tokens, int32_t num_q_heads,
                           int32_t head_dim, void* out, float* lse, pa_dtype dtype,
                           void* stream) {
  if (num_splits < 1 || num_splits > PA_MAX_SPLITS || num_tokens < 0 || num_q_heads <= 0)
    return PA_ERR_INVALID;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!partial_out || !partial_lse || !out) return PA_ERR_NULL;
  if (!aligned16(partial_out) || !aligned16(out)) return PA_ERR_INVALID;
  hipError_t e = launch_combine(partial_out, partial_lse, num_splits, num_tokens, num_q_heads,
                                head_dim, out, lse, dtype == PA_BF16, nullptr, 0, 0,
                                (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"

namespace {

// Shared by pa_attention_fwd (cache in the query dtype) and
// pa_attention_fwd_fp8 (E4M3 cache with per-KV-head scales, bf16 query).
pa_status attention_impl(const void* query, const void* key_cache, const void* value_cache,
                         const float* k_scale, const float* v_scale,
                         const int32_t* query_start_loc, const int32_t* seq_lens,
                         const int32_t* block_tables, int32_t num_seqs, int32_t num_tokens,
                         int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t block_table_stride, int64_t num_blocks, float scale,
                         int32_t num_splits, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, pa_dtype dtype, bool cache_fp8, void* stream,
                         const int32_t* sharers = nullptr, int32_t num_sharers = 0,
                         const int32_t* pre_blocks = nullptr, int32_t num_pre_blocks = 0,
                         const void* knew = nullptr, const void* vnew = nullptr,
                         const int64_t* slots = nullptr) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_blocks <= 0 || num_splits < 0 || num_splits > PA_MAX_SPLITS || !std::isfinite(scale) ||
      !(scale > 0.f))
    return PA_ERR_INVALID;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID;
  const int32_t group = num_q_heads / num_kv_heads;
  if (!is_pow2_group(group)) return PA_ERR_UNSUPPORTED;
  if (block_size != PA_BLOCK_SIZE) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (max_query_len < 1 || max_query_len > num_tokens || max_seq_len < max_query_len)
    return PA_ERR_INVALID;
  if ((int64_t)block_table_stride * PA_BLOCK_SIZE < (int64_t)max_seq_len) return PA_ERR_INVALID;
  if (!query || !key_cache || !value_cache || !query_start_loc || !seq_lens || !block_tables ||
      !out)
    return PA_ERR_NULL;
  if (cache_fp8 && (!k_scale || !v_scale)) return PA_ERR_NULL;
  if (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) || !aligned16(out))
    return PA_ERR_INVALID;

  const int32_t splits =
      num_splits == 0 ? pa_choose_num_splits(num_seqs, max_query_len, max_seq_len, num_q_heads,
                                             num_kv_heads, 0)
                      : num_splits;
  const bool cascade = sharers != nullptr && num_sharers > 0 && num_pre_blocks > 0;
  const int64_t casc_rows =
      cascade ? (int64_t)num_sharers * std::min<int32_t>(max_query_len, decode_max_q(group)) : 0;
  int32_t ksplits = 1, kchunk = 0;
  if (cascade)
    cascade_key_split(num_pre_blocks, casc_rows, group, num_kv_heads, device_cu_count(), &ksplits,
                      &kchunk);
  const size_t need =
      ws_layout(num_seqs, num_tokens, num_q_heads, head_dim, splits, casc_rows, ksplits).total;
  if (workspace == nullptr || workspace_bytes < need) return PA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PA_ERR_INVALID;

  AttnArgs a = {};
  a.q = query;
  a.kc = key_cache;
  a.vc = value_cache;
  a.qsl = query_start_loc;
  a.seq_lens = seq_lens;
  a.tables = block_tables;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.max_query_len = max_query_len;
  a.max_seq_len = max_seq_len;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.d = head_dim;
  a.table_stride = block_table_stride;
  a.scale = scale;
  a.splits = splits;
  a.out = out;
  a.lse = lse;
  char* ws = static_cast<char*>(workspace);
  const WsLayout lay =
      ws_layout(num_seqs, num_tokens, num_q_heads, head_dim, splits, casc_rows, ksplits);
  a.plan = reinterpret_cast<int32_t*>(ws + lay.plan);
  a.plan_tmp = reinterpret_cast<int32_t*>(ws + lay.plan_tmp);
  {
    // tighter bound for this group size (the workspace holds the loosest one)
    const int64_t tq = prefill_tile_tokens(group), dq = decode_max_q(group);
    const int64_t cap = num_tokens / tq + 1 +
                        std::min<int64_t>(num_seqs, num_tokens / (dq + 1) + 1);
    a.plan_cap = (int32_t)std::min<int64_t>(cap, (int64_t)plan_capacity(num_seqs, num_tokens));
  }
  // rank decode requests longest-first when they outnumber the compute units
  a.num_cus = device_cu_count();
  a.decode_order = nullptr;
  if ((int64_t)num_seqs * num_kv_heads * splits > a.num_cus && num_seqs >= 64)
    a.decode_order = reinterpret_cast<int32_t*>(ws + lay.order);
  a.claim = reinterpret_cast<int32_t*>(ws + lay.claim);
  a.cache_fp8 = cache_fp8 ? 1 : 0;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.part_out = nullptr;
  a.part_lse = nullptr;
  a.sem = nullptr;
  if (splits > 1 || cascade) {
    a.part_out = reinterpret_cast<float*>(ws + lay.part_out);
    a.part_lse = reinterpret_cast<float*>(ws + lay.part_lse);
    a.sem = reinterpret_cast<int32_t*>(ws + lay.sem);
  }
  // the decode rows' blocks are unshared when the caller says so, and in a
  // shared-prefix call once the prefix is read by its own stage
  const int32_t share_mode = g_unshared.load(std::memory_order_relaxed);
  a.unshared = (cascade || share_mode > 0) ? 1 : 0;
  // otherwise, by default, the decode order marks the requests that share no
  // block when the many-work-group shape or the persistent launch reads them
  const int32_t dq_group = decode_max_q(group);
  const bool many_units = (int64_t)num_seqs * num_kv_heads * splits > 2 * (int64_t)a.num_cus ||
                          max_query_len > dq_group;
  a.detect_sharing =
      (!a.unshared && share_mode == 0 && a.decode_order != nullptr && many_units) ? 1 : 0;
  a.sharers = cascade ? sharers : nullptr;
  a.num_sharers = cascade ? num_sharers : 0;
  a.pre_blocks = pre_blocks;
  a.num_pre_blocks = cascade ? num_pre_blocks : 0;
  a.knew = knew;
  a.vnew = vnew;
  a.slots = slots;
  a.num_blocks = num_blocks;
  a.casc_rows_max = (int32_t)casc_rows;
  a.casc_ksplits = ksplits;
  a.casc_kchunk = kchunk;
  a.pre_index = cascade ? reinterpret_cast<int32_t*>(ws + lay.pre_index) : nullptr;
  a.vtok = cascade ? reinterpret_cast<int32_t*>(ws + lay.vtok) : nullptr;
  a.vpos = cascade ? reinterpret_cast<int32_t*>(ws + lay.vpos) : nullptr;
  a.casc_count = cascade ? reinterpret_cast<int32_t*>(ws + lay.casc_count) : nullptr;
  a.pre_out = cascade ? reinterpret_cast<float*>(ws + lay.pre_out) : nullptr;
  a.pre_lse = cascade ? reinterpret_cast<float*>(ws + lay.pre_lse) : nullptr;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (dtype == PA_F32) {
    e = launch_attn_f32(a, s);
    if (e == hipSuccess && splits > 1)
      e = launch_combine(a.part_out, a.part_lse, splits, num_tokens, num_q_heads, head_dim, out,
                         lse, 0, query_start_loc, num_seqs, 1 << 30, s);
  } else {
    // The bf16 decode kernel merges its own split partials (the last split of
    // each request and KV head to finish does it).  A step with prefill rows
    // that certainly also has decode rows (more requests than can each hold
    // more than dq of the step's tokens) runs its MFMA-bound prefill units
    // and its HBM-bound decode units in one persistent launch (mixed.hip);
    // with a shared prefix, the prefix stage runs first, since the sharers'
    // decode units merge its partials.  Otherwise the matrix-core kernel runs
    // on its own: in persistent form it is ~4 % slower, which only an
    // overlap repays.
    const int32_t dq = decode_max_q(group);
    const bool prefill = max_query_len > dq;
    const bool has_decode_rows = (int64_t)num_seqs > (int64_t)num_tokens / (dq + 1);
    if (cascade) {
      if (a.knew != nullptr) {
        // one-call shared-prefix step: the setup's launch also writes every
        // new token (before the stage reads the cache), so nothing later
        // writes again
        e = launch_cascade_write_setup(a, s);
        a.casc_setup_ready = 1;
        a.knew = nullptr;
        a.vnew = nullptr;
        a.slots = nullptr;
      }
      if (e == hipSuccess) e = launch_cascade_prefix(a, s);
      a.order_ready = 1;  // its setup also ranked the decode requests
    }
    if (e == hipSuccess && prefill && has_decode_rows) {
      e = launch_mixed_bf16(a, s);
    } else if (e == hipSuccess) {
      if (prefill) e = launch_prefill_bf16(a, s);
      if (e == hipSuccess) e = launch_decode_bf16(a, s);
    }
  }
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

namespace pa {

pa_status decode_step_impl(const void* key, const void* value, void* key_cache,
                           void* value_cache, const int64_t* slot_mapping, const void* query,
                           const int32_t* query_start_loc, const int32_t* seq_lens,
                           const int32_t* block_tables, int32_t num_seqs, int32_t num_tokens,
                           int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t block_table_stride, int64_t num_blocks, float scale,
                           int32_t num_splits, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, pa_dtype dtype, void* stream) {
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return PA_ERR_INVALID;
  const int32_t group = num_q_heads / num_kv_heads;
  // one call for bf16: the decode kernel writes the decode rows' tokens (and
  // those after the last request), and in a step with prefill rows a write
  // over the matrix-core kernel's work list writes theirs ahead of it
  const bool fuse = dtype == PA_BF16 && is_pow2_group(group) && num_seqs > 0 &&
                    num_tokens > 0 && max_query_len >= 1;
  if (!fuse) {
    // the two calls in order (same results, two launches)
    pa_status st = pa_kv_write(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                               num_kv_heads, head_dim, block_size, num_blocks, dtype, stream);
    if (st != PA_OK) return st;
    return attention_impl(query, key_cache, value_cache, nullptr, nullptr, query_start_loc,
                          seq_lens, block_tables, num_seqs, num_tokens, max_query_len,
                          max_seq_len, num_q_heads, num_kv_heads, head_dim, block_size,
                          block_table_stride, num_blocks, scale, num_splits, out, lse, workspace,
                          workspace_bytes, dtype, false, stream);
  }
  if (!key || !value || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(key) || !aligned16(value)) return PA_ERR_INVALID;
  return attention_impl(query, key_cache, value_cache, nullptr, nullptr, query_start_loc,
                        seq_lens, block_tables, num_seqs, num_tokens, max_query_len, max_seq_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, block_table_stride,
                        num_blocks, scale, num_splits, out, lse, workspace, workspace_bytes,
                        dtype, false, stream, nullptr, 0, nullptr, 0, key, value, slot_mapping);
}

}  // namespace pa

extern "C" {

pa_status pa_attention_fwd(const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* query_start_loc, const int32_t* seq_lens,
                           const int32_t* block_tables, int32_t num_seqs, int32_t num_tokens,
                           int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t block_table_stride, int64_t num_blocks, float scale,
                           int32_t num_splits, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, pa_dtype dtype, void* stream) {
  return attention_impl(query, key_cache, value_cache, nullptr, nullptr, query_start_loc,
                        seq_lens, block_tables, num_seqs, num_tokens, max_query_len, max_seq_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, block_table_stride,
                        num_blocks, scale, num_splits, out, lse, workspace, workspace_bytes,
                        dtype, false, stream);
}

size_t pa_cascade_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t num_splits,
                                 int32_t num_sharers, int32_t max_query_len,
                                 int32_t num_prefix_blocks) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || num_splits < 1 || num_sharers < 0 || max_query_len < 0 ||
      num_prefix_blocks < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  const int32_t group = num_q_heads / num_kv_heads;
  const int64_t rows = num_prefix_blocks > 0 ? (int64_t)num_sharers *
                                                   std::min<int32_t>(max_query_len,
                                                                     decode_max_q(group))
                                             : 0;
  int32_t ks = 1, kc = 0;
  if (rows > 0)
    cascade_key_split(num_prefix_blocks, rows, group, num_kv_heads, device_cu_count(), &ks, &kc);
  return ws_layout(num_seqs, num_tokens, num_q_heads, head_dim, num_splits, rows, ks).total;
}

pa_status pa_attention_fwd_cascade(const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* query_start_loc,
                                   const int32_t* seq_lens, const int32_t* block_tables,
                                   int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                                   int32_t max_seq_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t block_table_stride, int64_t num_blocks, float scale,
                                   int32_t num_splits, const int32_t* sharers,
                                   int32_t num_sharers, const int32_t* prefix_blocks,
                                   int32_t num_prefix_blocks, void* out, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (num_sharers < 0 || num_prefix_blocks < 0) return PA_ERR_INVALID;
  if (num_sharers > 0 && num_prefix_blocks > 0 && (!sharers || !prefix_blocks))
    return PA_ERR_NULL;
  return attention_impl(query, key_cache, value_cache, nullptr, nullptr, query_start_loc,
                        seq_lens, block_tables, num_seqs, num_tokens, max_query_len, max_seq_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, block_table_stride,
                        num_blocks, scale, num_splits, out, lse, workspace, workspace_bytes,
                        PA_BF16, false, stream, sharers, num_sharers, prefix_blocks,
                        num_prefix_blocks);
}

pa_status pa_decode_step_cascade(const void* key, const void* value, void* key_cache,
                                 void* value_cache, const int64_t* slot_mapping,
                                 const void* query, const int32_t* query_start_loc,
                                 const int32_t* seq_lens, const int32_t* block_tables,
                                 int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                                 int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t block_table_stride,
                                 int64_t num_blocks, float scale, int32_t num_splits,
                                 const int32_t* sharers, int32_t num_sharers,
                                 const int32_t* prefix_blocks, int32_t num_prefix_blocks,
                                 void* out, float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (num_sharers < 0 || num_prefix_blocks < 0) return PA_ERR_INVALID;
  const bool cascade = num_sharers > 0 && num_prefix_blocks > 0;
  if (cascade && (!sharers || !prefix_blocks)) return PA_ERR_NULL;
  if (!cascade || num_seqs == 0)  // no shared prefix: the plain one-call step
    return pa::decode_step_impl(key, value, key_cache, value_cache, slot_mapping, query,
                                query_start_loc, seq_lens, block_tables, num_seqs, num_tokens,
                                max_query_len, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                                block_size, block_table_stride, num_blocks, scale, num_splits,
                                out, lse, workspace, workspace_bytes, PA_BF16, stream);
  if (num_tokens > 0 && (!key || !value || !slot_mapping)) return PA_ERR_NULL;
  if (!aligned16(key) || !aligned16(value)) return PA_ERR_INVALID;
  return attention_impl(query, key_cache, value_cache, nullptr, nullptr, query_start_loc,
                        seq_lens, block_tables, num_seqs, num_tokens, max_query_len, max_seq_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, block_table_stride,
                        num_blocks, scale, num_splits, out, lse, workspace, workspace_bytes,
                        PA_BF16, false, stream, sharers, num_sharers, prefix_blocks,
                        num_prefix_blocks, key, value, slot_mapping);
}

pa_status pa_decode_step(const void* key, const void* value, void* key_cache, void* value_cache,
                         const int64_t* slot_mapping, const void* query,
                         const int32_t* query_start_loc, const int32_t* seq_lens,
                         const int32_t* block_tables, int32_t num_seqs, int32_t num_tokens,
                         int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t block_table_stride, int64_t num_blocks, float scale,
                         int32_t num_splits, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, pa_dtype dtype, void* stream) {
  return pa::decode_step_impl(key, value, key_cache, value_cache, slot_mapping, query,
                              query_start_loc, seq_lens, block_tables, num_seqs, num_tokens,
                              max_query_len, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                              block_size, block_table_stride, num_blocks, scale, num_splits, out,
                              lse, workspace, workspace_bytes, dtype, stream);
}

pa_status pa_decode_step_fp8(const void* key, const void* value, void* key_cache,
                             void* value_cache, const int64_t* slot_mapping,
                             const float* k_scale, const float* v_scale, const void* query,
                             const int32_t* query_start_loc, const int32_t* seq_lens,
                             const int32_t* block_tables, int32_t num_seqs, int32_t num_tokens,
                             int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t block_table_stride, int64_t num_blocks, float scale,
                             int32_t num_splits, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, pa_dtype dtype, void* stream) {
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return PA_ERR_INVALID;
  const int32_t group = num_q_heads / num_kv_heads;
  // one call: the decode kernel writes the decode rows' tokens, and in a
  // step with prefill rows a write over the matrix-core kernel's work list
  // writes theirs ahead of it
  const bool fuse = dtype == PA_BF16 && is_pow2_group(group) && num_seqs > 0 &&
                    num_tokens > 0 && max_query_len >= 1;
  if (!fuse) {
    pa_status st = pa_kv_write_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale,
                                   v_scale, num_tokens, num_kv_heads, head_dim, block_size,
                                   num_blocks, dtype, stream);
    if (st != PA_OK) return st;
    return pa_attention_fwd_fp8(query, key_cache, value_cache, k_scale, v_scale,
                                query_start_loc, seq_lens, block_tables, num_seqs, num_tokens,
                                max_query_len, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                                block_size, block_table_stride, num_blocks, scale, num_splits,
                                out, lse, workspace, workspace_bytes, stream);
  }
  if (!key || !value || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(key) || !aligned16(value)) return PA_ERR_INVALID;
  return attention_impl(query, key_cache, value_cache, k_scale, v_scale, query_start_loc,
                        seq_lens, block_tables, num_seqs, num_tokens, max_query_len, max_seq_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, block_table_stride,
                        num_blocks, scale, num_splits, out, lse, workspace, workspace_bytes,
                        PA_BF16, true, stream, nullptr, 0, nullptr, 0, key, value, slot_mapping);
}

pa_status pa_attention_fwd_fp8(const void* query, const void* key_cache,
                               const void* value_cache, const float* k_scale,
                               const float* v_scale, const int32_t* query_start_loc,
                               const int32_t* seq_lens, const int32_t* block_tables,
                               int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                               int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t block_table_stride,
                               int64_t num_blocks, float scale, int32_t num_splits, void* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return attention_impl(query, key_cache, value_cache, k_scale, v_scale, query_start_loc,
                        seq_lens, block_tables, num_seqs, num_tokens, max_query_len, max_seq_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, block_table_stride,
                        num_blocks, scale, num_splits, out, lse, workspace, workspace_bytes,
                        PA_BF16, true, stream);
}

pa_status pa_rope_kv_write(void* query, const void* key, const void* value, void* key_cache,
                           void* value_cache, const int64_t* slot_mapping,
                           const int64_t* positions, const float* cos_sin, int32_t max_position,
                           int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           pa_dtype dtype, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_q_heads <= 0 || num_blocks <= 0 ||
      max_position < 0)
    return PA_ERR_INVALID;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID;
  if (block_size != PA_BLOCK_SIZE) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!query || !key || !value || !key_cache || !value_cache || !slot_mapping || !positions ||
      !cos_sin)
    return PA_ERR_NULL;
  if (!aligned16(query) || !aligned16(key) || !aligned16(value) || !aligned16(key_cache) ||
      !aligned16(value_cache) || !aligned16(cos_sin))
    return PA_ERR_INVALID;
  const int32_t esize = dtype == PA_BF16 ? 2 : 4;
  hipError_t e = launch_rope_kv_write(query, key, value, key_cache, value_cache, slot_mapping,
                                      positions, cos_sin, max_position, num_tokens, num_q_heads,
                                      num_kv_heads, head_dim, esize, num_blocks,
                                      (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_kv_write_fp8(const void* key, const void* value, void* key_cache, void* value_cache,
                          const int64_t* slot_mapping, const float* k_scale, const float* v_scale,
                          int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int64_t num_blocks, pa_dtype dtype, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID;
  if (block_size != PA_BLOCK_SIZE) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping || !k_scale || !v_scale)
    return PA_ERR_NULL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return PA_ERR_INVALID;
  const int32_t esize = dtype == PA_BF16 ? 2 : 4;
  hipError_t e = launch_kv_write_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale,
                                     v_scale, num_tokens, num_kv_heads, head_dim, esize,
                                     num_blocks, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
