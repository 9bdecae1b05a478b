// pa_decode_step_noalloc: pa_decode_step for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The step's workspace -- split-merge
// arrival counters, the matrix-core kernel's work list, the decode order and
// the split partials -- lives in one file-scope device array instead of a
// caller-provided buffer.  Nothing here allocates: the array is part of the
// library's code object, and each GPU the library runs on holds its own copy
// until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

// The workspace of every no-alloc call on a device.  In host code this name
// is only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, per device, and only that address is ever used.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct ScratchTable {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
};

ScratchTable& table() {
  static ScratchTable* t = new ScratchTable();  // never destroyed: safe at exit
  return *t;
}

// Device address of this device's copy of `scratch`, looked up once per
// device with that device current.  The first call on a device also clears
// the array on `stream` (ahead of the step's kernels), so the arrival
// counters start at zero even if the loader had not zero-filled it; every
// completed call leaves them at zero again.
pa_status scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  ScratchTable& t = table();
  std::lock_guard<std::mutex> lk(t.mu);
  if (t.ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_HIP;
    if (pa::launch_zero(p, PA_NOALLOC_SCRATCH_BYTES, stream) != hipSuccess) return PA_ERR_HIP;
    t.ptr[dev] = p;
  }
  *out = t.ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode_step_noalloc(
    const void* key, const void* value, void* key_cache, void* value_cache,
    const int64_t* slot_mapping, const void* query, const int32_t* query_start_loc,
    const int32_t* seq_lens, const int32_t* block_tables, int32_t num_seqs, int32_t num_tokens,
    int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t block_table_stride, int64_t num_blocks,
    float scale, int32_t num_splits, void* out, float* lse, pa_dtype dtype, void* stream) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || num_splits < 0 || num_splits > PA_MAX_SPLITS)
    return PA_ERR_INVALID;
  // the workspace this step needs, at the split count pa_decode_step will use
  const int32_t splits =
      num_splits > 0 ? num_splits
                     : pa_choose_num_splits(num_seqs, max_query_len, max_seq_len, num_q_heads,
                                            num_kv_heads, 0);
  const size_t need =
      pa_attention_workspace_size(num_seqs, num_tokens, num_q_heads, head_dim, splits);
  if (need == 0 || need > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  const pa_status st = scratch_of_current_device((hipStream_t)stream, &ws);
  if (st != PA_OK) return st;
  return pa::decode_step_impl(key, value, key_cache, value_cache, slot_mapping, query,
                              query_start_loc, seq_lens, block_tables, num_seqs, num_tokens,
                              max_query_len, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                              block_size, block_table_stride, num_blocks, scale, splits, out, lse,
                              ws, (size_t)PA_NOALLOC_SCRATCH_BYTES, dtype, stream);
}
