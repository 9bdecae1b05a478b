/*
 * pa.h -- C ABI of the paged-attention library for one flat engine step
 * (MI355X / gfx950).
 *
 * What a step is ("Model execution", section "Flattening a step"): all tokens
 * scheduled in the step are concatenated into one flat batch.  Attention gets
 * per-request offsets (query_start_loc), total context lengths (seq_lens) and
 * block tables; the KV write gets a slot mapping, slot = block_id * block_size
 * + offset.  The arithmetic is exact attention computed FlashAttention-style
 * ("Inside the engine: kernels, CUDA graphs and the life of a request",
 * sections "Never materialise the T x T matrix", "Prefill has a full grid;
 * decode at batch 1 has almost none" and "Attention over a block table, not
 * a contiguous tensor").
 *
 * Conventions common to every entry point
 * ---------------------------------------
 * - Every tensor argument is a DEVICE pointer owned by the caller.  The
 *   library allocates and frees no device memory and keeps no per-call state.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream) and never synchronises or reads device memory on the host: grid
 *   sizes come only from the host scalars passed in.
 * - Scalars and pointers are validated on the host before anything is
 *   enqueued; a non-OK status means nothing was launched.  A launch failure
 *   is reported as PA_ERR_HIP.  No call aborts or throws.
 * - Data-dependent faults are NOT checked on the fast path (that would need a
 *   device-to-host read): block ids outside [0, num_blocks), duplicate slots,
 *   seq_len < q_len, a non-monotone query_start_loc, or q_len / seq_len above
 *   the max_query_len / max_seq_len passed in give undefined results.
 * - Identical inputs and num_splits give bitwise-identical outputs (no atomics
 *   in any reduction; reduction order depends only on logical positions).
 *
 * Layouts (row-major, innermost last; d = head_dim, bs = block_size = 16):
 *   query        [num_tokens][num_q_heads][d]
 *   key, value   [num_tokens][num_kv_heads][d]           (the step's new tokens)
 *   key_cache    [num_blocks][num_kv_heads][bs][d]        (token-major block)
 *   value_cache  [num_blocks][num_kv_heads][d][bs]        (dim-major block)
 *   out          [num_tokens][num_q_heads][d]
 *   lse          [num_tokens][num_q_heads]   float32, natural log
 *   query_start_loc [num_seqs + 1] int32, seq_lens [num_seqs] int32,
 *   block_tables [num_seqs][block_table_stride] int32,
 *   slot_mapping [num_tokens] int64.
 * The value block is stored dim-major so that the P*V product reads 8
 * consecutive keys of one dimension as a single matrix-core operand.
 *
 * Grouped-query attention: query head h reads KV head h / (num_q_heads /
 * num_kv_heads).  Causality with prior context: row i of request b sits at
 * position p = seq_lens[b] - q_len_b + i and attends to positions 0..p.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  PA_ERR_INVALID = 2,     /* a scalar is out of range or inconsistent          */
  PA_ERR_UNSUPPORTED = 3, /* valid, but outside what the kernels implement      */
  PA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required        */
  PA_ERR_HIP = 5          /* the HIP runtime reported an error on launch       */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,             /* float32 activations and cache                     */
  PA_BF16 = 1             /* bfloat16 activations and cache (fp32 accumulate)  */
} pa_dtype;

#define PA_BLOCK_SIZE 16
#define PA_MAX_SPLITS 256

/*
 * pa_kv_write -- scatter the step's new K and V into the paged cache.
 * ("Model execution", section "Flattening a step": the KV write uses the
 * slot mapping, slot = block_id * block_size + offset.)
 *
 * For every t < num_tokens with s = slot_mapping[t] >= 0, and every KV head h:
 *   key_cache  [s / bs][h][s % bs][:] = key  [t][h][:]
 *   value_cache[s / bs][h][:][s % bs] = value[t][h][:]
 * A negative slot marks a padded token: nothing is written for it; a slot at
 * or past num_blocks * bs is dropped the same way (the pool is never written
 * out of bounds).  The copy is bit-exact (cache dtype = input dtype, nothing
 * converts) and no other cache entry changes.  Slots must be distinct
 * (unchecked; with duplicates the surviving row is unspecified).
 *
 * Supported: head_dim in {64, 128}, block_size == 16, num_kv_heads >= 1.
 * num_tokens == 0 is a no-op (pointers may then be NULL).
 */
pa_status pa_kv_write(const void* key, const void* value,
                      void* key_cache, void* value_cache,
                      const int64_t* slot_mapping,
                      int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int64_t num_blocks,
                      pa_dtype dtype, void* stream);

/*
 * pa_attention_fwd -- causal attention of every scheduled row of the flat
 * batch through the block tables ("Inside the engine ...", sections "Never
 * materialise the T x T matrix" and "Attention over a block table, not a
 * contiguous tensor"; metadata as in "Model execution", "Flattening a step").
 *
 * For request b, q_len_b = query_start_loc[b+1] - query_start_loc[b] rows at
 * flat indices query_start_loc[b] ..; row i has position
 * p = seq_lens[b] - q_len_b + i and, for every query head h,
 *   out[t][h] = softmax(scale * q[t][h] . K[0..p]) V[0..p]
 *   lse[t][h] = ln sum_j exp(scale * q[t][h] . K[j])          (if lse != NULL)
 * where K[j], V[j] are read from block block_tables[b][j / 16], offset j % 16,
 * KV head h / (num_q_heads / num_kv_heads).  Rows at or after
 * query_start_loc[num_seqs] are not written.  The cache must already hold the
 * step's new tokens (call pa_kv_write first on the same stream).
 *
 * Execution: rows of requests with few new tokens (decode) run a
 * bandwidth-bound kernel; with num_splits > 1 their key range is cut into
 * num_splits block ranges whose partial results are merged by a second
 * reduction (the split-KV method of "Prefill has a full grid; decode at batch
 * 1 has almost none"): in bf16 mode the last split of each request and KV
 * head to finish performs it inside the same launch, in fp32 mode a separate
 * combine kernel does.  Rows of requests with many new tokens run the tiled
 * matrix-core kernel.  In bf16 mode, when the host scalars show that the
 * step also has decode rows (num_seqs > num_tokens / (16 / group + 1)), the
 * two run as one persistent launch whose work-groups take prefill and
 * decode work units from two counters in the workspace, so the MFMA-bound
 * and the HBM-bound rows overlap.  num_splits: 0 = pa_choose_num_splits() for these
 * scalars, 1 = no split, 2..PA_MAX_SPLITS = forced.  The result does not
 * depend on num_splits beyond rounding.
 *
 * max_query_len / max_seq_len: host-known upper bounds of q_len_b / seq_lens
 * (they size the grids).  block_table_stride >= ceil(max_seq_len / 16); table
 * entries past a request's last block are never read.
 *
 * scale must be positive and finite (e.g. 1 / sqrt(head_dim)).
 *
 * workspace: device scratch of at least pa_attention_workspace_size(num_seqs,
 * num_tokens, num_q_heads, head_dim, S) bytes, S the split count in use
 * (resolve num_splits = 0 with pa_choose_num_splits first), 16-byte aligned.
 * Its first num_seqs * num_q_heads int32 are arrival counters of the split
 * merge: they must be zero before the first call (pa_attention_workspace_init
 * or any zero-filled allocation) and every call leaves them zero.  The rest
 * of the workspace needs no initialisation.  Calls that share a workspace
 * must not overlap in time (use one stream, or one workspace per stream).
 *
 * Supported: dtype PA_BF16 or PA_F32, head_dim in {64, 128}, block_size 16,
 * num_q_heads % num_kv_heads == 0 with group size in {1, 2, 4, 8, 16}.
 */
pa_status pa_attention_fwd(const void* query,
                           const void* key_cache, const void* value_cache,
                           const int32_t* query_start_loc,
                           const int32_t* seq_lens,
                           const int32_t* block_tables,
                           int32_t num_seqs, int32_t num_tokens,
                           int32_t max_query_len, int32_t max_seq_len,
                           int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size,
                           int32_t block_table_stride, int64_t num_blocks,
                           float scale, int32_t num_splits,
                           void* out, float* lse,
                           void* workspace, size_t workspace_bytes,
                           pa_dtype dtype, void* stream);

/*
 * pa_rope_kv_write -- rotary position embedding of the step's queries and new
 * keys fused with the KV write (positions: "Model execution", section
 * "Flattening a step", kept "for rotary embeddings" in "Inside the engine";
 * the pages do not write the rotation out).  For every t < num_tokens whose
 * p = positions[t] lies in [0, max_position), every head row x of length d
 * (query[t][hq] for all query heads, key[t][hkv]) is rotated pairwise,
 *   x'[i]       = x[i] c_i - x[i + d/2] s_i
 *   x'[i + d/2] = x[i + d/2] c_i + x[i] s_i,     i < d/2,
 * with c_i = cos_sin[p][i], s_i = cos_sin[p][d/2 + i] (fp32 table
 * [max_position][head_dim], 16-byte aligned), computed in fp32 and rounded
 * once to dtype.  query is rotated in place; the rotated key and the
 * unchanged value are written at slot_mapping[t] exactly as pa_kv_write
 * (slot < 0 or past the pool: nothing written).  Tokens whose position is
 * outside the table are left alone (query unchanged, nothing written).
 * Supported as pa_kv_write; num_q_heads a multiple of num_kv_heads.
 */
pa_status pa_rope_kv_write(void* query, const void* key, const void* value,
                           void* key_cache, void* value_cache,
                           const int64_t* slot_mapping, const int64_t* positions,
                           const float* cos_sin, int32_t max_position,
                           int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           pa_dtype dtype, void* stream);

/*
 * pa_decode_step -- pa_kv_write followed by pa_attention_fwd, as one call
 * (arguments as those two; key/value/slot_mapping for the write, the rest
 * for attention).  When every request has at most 16 / group new tokens
 * (max_query_len) and dtype is bf16, the decode kernel performs the write
 * itself, in one launch: the work-group whose block range holds a request's
 * new token writes that token's K/V for its KV head before it reads any
 * block, and one work-group writes tokens after the last request's rows.
 * This relies on the definition of the flat batch ("Model execution",
 * "Flattening a step"): the slot of position p of request b is
 * block_tables[b][p / 16] * 16 + p % 16, so no other work-group reads a
 * new token's entry.  A bf16 step that also has prefill rows (more than
 * 16 / group new tokens) writes their tokens with a kernel over the
 * matrix-core kernel's work list, ahead of the attention launch, while the
 * decode work writes the decode rows' tokens and those after the last
 * request.  fp32 steps run the two calls in order.
 * Results (pool bytes, out, lse) are those of the two calls.
 */
pa_status pa_decode_step(const void* key, const void* value, void* key_cache, void* value_cache,
                         const int64_t* slot_mapping, const void* query,
                         const int32_t* query_start_loc, const int32_t* seq_lens,
                         const int32_t* block_tables, int32_t num_seqs, int32_t num_tokens,
                         int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t block_table_stride, int64_t num_blocks, float scale,
                         int32_t num_splits, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, pa_dtype dtype, void* stream);

/*
 * pa_decode_step_noalloc -- pa_decode_step for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of pa_decode_step without the workspace: the step's workspace is a
 * library-owned device array of PA_NOALLOC_SCRATCH_BYTES per GPU (each GPU
 * the library runs on keeps its own copy until the process ends).  A step
 * whose workspace (pa_attention_workspace_size at the split count used: the
 * heuristic's when num_splits is 0) exceeds that size returns
 * PA_ERR_WORKSPACE before anything is enqueued.  The call allocates and
 * frees nothing; its first call on a device looks the array up and clears
 * it on `stream`.  Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (different streams, or different host threads,
 * without ordering between them) race and give undefined results; calls
 * ordered on one stream are safe.
 */
#define PA_NOALLOC_SCRATCH_BYTES (16u << 20)
pa_status pa_decode_step_noalloc(const void* key, const void* value, void* key_cache,
                                 void* value_cache, const int64_t* slot_mapping,
                                 const void* query, const int32_t* query_start_loc,
                                 const int32_t* seq_lens, const int32_t* block_tables,
                                 int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                                 int32_t max_seq_len, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t block_table_stride, int64_t num_blocks, float scale,
                                 int32_t num_splits, void* out, float* lse, pa_dtype dtype,
                                 void* stream);

/*
 * pa_attention_fwd_cascade -- pa_attention_fwd (bf16) with a shared prefix
 * read once.  Block tables may point several requests at the same physical
 * blocks ("Model execution", "Flattening a step"; prefix caching in "Anatomy
 * of a serving engine"); here `sharers` [num_sharers] are requests whose
 * tables start with the num_prefix_blocks blocks `prefix_blocks` (device
 * int32, caller's contract, unchecked).  The decode rows of the sharers are
 * gathered and attend to the shared blocks in one matrix-core pass (each
 * prefix tile staged once per 64-token tile of gathered rows, not once per
 * request) as a partial (o, lse); the decode kernel then reads only each
 * sharer's own later blocks and merges that partial with its splits.  The
 * result is the attention of pa_attention_fwd (up to rounding): causality is
 * kept per row, so a sharer whose context is shorter than the prefix is still
 * exact.  The prefix keys are cut into ranges (one partial each) so that the
 * stage fills the device even for few sharers.  Sharers with more new tokens
 * than the decode kernel packs, or none, are computed as usual.  The stage
 * runs first; the rest of the step (the decode rows, and any prefill rows,
 * in one persistent launch under pa_attention_fwd's rule) follows.  The
 * decode rows read the remaining blocks as unshared (pa_set_unshared_blocks),
 * whatever the process-wide setting.  Workspace: pa_cascade_workspace_size (zeroed once
 * like pa_attention_fwd's).  Every other argument and error as
 * pa_attention_fwd with dtype PA_BF16.
 */
pa_status pa_attention_fwd_cascade(const void* query, const void* key_cache,
                                   const void* value_cache,
                                   const int32_t* query_start_loc, const int32_t* seq_lens,
                                   const int32_t* block_tables,
                                   int32_t num_seqs, int32_t num_tokens,
                                   int32_t max_query_len, int32_t max_seq_len,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t block_table_stride,
                                   int64_t num_blocks, float scale, int32_t num_splits,
                                   const int32_t* sharers, int32_t num_sharers,
                                   const int32_t* prefix_blocks, int32_t num_prefix_blocks,
                                   void* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* pa_cascade_workspace_size -- bytes of workspace for pa_attention_fwd_cascade
 * (num_splits resolved, >= 1; on the device the call will run on). */
size_t pa_cascade_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t num_splits,
                                 int32_t num_sharers, int32_t max_query_len,
                                 int32_t num_prefix_blocks);

/*
 * pa_decode_step_cascade -- pa_kv_write followed by pa_attention_fwd_cascade,
 * as one call (bf16; arguments as those two, workspace sized by
 * pa_cascade_workspace_size).  The decode step of requests that share a
 * cached prefix ("Anatomy of a serving engine", prefix caching; "Model
 * execution", "Flattening a step": tables may point several requests at the
 * same blocks, and every new token goes to its slot before attention).  The
 * write of all num_tokens tokens (slot < 0 or past the pool: nothing
 * written) shares its launch with the stage's setup, which reads only
 * metadata, so the setup costs no launch of its own; the prefix stage and
 * the rest of the step follow as in pa_attention_fwd_cascade and read the
 * cache after the write.  Without sharers or prefix blocks (or requests) it
 * is pa_decode_step with dtype PA_BF16.  Results (pool bytes, out, lse) are
 * those of the two calls, bit for bit.  Errors as those two calls; nothing
 * is enqueued when the arguments are rejected.
 */
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
                                 void* stream);

/*
 * FP8 KV cache (E4M3).  The pages name an 8-bit cache as the way to halve the
 * bytes every decode step reads ("Anatomy of a serving engine", KV-cache
 * capacity; "Model execution", section "Attention backends") without fixing
 * the format.  Format here: OCP E4M3 -- sign, 4-bit exponent (bias 7), 3-bit
 * mantissa, subnormals m/8 * 2^-6, no infinities, 0x7F / 0xFF NaN, largest
 * finite magnitude 448.  Same block layouts as the 16-bit cache, one byte per
 * element: K [num_blocks][num_kv_heads][16][head_dim], V
 * [num_blocks][num_kv_heads][head_dim][16].  Scales: k_scale[num_kv_heads],
 * v_scale[num_kv_heads], device fp32, positive and finite (unchecked): a
 * cached value of KV head h stands for code * scale[h].
 */

/*
 * pa_kv_write_fp8 -- quantising scatter of the step's new K and V into an
 * E4M3 cache.  For every t < num_tokens with 0 <= s = slot_mapping[t] <
 * num_blocks * 16 and every KV head h:
 *   key_cache[s / 16][h][s % 16][j] = e4m3(clamp(key[t][h][j] / k_scale[h]))
 * (and V dim-major), where the division is IEEE fp32 (key widened exactly
 * from bf16 or fp32, `dtype`), clamp is to [-448, 448] and e4m3() rounds to
 * the nearest code, ties to the even mantissa; +-inf clamp to +-448.  Every
 * NaN input, whatever its sign bit, gives the one code 0x7F.  Negative or
 * out-of-pool slots write nothing.  Errors as pa_kv_write.
 */
pa_status pa_kv_write_fp8(const void* key, const void* value,
                          void* key_cache, void* value_cache,
                          const int64_t* slot_mapping,
                          const float* k_scale, const float* v_scale,
                          int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int64_t num_blocks,
                          pa_dtype dtype, void* stream);

/*
 * pa_attention_fwd_fp8 -- pa_attention_fwd over an E4M3 cache: every
 * argument as there (query and out bf16, dtype implied), plus the cache's
 * per-KV-head scales.  Computes exactly the attention of pa_attention_fwd
 * with K[j] = code * k_scale[h] and V[j] = code * v_scale[h]; the codes are
 * widened to bf16 exactly, k_scale folds into the score scale and v_scale
 * multiplies the normalised output, so no extra rounding enters.  Same
 * workspace (pa_attention_workspace_size), same split behaviour.
 */
pa_status pa_attention_fwd_fp8(const void* query, const void* key_cache,
                               const void* value_cache,
                               const float* k_scale, const float* v_scale,
                               const int32_t* query_start_loc, const int32_t* seq_lens,
                               const int32_t* block_tables,
                               int32_t num_seqs, int32_t num_tokens,
                               int32_t max_query_len, int32_t max_seq_len,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t block_table_stride,
                               int64_t num_blocks, float scale, int32_t num_splits,
                               void* out, float* lse, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * pa_decode_step_fp8 -- pa_kv_write_fp8 followed by pa_attention_fwd_fp8 as
 * one call, fused as pa_decode_step is (bf16 key / value / query): the
 * decode kernel quantises its rows' new tokens, and in a step with prefill
 * rows a write over the matrix-core kernel's work list quantises theirs,
 * each exactly as pa_kv_write_fp8 does.  dtype: of key / value (the query is
 * bf16); PA_F32 runs the two calls.
 */
pa_status pa_decode_step_fp8(const void* key, const void* value, void* key_cache,
                             void* value_cache, const int64_t* slot_mapping,
                             const float* k_scale, const float* v_scale, const void* query,
                             const int32_t* query_start_loc, const int32_t* seq_lens,
                             const int32_t* block_tables, int32_t num_seqs, int32_t num_tokens,
                             int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t block_table_stride, int64_t num_blocks, float scale,
                             int32_t num_splits, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, pa_dtype dtype, void* stream);

/*
 * pa_attention_workspace_init -- zero `workspace_bytes` of a workspace on
 * `stream` with a kernel (no memset node, so it may be captured in a HIP
 * graph).  Needed once for a new workspace whose memory is not already zero.
 */
pa_status pa_attention_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_split_combine -- merge split-KV partials ("Prefill has a full grid;
 * decode at batch 1 has almost none": the partials are combined in a second
 * reduction kernel).
 *
 * partial_out [num_splits][num_tokens][num_q_heads][head_dim] float32 holds
 * each split's normalised output o_s, partial_lse [num_splits][num_tokens]
 * [num_q_heads] float32 its natural-log sum-exp (-inf for a split that saw no
 * key; its o_s is ignored).  With M = max_s lse_s:
 *   lse = M + ln sum_s exp(lse_s - M),   out = sum_s exp(lse_s - lse) o_s
 * written as `dtype` (bf16 rounds to nearest even once).  An entry whose
 * splits are all -inf gets out = NaN and lse = -inf.  lse may be NULL.
 * Supported: 1 <= num_splits <= PA_MAX_SPLITS, head_dim in {64, 128}.
 */
pa_status pa_split_combine(const float* partial_out, const float* partial_lse,
                           int32_t num_splits, int32_t num_tokens,
                           int32_t num_q_heads, int32_t head_dim,
                           void* out, float* lse, pa_dtype dtype, void* stream);

/*
 * pa_attention_workspace_size -- bytes of workspace pa_attention_fwd needs for
 * this batch shape at `num_splits` splits (num_splits >= 1; the split
 * partials, plus a small work list for the matrix-core kernel).
 */
size_t pa_attention_workspace_size(int32_t num_seqs, int32_t num_tokens,
                                   int32_t num_q_heads, int32_t head_dim,
                                   int32_t num_splits);

/*
 * pa_choose_num_splits -- the split / no-split crossover ("Prefill has a full
 * grid; decode at batch 1 has almost none": the split pays at low batch and
 * is disabled once the query rows fill the grid).  Returns 1 when any request
 * may have more new tokens than the decode kernel packs (max_query_len above
 * 16 / group size) or when num_seqs * num_kv_heads work units already fill
 * the device; otherwise enough splits to give every compute unit work,
 * bounded by 64 (the in-launch merge of more partials costs more than the
 * extra work-groups gain), by PA_MAX_SPLITS and by the number of 16-token
 * blocks (at least 8 per split).  num_cus <= 0
 * means "ask the current device".  Performance only: results do not depend on
 * it.
 */
int32_t pa_choose_num_splits(int32_t num_seqs, int32_t max_query_len,
                             int32_t max_seq_len, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t num_cus);

/*
 * pa_capture_size -- the padded size a step of num_tokens tokens is replayed
 * at from a captured HIP graph ("Model execution", section "Code": graphs are
 * captured for a ladder of batch sizes 1, 2, 4, then every multiple of 8
 * below 256, then every multiple of 16 up to the largest captured size, and a
 * step runs the graph of the smallest size that holds it, the extra rows
 * padded; larger steps run without a graph).  max_size is the largest
 * captured size (512 on the page; it must be a ladder size >= 256 or one of
 * the sizes below 256).  Returns the ladder size, or -1 when num_tokens < 1 or
 * num_tokens > max_size.  Host-only.
 *
 * Padding that keeps a captured step exact: padded tokens get slot -1 (the
 * KV write skips them) and belong to no request's rows; padded requests have
 * q_len 0 and seq_len 0 (no rows, no keys).  Grids are then sized from the
 * padded shapes and host bounds fixed at capture (max_query_len, and
 * max_seq_len = the block-table capacity), so one graph serves every step of
 * that size.
 */
int32_t pa_capture_size(int32_t num_tokens, int32_t max_size);

/*
 * pa_set_unshared_blocks -- cache-read policy of the decode rows for later
 * calls in this process.  Block tables may point several requests of a step
 * at the same physical blocks (prefix caching: "Anatomy of a serving
 * engine"; "Model execution", "Flattening a step").  A request whose blocks
 * no other request reads has its V read with the non-temporal policy, which
 * streams it without keeping it in L2/MALL (measured: 256 unshared decodes
 * ~8 % faster with a bf16 cache, ~9 % with E4M3); blocks that several
 * requests read stay cached, since the non-temporal policy would re-read them
 * from HBM (256 decodes that all re-read one 16K-token prefix: ~25 % slower).
 * This applies to the decode rows of pa_attention_fwd(_fp8) /
 * pa_decode_step(_fp8) when the step has more decode work units than two per
 * compute unit or also has prefill rows.  mode:
 *    0 (default) automatic: a request counts as unshared when its first
 *      block is no other request's first block (sharing goes through common
 *      prefixes); tested while the decode requests are ranked (steps of 64
 *      to 8192 requests), otherwise every request counts as shared;
 *    1 every request counts as unshared (the caller states that no block is
 *      read by two requests of a step);
 *   -1 every request counts as shared.
 * Results are the same under every mode, bit for bit.
 * pa_attention_fwd_cascade always reads the unshared way (its decode rows
 * skip the shared prefix).  Process-wide, takes effect for launches issued
 * after the call (a captured HIP graph keeps the loads it was captured
 * with).  Returns the previous mode.
 */
int32_t pa_set_unshared_blocks(int32_t mode);

/* pa_status_string -- static text for a status code (never NULL). */
const char* pa_status_string(pa_status status);

/* pa_version -- library version, major * 10000 + minor * 100 + patch. */
int32_t pa_version(void);

/*
 * Kernel tracing (measurement aid).  pa_trace_begin(capacity) makes every
 * later launch inside this library record a pair of HIP events around itself
 * on its stream, for up to `capacity` launches; it creates the events (host
 * call, may allocate).  pa_trace_end() stops recording.  After the caller has
 * synchronised the streams, pa_trace_read() fills kernel_ids[i] and
 * milliseconds[i] for the recorded launches (at most `capacity` entries) and
 * returns their number (-1 on error).  pa_kernel_name() names a kernel id.
 * Tracing is process-wide and not thread-safe against concurrent launches.
 */
pa_status   pa_trace_begin(int32_t capacity);
pa_status   pa_trace_end(void);
int32_t     pa_trace_read(int32_t* kernel_ids, float* milliseconds, int32_t capacity);
const char* pa_kernel_name(int32_t kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
