// The KV write of up to 16 consecutive flat tokens of one KV head ("Model
// execution", section "Flattening a step": each new token's K and V go to
// slot block_id * block_size + offset), shared by the write kernels and by
// the first launch of the one-call shared-prefix step.
#pragma once

#include "device_common.h"
#include "pa_internal.h"

namespace pa {

constexpr int kWriteTokens = 16;

// LDS staging of one write_tokens call: the tokens' V rows (padded by 16
// bytes) and their slots.
template <typename E>
struct WriteStage {
  E vrow[kWriteTokens][128 + 16 / sizeof(E)];
  int64_t slot[kWriteTokens];
};

// Writes the `ntok` (<= 16) tokens t0 .. t0 + ntok - 1 of KV head h with 256
// threads; `tid` in [0, 256) is the thread's index among them.  Every thread
// of the work-group calls it the same number of times (it holds a work-group
// barrier), with ntok = 0 where a group of 256 threads has nothing to write.
// The K row of a token is a contiguous run of the token-major K block, copied
// in 16-byte pieces.  The V block is dim-major, so the V rows are staged in
// LDS first and then written column by column: lanes that differ in the token
// index write neighbouring offsets of one dimension, which coalesce when the
// tokens fill consecutive slots of a block.  A slot < 0 or past the pool
// (num_slots) is skipped.
template <typename E>
__device__ __forceinline__ void write_tokens(const E* __restrict__ key,
                                             const E* __restrict__ value, E* __restrict__ kc,
                                             E* __restrict__ vc,
                                             const int64_t* __restrict__ slots, int t0,
                                             int ntok, int h, int32_t hkv, int32_t d,
                                             int64_t num_slots, E (*vrow)[128 + 16 / sizeof(E)],
                                             int64_t* sslot, int tid) {
  constexpr int kTok = kWriteTokens;
  // The K/V loads do not depend on the slot, so they are issued together with
  // the slot load (one memory round trip before the stores).
  const int cpr = d * (int)sizeof(E) / 16;  // 16-byte pieces per row
  for (int c = tid; c < kTok * cpr; c += 256) {
    const int ti = c / cpr, part = c - ti * cpr;
    if (ti >= ntok) break;
    int64_t s = slots[t0 + ti];
    if (s >= num_slots) s = -1;  // out of the pool: dropped like a padded token
    const size_t src = ((size_t)(t0 + ti) * hkv + h) * d;
    // the new tokens are read once: non-temporal loads (the cache rows they
    // are stored to stay cached for the attention that follows)
    const uint4 kv = load_stream16(reinterpret_cast<const uint4*>(key + src) + part);
    const uint4 vv = load_stream16(reinterpret_cast<const uint4*>(value + src) + part);
    if (part == 0) sslot[ti] = s;
    reinterpret_cast<uint4*>(&vrow[ti][0])[part] = vv;
    if (s < 0) continue;
    const size_t blk = (size_t)(s >> 4), off = (size_t)(s & 15);
    E* kdst = kc + ((blk * hkv + h) * kTok + off) * d;
    reinterpret_cast<uint4*>(kdst)[part] = kv;
  }
  __syncthreads();

  for (int e = tid; e < kTok * d; e += 256) {
    const int ti = e & (kTok - 1), c = e >> 4;
    if (ti >= ntok) continue;
    const int64_t s = sslot[ti];
    if (s < 0) continue;
    const size_t blk = (size_t)(s >> 4), off = (size_t)(s & 15);
    vc[((blk * hkv + h) * d + c) * kTok + off] = vrow[ti][c];
  }
}

}  // namespace pa
