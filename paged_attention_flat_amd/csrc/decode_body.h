// Decode attention body shared by the decode kernel and the mixed
// prefill + decode kernel: the per-unit computation of a (KV head, request,
// split) work unit, its parameters and its shared memory.  The method and the
// MI355X design are described in decode.hip.
#pragma once

#include "device_common.h"
#include "pa_internal.h"

namespace pa {

struct DecodeParams {
  const uint16_t* q;
  const void* kc;         // bf16 elements, or E4M3 codes (F8 kernels)
  const void* vc;
  const float* k_scale;   // F8 kernels: per-KV-head dequantisation scales
  const float* v_scale;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* tables;
  const int32_t* order;   // nullable: order[0] = count, order[1 + rank] = request
  int32_t num_seqs, hq, hkv, table_stride, splits, nt;
  int32_t split_blocks;   // blocks per split (even), from max_seq_len
  int32_t* sem;           // nullable: per (request, KV head) arrival counters
  float scale_log2;
  uint16_t* out;
  float* lse;
  float* part_out;
  float* part_lse;
  // shared-prefix attention: sharers skip the first pre_blocks blocks and
  // merge the prefix partial (row pre_index[b] + token) with their splits
  const int32_t* pre_index;  // nullable: [num_seqs], -1 for a non-sharer
  const float* pre_out;      // [pre_splits][pre_rows][hq][D]
  const float* pre_lse;      // [pre_splits][pre_rows][hq]
  int32_t pre_blocks;
  int32_t pre_splits;        // prefix partials per row (key ranges)
  int32_t pre_rows;
  // fused KV write (nullable): the step's new K/V rows [nt][hkv][D] and their
  // slots; the work-group whose block range holds a new token writes it
  const uint16_t* knew;
  const uint16_t* vnew;
  const int64_t* slots;
  int64_t num_slots;
};

// Two launch shapes.  Many work units: 4 waves per work-group, one pair in
// flight per wave (118 VGPRs, four work-groups and 16 waves per CU; against
// 8-wave work-groups: equal on 256 decodes of 512..8192 keys, 7 % faster on
// 256 short private suffixes behind a shared prefix, where each unit holds
// only a few pairs and four units per CU hide more of each unit's start and
// merge latency).  Few work units (at most two work-groups per CU): 4 waves
// per work-group, each keeping its next pair in flight while it computes the
// current one.
#ifndef PA_DECODE_WAVES_WIDE
#define PA_DECODE_WAVES_WIDE 4
#endif
#ifndef PA_DECODE_WAVES_PIPE
#define PA_DECODE_WAVES_PIPE 4
#endif
constexpr int kBuckets = 4096;

// Right shift that fits every request's block count into the sort's buckets.
inline int decode_order_shift(int32_t max_seq_len) {
  int shift = 0;
  const int max_blocks = (max_seq_len + 15) / 16;
  while ((max_blocks >> shift) >= kBuckets) ++shift;
  return shift;
}

// Shared memory of decode_order_block: the sort's histogram and scan, and
// (for the sharing test) an open-addressing set of first blocks (key = block
// id + 1, 0 = empty) with a bit per slot that marks a first block met more
// than once.
constexpr int kShareSlots = 16384;
struct OrderSmem {
  int hist[kBuckets];
  int part[kScanParts];
};
struct ShareSmem {
  uint32_t keys[kShareSlots];
  uint32_t multi[kShareSlots / 32];
};

// Requests whose first blocks the sharing test can hold (half the set).
constexpr int kShareMaxSeqs = kShareSlots / 2;

__device__ __forceinline__ int share_slot(uint32_t key) {
  return (int)((key * 2654435761u) >> 18);  // 14 bits: kShareSlots
}

// Bit 31 of an order entry: the request's blocks are taken as read by it
// alone (its V is streamed non-temporally by the decode units that read the
// order with the automatic policy).
constexpr uint32_t kOrderUnshared = 0x80000000u;

// Counting sort of the decode requests (0 < q_len <= dq) by block count,
// largest first, into order[0] = count, order[1 + rank] = request.  Called
// by every thread of one NT-thread work-group (it holds barriers); sm is its
// shared memory.  Ties keep no particular order (the order only schedules
// work, it never changes a result).
//
// With `tables` and `share` (nullable; num_seqs <= kShareMaxSeqs and 8 NT), each entry also
// says whether the request shares blocks with another request of the step:
// it does when its first block is the first block of another request (with
// any new or cached token).  Blocks are shared through common prefixes (a
// cached prefix, a forked sequence), so a request whose first block is its
// own reads no block that another request reads; a step that shares blocks
// any other way is only slower under the flag, never different.
template <int NT = 1024>
__device__ __forceinline__ void decode_order_block(const int32_t* __restrict__ qsl,
                                                   const int32_t* __restrict__ seq_lens,
                                                   const int32_t* __restrict__ tables,
                                                   int32_t table_stride, int32_t num_seqs,
                                                   int32_t dq, int32_t shift,
                                                   int32_t* __restrict__ order, OrderSmem& sm,
                                                   ShareSmem* share) {
  constexpr int kPer = kBuckets / NT;  // buckets per thread in the scan
  constexpr int kIt = 8;               // requests per thread held in registers
  const int tid = threadIdx.x;
  const bool in_regs = num_seqs <= kIt * NT;
  const bool detect = tables != nullptr && share != nullptr && in_regs &&
                      num_seqs <= kShareMaxSeqs;
  auto bucket = [&](int sl) {
    return kBuckets - 1 - min(((sl + 15) >> 4) >> shift, kBuckets - 1);
  };
  for (int i = tid; i < kBuckets; i += NT) sm.hist[i] = 0;
  if (detect) {
    for (int i = tid; i < kShareSlots; i += NT) share->keys[i] = 0u;
    for (int i = tid; i < kShareSlots / 32; i += NT) share->multi[i] = 0u;
  }
  int ql[kIt], sl[kIt], first[kIt];
  if (in_regs) {
    // every request's metadata loaded at once (one round trip), kept for
    // both passes
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int b = tid + it * NT;
      ql[it] = 0;
      sl[it] = 0;
      first[it] = -1;
      if (b < num_seqs) {
        ql[it] = qsl[b + 1] - qsl[b];
        sl[it] = seq_lens[b];
        if (detect) first[it] = tables[(size_t)b * table_stride];
      }
    }
  }
  __syncthreads();
  if (in_regs) {
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      if (detect && sl[it] > 0 && first[it] >= 0) {
        const uint32_t key = (uint32_t)first[it] + 1u;
        int h = share_slot(key);
        // the set is at most half full, so a free slot or the key is found
        for (int probe = 0; probe < kShareSlots; ++probe) {
          const uint32_t prev = atomicCAS(&share->keys[h], 0u, key);
          if (prev == 0u) break;
          if (prev == key) {
            atomicOr(&share->multi[h >> 5], 1u << (h & 31));
            break;
          }
          h = (h + 1) & (kShareSlots - 1);
        }
      }
      if (ql[it] > 0 && ql[it] <= dq) atomicAdd(&sm.hist[bucket(sl[it])], 1);
    }
  } else {
    for (int b = tid; b < num_seqs; b += NT) {
      const int q = qsl[b + 1] - qsl[b];
      if (q > 0 && q <= dq) atomicAdd(&sm.hist[bucket(seq_lens[b])], 1);
    }
  }
  __syncthreads();
  // exclusive scan of hist: kPer buckets per thread, then a scan of the partials
  int loc[kPer], s = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    loc[k] = s;
    s += sm.hist[tid * kPer + k];
  }
  int total;
  const int base = block_scan<NT>(s, sm.part, total) - s;
#pragma unroll
  for (int k = 0; k < kPer; ++k) sm.hist[tid * kPer + k] = base + loc[k];
  if (tid == 0) order[0] = total;
  __syncthreads();
  if (in_regs) {
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      if (ql[it] <= 0 || ql[it] > dq) continue;  // (also every b past num_seqs)
      uint32_t flag = 0u;
      if (detect && sl[it] > 0 && first[it] >= 0) {
        // the first block was entered above
        const uint32_t key = (uint32_t)first[it] + 1u;
        int h = share_slot(key);
        for (int probe = 0; probe < kShareSlots && share->keys[h] != key; ++probe)
          h = (h + 1) & (kShareSlots - 1);
        if (!((share->multi[h >> 5] >> (h & 31)) & 1u)) flag = kOrderUnshared;
      }
      const int pos = atomicAdd(&sm.hist[bucket(sl[it])], 1);
      order[1 + pos] = (int32_t)((uint32_t)(tid + it * NT) | flag);
    }
  } else {
    for (int b = tid; b < num_seqs; b += NT) {
      const int q = qsl[b + 1] - qsl[b];
      if (q <= 0 || q > dq) continue;
      const int pos = atomicAdd(&sm.hist[bucket(seq_lens[b])], 1);
      order[1 + pos] = b;
    }
  }
}

// The kernel's view of one call's arguments (host side).
inline DecodeParams make_decode_params(const AttnArgs& a) {
  DecodeParams p = {};
  p.q = (const uint16_t*)a.q;
  p.kc = a.kc;
  p.vc = a.vc;
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
  p.qsl = a.qsl;
  p.seq_lens = a.seq_lens;
  p.tables = a.tables;
  p.order = a.decode_order;
  p.num_seqs = a.num_seqs;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.table_stride = a.table_stride;
  p.splits = a.splits;
  p.nt = a.num_tokens;
  {
    const int max_blocks = (a.max_seq_len + 15) / 16;
    const int bps = (max_blocks + a.splits - 1) / a.splits;
    p.split_blocks = (bps + 1) & ~1;  // whole pairs per split
  }
  p.scale_log2 = a.scale * kLog2e;
  p.out = (uint16_t*)a.out;
  p.lse = a.lse;
  p.part_out = a.part_out;
  p.part_lse = a.part_lse;
  p.sem = a.sem;
  p.pre_index = a.sharers != nullptr ? a.pre_index : nullptr;
  p.pre_out = a.pre_out;
  p.pre_lse = a.pre_lse;
  p.pre_blocks = a.num_pre_blocks;
  p.pre_splits = a.casc_ksplits;
  p.pre_rows = a.casc_rows_max;
  p.knew = (const uint16_t*)a.knew;
  p.vnew = (const uint16_t*)a.vnew;
  p.slots = a.slots;
  p.num_slots = a.num_blocks * 16;
  return p;
}

// Shared memory of one decode work-group: the lane-local exchange buffer of
// the waves' merge (a slot per wave in the two-fragment-set shape, per pair
// of waves in the tree merge of the many-work-group shape; also the staging
// of the split merge) and the flag that elects the merging work-group.
template <int D, int NW, int PIPE>
struct DecodeSmem {
  float x[PIPE == 2 ? NW : NW / 2][4 * (D / 16) + 2][64];
  int last;
};

// Cache policy of a decode unit's K/V loads: non-temporal loads
// are not kept in L2/MALL for other readers.  A stream of whole 128-byte lines
// gains from them (V: each load covers 512 contiguous bytes of a block); K
// loads cover 64 bytes of 16 rows, which gains only in the long single
// decode.  Blocks read by several requests of a step are re-read from HBM
// under this policy.
constexpr int kNtK = 1;     // K loads non-temporal (bf16 cache)
constexpr int kNtV = 2;     // V loads non-temporal
constexpr int kNtAuto = 4;  // V loads non-temporal for requests the order marks unshared

// One decode work unit: (KV head, request rank) = bx (KV head fastest) and
// split = by, computed by the NW waves of the calling work-group (tidx: the
// thread's index in it) for request b (live = 0: a rank past the order's
// count, whose work-group only takes part in the tail write).  NTP: kNtK |
// kNtV, the loads that take the non-temporal policy.  Every exit is
// work-group uniform.
template <int D, int G, int NW, int PIPE, bool F8, int NTP>
__device__ __forceinline__ void decode_unit_body(const DecodeParams& p, int bx, int by, int b,
                                                 int live, DecodeSmem<D, NW, PIPE>& sm,
                                                 const int tidx) {
  typedef typename Frag8<F8>::elem CT;
  typedef typename Frag8<F8>::raw RT;
  constexpr int DQ = 16 / G;       // new tokens per request packed in the columns
  constexpr int KSTEPS = D / 32;   // MFMA steps over head_dim for S^T
  constexpr int DB = D / 16;       // 16-row blocks of O^T
  constexpr int NREG = 4 * DB + 2; // per-lane state: acc, m, l

  // lane-local exchange buffer for the tree merge of the waves' states
  constexpr int kSlots = PIPE == 2 ? NW : NW / 2;
  float (&s_x)[kSlots][NREG][64] = sm.x;

  const int kvh = bx % p.hkv;
  const int split = by;
  const int lane = tidx & 63, wave = tidx >> 6;
  const int col = lane & 15, kg = lane >> 4;

  CT* const kc_w = const_cast<CT*>(static_cast<const CT*>(p.kc));
  CT* const vc_w = const_cast<CT*>(static_cast<const CT*>(p.vc));
  const bool tail_wg = p.knew != nullptr && bx == 0 && by == 0;
  if (tail_wg) {
    // fused KV write of tokens after the last request's rows (no row reads
    // them; written for the pool's sake, every KV head)
    for (int t = p.qsl[p.num_seqs]; t < p.nt; ++t) {
      const int64_t sl = p.slots[t];
      if (sl < 0 || sl >= p.num_slots) continue;
      const size_t cb = (size_t)(sl >> 4), off = (size_t)(sl & 15);
      for (int e = tidx; e < p.hkv * D; e += 64 * NW) {
        const int hh = e / D, dd = e - hh * D;
        const size_t head = (cb * p.hkv + hh) * 16 * D;
        const size_t src = ((size_t)t * p.hkv + hh) * D + dd;
        if constexpr (F8) {
          kc_w[head + off * D + dd] = e4m3_code(bf16_bits_to_f32(p.knew[src]) / p.k_scale[hh]);
          vc_w[head + (size_t)dd * 16 + off] =
              e4m3_code(bf16_bits_to_f32(p.vnew[src]) / p.v_scale[hh]);
        } else {
          kc_w[head + off * D + dd] = p.knew[src];
          vc_w[head + (size_t)dd * 16 + off] = p.vnew[src];
        }
      }
    }
  }
  if (!live) return;
  // Split s covers blocks [s * bps, (s + 1) * bps) of every request, bps from
  // the host-known max_seq_len, so the first 64 block-table entries can be
  // fetched together with query_start_loc / seq_lens (one round trip fewer
  // before the first K/V load).  Splits past a shorter request are empty.
  const int pv0 = p.pre_index != nullptr ? p.pre_index[b] : -1;
  const int q0 = p.qsl[b];
  const int q1 = p.qsl[b + 1];
  const int seq_len = p.seq_lens[b];
  const int blk_lo = (pv0 >= 0 ? p.pre_blocks : 0) + split * p.split_blocks;
  const int32_t* table = p.tables + (size_t)b * p.table_stride;
  int tab = 0, tab_base = 0;
  {
    const int j = blk_lo + lane;
    tab = j < p.table_stride ? table[j] : 0;
  }
  const int q_len = q1 - q0;
  // empty request, a prefill row set, or (invalid) fewer cached than new
  // tokens; seq_len in the test keeps its load in the same round trip
  if (q_len <= 0 || q_len > DQ || seq_len < q_len) return;
  const int ctx = seq_len - q_len;
  const int nblocks = (seq_len + 15) >> 4;
  const int blk_hi = min(nblocks, blk_lo + p.split_blocks);

  const int qi = col / G, g = col - (col / G) * G;
  const int qpos = ctx + min(qi, q_len - 1);
  const bool col_valid = qi < q_len;

  // Fused KV write.  The slot of position p is table[p / 16] * 16 + p % 16
  // ("Model execution", "Flattening a step"), so the only reader of a new
  // token's entry (for this KV head) is the wave of this unit that processes
  // the pair of blocks holding it: that wave writes the token (K row and V
  // column; E4M3 cache: quantised exactly as pa_kv_write_fp8 does) and waits
  // for its own stores (vmcnt(0)) before it loads that pair.  No barrier:
  // the other waves never read these entries.  No stale copy can be read
  // either: the vector L1 is write-through and starts each launch empty, and
  // within a launch nothing else reads those bytes before the write -- other
  // units of this request and KV head cover other blocks, other requests'
  // units read other blocks (the slot rule puts a request's new tokens in its
  // own last blocks, which no other request reads), and in the persistent
  // mixed launch the prefill units read prefill requests' blocks only.  So
  // the load, issued after the stores were acknowledged by this XCD's L2,
  // finds no L1 line for them and reads the new bytes from that L2.
  // The first token a wave writes is fetched before its first K/V loads are
  // issued, so the write costs no round trip of its own.
  auto own_tok = [&](int i) {
    const int blk = (ctx + i) >> 4;
    return blk >= blk_lo && blk < blk_hi && (((blk - blk_lo) >> 1) % NW) == wave;
  };
  int own0 = -1;
  if (p.knew != nullptr) {
    for (int i = q_len - 1; i >= 0; --i)
      if (own_tok(i)) own0 = i;
  }
  const bool own_any = own0 >= 0;
  auto pair_new = [&](int pr) {  // pair pr of this wave holds a token it wrote
    const int k0 = 16 * (blk_lo + 2 * pr);
    return own_any && k0 + 32 > ctx && k0 < seq_len;
  };
  struct NewTok {
    int64_t slot;
    uint4 k;             // lanes < D / 8: 8 elements of the K row
    uint16_t v[D / 64];  // elements lane + 64 j of the V row
  };
  auto fetch_tok = [&](int i, NewTok& t) {
    const size_t src = ((size_t)(q0 + i) * p.hkv + kvh) * D;
    t.slot = p.slots[q0 + i];
    t.k = lane < D / 8 ? *reinterpret_cast<const uint4*>(p.knew + src + 8 * lane)
                       : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < D / 64; ++j) t.v[j] = p.vnew[src + lane + 64 * j];
  };
  auto put_tok = [&](const NewTok& t) {
    if (t.slot < 0 || t.slot >= p.num_slots) return;
    const size_t cb = (size_t)(t.slot >> 4), off = (size_t)(t.slot & 15);
    const size_t head = (cb * p.hkv + kvh) * 16 * D;
    if (lane < D / 8) {
      if constexpr (F8) {
        const float ks = p.k_scale[kvh];
        const uint32_t w[4] = {t.k.x, t.k.y, t.k.z, t.k.w};
        float f[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f[2 * j] = __uint_as_float(w[j] << 16) / ks;
          f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u) / ks;
        }
        *reinterpret_cast<uint2*>(kc_w + head + off * D + 8 * lane) =
            make_uint2(e4m3_pack4(f[0], f[1], f[2], f[3]), e4m3_pack4(f[4], f[5], f[6], f[7]));
      } else {
        *reinterpret_cast<uint4*>(kc_w + head + off * D + 8 * lane) = t.k;
      }
    }
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
      const size_t dd = lane + 64 * j;
      if constexpr (F8)
        vc_w[head + dd * 16 + off] = e4m3_code(bf16_bits_to_f32(t.v[j]) / p.v_scale[kvh]);
      else
        vc_w[head + dd * 16 + off] = t.v[j];
    }
  };
  // (G = 16, bf16: the early fetch would cost a register spill in the
  // two-set loop, so the token is fetched when it is written)
  constexpr bool kEarly = !(G >= 16 && !F8 && D == 128);
  NewTok tok0;
  if (kEarly && own_any) fetch_tok(own0, tok0);
  // called once this wave's first loads are issued: its stores, then (rare)
  // the further tokens it owns, each fetched and stored in turn
  auto write_own = [&]() {
    if (!own_any) return;
    if (!kEarly) fetch_tok(own0, tok0);
    put_tok(tok0);
    for (int i = own0 + 1; i < q_len; ++i) {
      if (!own_tok(i)) continue;
      NewTok t;
      fetch_tok(i, t);
      put_tok(t);
    }
  };

  // Q as the B operand: lane (col, kg) holds d = kd(st) .. +8 with
  // kd(st) = 32*st + 8*kg.  E4M3 cache: the head dimension is taken in the
  // order kd(st) = 64*(st/2) + 16*kg + 8*(st%2) (a permutation of the
  // dot product's terms, the same for K and Q), so that one 16-byte load
  // gives a lane its K codes for two steps.
  static_assert(!F8 || KSTEPS % 2 == 0, "E4M3 K loads cover two steps");
  auto kd = [&](int st) { return F8 ? 64 * (st >> 1) + 16 * kg + 8 * (st & 1) : 32 * st + 8 * kg; };
  bf16x8 qf[KSTEPS];
  if (col_valid) {
    const uint16_t* qrow = p.q + ((size_t)(q0 + qi) * p.hq + kvh * G + g) * D;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
      qf[st] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + kd(st)));
  } else {
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) qf[st] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  // Key order inside a pair of blocks (32 keys).  MFMA row r of the first
  // S^T product is key 8*(r/4) + r%4, of the second key 8*(r/4) + 4 + r%4, so
  // lane (col, kg) ends up with the 8 consecutive keys 8*kg .. 8*kg+7 of the
  // pair: the same 8 keys its V operand reads as one 16-byte run of the
  // dim-major block (block kg/2, keys 8*(kg%2) ..).
  const int ra = 8 * (col >> 2) + (col & 3);   // pair key of A row `col`, first product
  const int rb = ra + 4;                       // second product
  const size_t head_elems = 16 * D;
  const size_t block_elems = (size_t)p.hkv * head_elems;
  const CT* kbase = static_cast<const CT*>(p.kc) + kvh * head_elems + kd(0);
  const CT* vbase = static_cast<const CT*>(p.vc) + kvh * head_elems + col * 16 + 8 * (kg & 1);
  // E4M3 cache: a cached K value is code * k_scale, so the scale folds into
  // the score scale; V's scale multiplies the normalised output
  const float scale_log2 = F8 ? p.scale_log2 * p.k_scale[kvh] : p.scale_log2;
  const float v_scale = F8 ? p.v_scale[kvh] : 1.f;

  float m = -INFINITY, l = 0.f;
  f32x4 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int npairs = blk_hi > blk_lo ? (blk_hi - blk_lo + 1) >> 1 : 0;

  struct Frag {
    RT a[KSTEPS], b[KSTEPS];
    RT v[DB];
  };
  auto load = [&](Frag& f, int pr) {
    const int rel = 2 * pr;  // block offset inside the split
    if ((rel & ~63) != tab_base) {
      // 64 table entries per load, read back with readlane
      tab_base = rel & ~63;
      const int j = blk_lo + tab_base + lane;
      tab = j < blk_hi ? table[j] : 0;
    }
    // (entries at or past blk_hi are never picked: a missing second block
    // of a pair falls back to the first)
    const bool has1 = blk_lo + rel + 1 < blk_hi;
    const int phys0 = __builtin_amdgcn_readlane(tab, rel & 63);
    const int phys1 = has1 ? __builtin_amdgcn_readlane(tab, (rel & 63) + 1) : phys0;
    const int pa_ = ra < 16 ? phys0 : phys1, pb_ = rb < 16 ? phys0 : phys1;
    const CT* ka = kbase + (size_t)pa_ * block_elems + (ra & 15) * D;
    const CT* kb = kbase + (size_t)pb_ * block_elems + (rb & 15) * D;
    const CT* vp = vbase + (size_t)(kg < 2 ? phys0 : phys1) * block_elems;
    auto ldk = [](const CT* ptr) -> RT {
      if constexpr ((NTP & kNtK) && !F8) return load_stream16(reinterpret_cast<const uint4*>(ptr));
      else return *reinterpret_cast<const RT*>(ptr);
    };
    auto ldv = [](const CT* ptr) -> RT {
      if constexpr ((NTP & kNtV) && !F8) {
        return load_stream16(reinterpret_cast<const uint4*>(ptr));
      } else if constexpr ((NTP & kNtV) && F8) {
        // 8 codes: 256 contiguous bytes per 16 lanes, whole lines as for bf16
        return load_stream8(reinterpret_cast<const uint2*>(ptr));
      } else {
        return *reinterpret_cast<const RT*>(ptr);
      }
    };
    if constexpr (F8) {
      // 16 codes per load: steps 2t and 2t+1 (kd(2t + 1) = kd(2t) + 8)
#pragma unroll
      for (int t = 0; t < KSTEPS / 2; ++t) {
        const uint4 wa = *reinterpret_cast<const uint4*>(ka + 64 * t);
        const uint4 wb = *reinterpret_cast<const uint4*>(kb + 64 * t);
        f.a[2 * t] = make_uint2(wa.x, wa.y);
        f.a[2 * t + 1] = make_uint2(wa.z, wa.w);
        f.b[2 * t] = make_uint2(wb.x, wb.y);
        f.b[2 * t + 1] = make_uint2(wb.z, wb.w);
      }
    } else {
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        f.a[st] = ldk(ka + 32 * st);
        f.b[st] = ldk(kb + 32 * st);
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) f.v[db] = ldv(vp + db * 256);
  };
  auto compute = [&](Frag& f, int pr) {
    const int j0 = blk_lo + 2 * pr;
    const bool has1 = j0 + 1 < blk_hi;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Frag8<F8>::bits(f.a[st])), qf[st], s0,
                                                   0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Frag8<F8>::bits(f.b[st])), qf[st], s1,
                                                   0, 0, 0);
    }
    // lane (col, kg): sv[e] is the score of pair key 8*kg + e
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = s0[i];
      sv[4 + i] = s1[i];
    }
    const int kp0 = 16 * j0 + 8 * kg;  // position of sv[0]
    if (16 * j0 + 31 > ctx) {
      // the pair reaches past the first new token: causal mask per column;
      // keys past the context (tail of the last block, or a missing second
      // block) must not reach the P.V product even as NaN * 0
      uint32_t vm[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
      const bool blk_ok = has1 || kg < 2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kp = kp0 + e;
        if (!blk_ok || kp > qpos) sv[e] = -INFINITY;
        if (!blk_ok || kp >= seq_len) {
          if constexpr (F8) vm[e >> 2] &= ~(0xffu << (8 * (e & 3)));  // code 0 = +0
          else vm[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if constexpr (F8) {
          f.v[db].x &= vm[0];
          f.v[db].y &= vm[1];
        } else {
          f.v[db].x &= vm[0];
          f.v[db].y &= vm[1];
          f.v[db].z &= vm[2];
          f.v[db].w &= vm[3];
        }
      }
    }
    float mt = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mt = max_xor32(max_xor16(mt));
    mt *= scale_log2;  // scale > 0 commutes with max
    const float m_new = fmaxf(m, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float pv[8], rs = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = fast_exp2(__builtin_fmaf(sv[i], scale_log2, -m_use));
      rs += pv[i];
    }
    l = l * alpha + rs;
    m = m_new;

    const bf16x8 pf = as_bf16x8(make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                           pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])));
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] *= alpha;
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Frag8<F8>::bits(f.v[db])), pf,
                                                        acc[db], 0, 0, 0);
    }
  };

  // waits for this wave's KV-write stores before it loads a pair they hit
  auto load_after_write = [&](Frag& f, int pr) {
    if (pair_new(pr)) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    load(f, pr);
  };
  if constexpr (PIPE == 1) {
    // many work-groups per CU: the write's round trip hides behind the others
    write_own();
    for (int pr = wave; pr < npairs; pr += NW) {
      Frag f;
      load_after_write(f, pr);
      compute(f, pr);
    }
  } else {
    // two fragment sets: the next pair's loads are in flight during compute
    Frag fa, fb;
    int pr = wave;
    const bool d0 = pair_new(pr);
    if (pr < npairs && !d0) load(fa, pr);
    write_own();
    if (pr < npairs && d0) load_after_write(fa, pr);
    while (pr < npairs) {
      int pn = pr + NW;
      if (pn < npairs) load_after_write(fb, pn);
      compute(fa, pr);
      pr = pn;
      if (pr >= npairs) break;
      pn = pr + NW;
      if (pn < npairs) load_after_write(fa, pn);
      compute(fb, pr);
      pr = pn;
    }
  }

  // per-column denominator: sum the four key groups of the wave
  l = sum_xor32(sum_xor16(l));

  // Merge of the waves' states.  Each wave ends up with the merged result
  // for its share of the head dimension (dim blocks db0 .. db1 - 1, in
  // mac[0 .. db1 - db0)) and the merged (m, l) of its columns.
  //  - two-fragment-set shape: one exchange.  Every wave writes its (acc, m,
  //    l) to LDS, then wave w combines the NW states for its share.  Every
  //    wave holds the same (column, dim) layout, so the merge is lane-local.
  //    Against a tree merge (one pair of waves per level: two LDS rounds and
  //    four barriers at four waves) it takes 1.5 % off the long single decode
  //    and the mixed step;
  //  - many-work-group shape: the tree merge, wave 0 keeping every dim (twice
  //    the LDS per work-group for the one exchange cost the short units of the
  //    shared-prefix decode 10 %).
  constexpr int DPW = PIPE == 2 ? (DB + NW - 1) / NW : DB;  // dim blocks per wave
  int db0 = 0, db1 = 0;
  f32x4 mac[DPW];
  if constexpr (PIPE == 2) {
    db0 = min(DB, wave * DPW);
    db1 = min(DB, db0 + DPW);
    {
      float* x = &s_x[wave][0][lane];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[(4 * db + i) * 64] = acc[db][i];
      x[(4 * DB) * 64] = m;
      x[(4 * DB + 1) * 64] = l;
    }
    __syncthreads();
    float wgt[NW];
    {
      float M = -INFINITY;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, s_x[w2][4 * DB][lane]);
      float L = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) {
        const float mo = s_x[w2][4 * DB][lane];
        wgt[w2] = (mo == -INFINITY) ? 0.f : fast_exp2(mo - M);
        L += wgt[w2] * s_x[w2][4 * DB + 1][lane];
      }
      m = M;
      l = L;
    }
#pragma unroll
    for (int k = 0; k < DPW; ++k) {
      mac[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int db = db0 + k;
      if (db < db1) {
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2)
#pragma unroll
          for (int i = 0; i < 4; ++i) mac[k][i] += wgt[w2] * s_x[w2][4 * db + i][lane];
      }
    }
  } else {
#pragma unroll
    for (int half = NW / 2; half >= 1; half >>= 1) {
      if (wave >= half && wave < 2 * half) {
        float* x = &s_x[wave - half][0][lane];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[(4 * db + i) * 64] = acc[db][i];
        x[(4 * DB) * 64] = m;
        x[(4 * DB + 1) * 64] = l;
      }
      __syncthreads();
      if (wave < half) {
        const float* x = &s_x[wave][0][lane];
        const float mo = x[(4 * DB) * 64], lo = x[(4 * DB + 1) * 64];
        const float M = fmaxf(m, mo);
        const float wa = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
        const float wb = (mo == -INFINITY) ? 0.f : fast_exp2(mo - M);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[db][i] = acc[db][i] * wa + x[(4 * db + i) * 64] * wb;
        l = l * wa + lo * wb;
        m = M;
      }
      __syncthreads();
    }
    if (wave == 0) db1 = DB;
#pragma unroll
    for (int k = 0; k < DPW; ++k) mac[k] = acc[k];
  }
  const int t = q0 + qi;
  const int h = kvh * G + g;
  // a sharer always merges (its splits and the prefix partial)
  const bool merged = p.splits > 1 || pv0 >= 0;
  if (col_valid && db0 < db1) {
    if (!merged) {
      const float inv = v_scale / l;
      uint16_t* dst = p.out + ((size_t)t * p.hq + h) * D + 4 * kg;
#pragma unroll
      for (int k = 0; k < DPW; ++k) {
        const int db = db0 + k;
        if (db < db1)
          *reinterpret_cast<uint2*>(dst + 16 * db) =
              make_uint2(pack_bf16x2(mac[k][0] * inv, mac[k][1] * inv),
                         pack_bf16x2(mac[k][2] * inv, mac[k][3] * inv));
      }
      if (p.lse != nullptr && wave == 0 && kg == 0)
        p.lse[(size_t)t * p.hq + h] = (m + fast_log2(l)) * kLn2;
    } else if (p.splits == 1) {
      // a sharer without a split: merge the prefix partials (written by the
      // previous launch on this stream) with this work-group's own result
      const size_t prer = (size_t)(pv0 + qi) * p.hq + h;
      const size_t kstride = (size_t)p.pre_rows * p.hq;
      const float lb = (l == 0.f) ? -INFINITY : (m + fast_log2(l)) * kLn2;
      float M = lb;
      for (int ks = 0; ks < p.pre_splits; ++ks) M = fmaxf(M, p.pre_lse[ks * kstride + prer]);
      const float wb = (lb == -INFINITY) ? 0.f : fast_exp2((lb - M) * kLog2e);
      float den = wb;
      float4 o[DPW];
      const float cb = (l == 0.f) ? 0.f : wb * v_scale / l;
#pragma unroll
      for (int k = 0; k < DPW; ++k)
        o[k] = make_float4(cb * mac[k][0], cb * mac[k][1], cb * mac[k][2], cb * mac[k][3]);
      for (int ks = 0; ks < p.pre_splits; ++ks) {
        const float la = p.pre_lse[ks * kstride + prer];
        const float wa = (la == -INFINITY) ? 0.f : fast_exp2((la - M) * kLog2e);
        den += wa;
        const float* src = p.pre_out + (ks * kstride + prer) * D + 4 * kg;
#pragma unroll
        for (int k = 0; k < DPW; ++k) {
          const int db = db0 + k;
          if (db < db1) {
            const float4 oa = *reinterpret_cast<const float4*>(src + 16 * db);
            o[k].x += wa * oa.x; o[k].y += wa * oa.y; o[k].z += wa * oa.z; o[k].w += wa * oa.w;
          }
        }
      }
      const float inv = 1.f / den;
      uint16_t* dst = p.out + ((size_t)t * p.hq + h) * D + 4 * kg;
#pragma unroll
      for (int k = 0; k < DPW; ++k) {
        const int db = db0 + k;
        if (db < db1)
          *reinterpret_cast<uint2*>(dst + 16 * db) =
              make_uint2(pack_bf16x2(o[k].x * inv, o[k].y * inv),
                         pack_bf16x2(o[k].z * inv, o[k].w * inv));
      }
      if (p.lse != nullptr && wave == 0 && kg == 0)
        p.lse[(size_t)t * p.hq + h] = M + fast_log2(den) * kLn2;
    } else {
      const bool empty = (l == 0.f);
      const float inv = empty ? 0.f : v_scale / l;
      float* dst = p.part_out + (((size_t)split * p.nt + t) * p.hq + h) * D + 4 * kg;
      // device-scope atomic stores write through this XCD's L2, so the
      // merging work-group (possibly on another XCD) reads them from memory
      // without an L2 write-back here
#pragma unroll
      for (int k = 0; k < DPW; ++k) {
        const int db = db0 + k;
        if (db < db1) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __hip_atomic_store(dst + 16 * db + i, mac[k][i] * inv, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (wave == 0 && kg == 0)
        __hip_atomic_store(p.part_lse + ((size_t)split * p.nt + t) * p.hq + h,
                           empty ? -INFINITY : (m + fast_log2(l)) * kLn2, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (!merged || p.splits == 1 || p.sem == nullptr) return;

  // ---- merge of the split partials by the last split to finish ------------
  // (the split-KV method merges its partials in a separate reduction pass:
  // "Inside the engine: kernels, CUDA graphs and the life of a request",
  // section "Prefill has a full grid; decode at batch 1 has almost none";
  // here that pass is done by whichever work-group of this (request, KV head)
  // completes last, so the step needs no second launch).  Every wave stored
  // its share of the partial with device-scope atomic stores: once each
  // wave's store counter has drained they are visible device-wide, and after
  // a barrier thread 0 counts the arrival.  (A release fence would also write
  // back this XCD's whole L2, which costs microseconds per work-group;
  // nothing else here needs publishing.)  The last arrival acquires, which
  // drops stale L2 lines, before reading the other splits' partials.  The
  // counter is returned to zero for the next call.
  int& s_last = sm.last;
  int* sem = p.sem + (size_t)b * p.hkv + kvh;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tidx == 0)
    s_last = __hip_atomic_fetch_add(sem, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             p.splits - 1;
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // Items are (row, 4 dims); with fewer items than threads the splits are
  // dealt round-robin to SG groups of threads.  Each thread keeps its own
  // running (max, sum, acc) over chunks of CH splits whose loads are all in
  // flight together, then the groups are merged through LDS.
  constexpr int NT = 64 * NW;
  constexpr int QUADS = D / 4;
  constexpr int CH = (PIPE == 2) ? 16 : 8;
  const int rows = q_len * G;
  const int items = rows * QUADS;
  const int sg = items >= NT ? 1 : NT / items;
  const size_t split_rows = (size_t)p.nt * p.hq;
  // the prefix partials (one per key range) come after the splits
  const int nparts = p.splits + (pv0 >= 0 ? p.pre_splits : 0);
  const size_t kstride = (size_t)p.pre_rows * p.hq;
  float* s_m = &s_x[0][0][0];  // [6][NT] staging for the group merge
  static_assert(sizeof(s_x) >= 6 * NT * sizeof(float), "LDS staging too small");
  for (int base = 0; base < items * sg; base += NT) {
    const int slot = base + tidx;
    const bool act = slot < items * sg;
    const int item = slot % items, grp = slot / items;
    const int r = item / QUADS, quad = item - (item / QUADS) * QUADS;
    const int tt = q0 + r / G, hh = kvh * G + (r - (r / G) * G);
    const size_t rowi = (size_t)tt * p.hq + hh;
    const float* ob = p.part_out + rowi * D + quad * 4;
    const size_t prer = (size_t)(pv0 + r / G) * p.hq + hh;  // row of the prefix partial
    float mm = -INFINITY, ll = 0.f;
    float4 ac = make_float4(0.f, 0.f, 0.f, 0.f);
    if (act) {
      for (int s0 = grp; s0 < nparts; s0 += CH * sg) {
        float x[CH];
        float4 v[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int sp = s0 + c * sg;
          x[c] = -INFINITY;
          v[c] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (sp < p.splits) {
            x[c] = p.part_lse[sp * split_rows + rowi];
            v[c] = *reinterpret_cast<const float4*>(ob + sp * split_rows * D);
          } else if (sp < nparts) {
            const size_t pi = (size_t)(sp - p.splits) * kstride + prer;
            x[c] = p.pre_lse[pi];
            v[c] = *reinterpret_cast<const float4*>(p.pre_out + pi * D + quad * 4);
          }
        }
        float mc = mm;
#pragma unroll
        for (int c = 0; c < CH; ++c) mc = fmaxf(mc, x[c]);
        if (mc == -INFINITY) continue;  // only empty splits so far
        const float a = fast_exp2((mm - mc) * kLog2e);  // 0 while mm = -inf
        ac.x *= a; ac.y *= a; ac.z *= a; ac.w *= a;
        ll *= a;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const float w = fast_exp2((x[c] - mc) * kLog2e);  // 0 for an empty split
          // empty splits carry zeros, so w * v stays finite
          ac.x += w * v[c].x; ac.y += w * v[c].y; ac.z += w * v[c].z; ac.w += w * v[c].w;
          ll += w;
        }
        mm = mc;
      }
    }
    if (sg == 1) {
      if (act) {
        const float inv = 1.f / ll;
        uint16_t* dst = p.out + rowi * D + quad * 4;
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(ac.x * inv, ac.y * inv),
                                                    pack_bf16x2(ac.z * inv, ac.w * inv));
        if (p.lse != nullptr && quad == 0) p.lse[rowi] = mm + fast_log2(ll) * kLn2;
      }
      continue;
    }
    // sg > 1: a single pass (items * sg <= NT); merge the groups of each item
    s_m[0 * NT + tidx] = mm;
    s_m[1 * NT + tidx] = ll;
    s_m[2 * NT + tidx] = ac.x;
    s_m[3 * NT + tidx] = ac.y;
    s_m[4 * NT + tidx] = ac.z;
    s_m[5 * NT + tidx] = ac.w;
    __syncthreads();
    if (tidx < items) {
      float M = -INFINITY;
      for (int g2 = 0; g2 < sg; ++g2) M = fmaxf(M, s_m[g2 * items + tidx]);
      float L = 0.f;
      float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int g2 = 0; g2 < sg; ++g2) {
        const int k = g2 * items + tidx;
        const float mg = s_m[k];
        const float a = mg == -INFINITY ? 0.f : fast_exp2((mg - M) * kLog2e);
        L += a * s_m[NT + k];
        A.x += a * s_m[2 * NT + k];
        A.y += a * s_m[3 * NT + k];
        A.z += a * s_m[4 * NT + k];
        A.w += a * s_m[5 * NT + k];
      }
      const float inv = 1.f / L;
      uint16_t* dst = p.out + rowi * D + quad * 4;
      *reinterpret_cast<uint2*>(dst) =
          make_uint2(pack_bf16x2(A.x * inv, A.y * inv), pack_bf16x2(A.z * inv, A.w * inv));
      if (p.lse != nullptr && quad == 0) p.lse[rowi] = M + fast_log2(L) * kLn2;
    }
  }
  if (tidx == 0) __hip_atomic_store(sem, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The work unit of decode_unit_body, its request read from the decode order
// (one scalar round trip, before the request's own metadata).  NTP may add
// kNtAuto: the unit then streams V non-temporally when the order marks its
// request as reading no block another request reads.  order[1 + rank] is in
// bounds for every rank (rank < num_seqs).
template <int D, int G, int NW, int PIPE, bool F8, int NTP>
__device__ __forceinline__ void decode_unit(const DecodeParams& p, int bx, int by,
                                            DecodeSmem<D, NW, PIPE>& sm, const int tidx) {
  const int rank = bx / p.hkv;
  int b = rank, live = 1;
  bool unshared = false;
  if (p.order != nullptr) {
    live = rank < p.order[0];
    const uint32_t v = (uint32_t)p.order[1 + rank];
    b = (int)(v & ~kOrderUnshared);
    unshared = (v & kOrderUnshared) != 0u;
  }
  if constexpr ((NTP & kNtAuto) != 0) {
    constexpr int kBase = NTP & ~kNtAuto;
    if (unshared)
      decode_unit_body<D, G, NW, PIPE, F8, kBase | kNtV>(p, bx, by, b, live, sm, tidx);
    else
      decode_unit_body<D, G, NW, PIPE, F8, kBase>(p, bx, by, b, live, sm, tidx);
  } else {
    decode_unit_body<D, G, NW, PIPE, F8, NTP>(p, bx, by, b, live, sm, tidx);
  }
}

}  // namespace pa
