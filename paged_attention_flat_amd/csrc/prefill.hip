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
// MI355X design.  A work-group owns 128 query rows = (128 / G) tokens x the G
// query heads of one KV head (token-major), so each K/V tile staged in LDS
// serves every head that reads it.  Each of its four waves owns 32 rows and
// runs 32x32x16 bf16 MFMAs:
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
// Key tiles are 64 keys (four cache blocks), double-buffered in LDS: the
// global loads of tile k+1 are issued before the MFMAs of tile k and written
// to the other buffer afterwards, one barrier per tile.  The running max is
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
#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* tables;
  const int32_t* plan;
  int32_t hq, hkv, table_stride;
  float scale_log2;
  uint16_t* out;
  float* lse;
};

constexpr int kPlanBuckets = 4096;

// Work list: plan[0] = item count, then (request, query tile) pairs sorted by
// the number of keys the tile's last row sees, largest first.  `tmp` holds
// the unsorted list (2 ints per item).  One work-group.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ qsl,
                                                    const int32_t* __restrict__ seq_lens,
                                                    int32_t num_seqs, int32_t dq, int32_t tq,
                                                    int32_t shift, int32_t* __restrict__ plan,
                                                    int32_t* __restrict__ tmp, int32_t cap) {
  __shared__ int s_scan[1024];
  __shared__ int hist[kPlanBuckets];
  __shared__ int s_base;
  const int tid = threadIdx.x;
  if (tid == 0) s_base = 0;
  for (int i = tid; i < kPlanBuckets; i += 1024) hist[i] = 0;
  __syncthreads();
  // 1. enumerate items (request, tile) into tmp, histogram of weights
  for (int c0 = 0; c0 < num_seqs; c0 += 1024) {
    const int b = c0 + tid;
    int n = 0, ql = 0, ctx = 0;
    if (b < num_seqs) {
      ql = qsl[b + 1] - qsl[b];
      ctx = seq_lens[b] - ql;
      if (ql > dq) n = (ql + tq - 1) / tq;
    }
    s_scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const int base = s_base + s_scan[tid] - n;
    for (int k = 0; k < n; ++k) {
      const int idx = base + k;
      if (idx < cap) {
        tmp[2 * idx] = b;
        tmp[2 * idx + 1] = k;
        const int keys = ctx + min((k + 1) * tq, ql);
        atomicAdd(&hist[kPlanBuckets - 1 - min(keys >> shift, kPlanBuckets - 1)], 1);
      }
    }
    __syncthreads();
    if (tid == 1023) s_base = s_base + s_scan[1023];
    __syncthreads();
  }
  const int count = min(s_base, cap);
  // 2. exclusive scan of the histogram (4 buckets per thread)
  int loc[4], s = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    loc[k] = s;
    s += hist[tid * 4 + k];
  }
  s_scan[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  const int base = s_scan[tid] - s;
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

constexpr int kBK = 64;     // keys per tile
constexpr int kKPad = 8;    // bf16 padding per K row in LDS
constexpr int kVPad = 8;    // bf16 padding per V^T row in LDS
constexpr float kLazy = 8.f;  // base-2 headroom before the running max moves
constexpr int kTabWin = 512;  // block-table entries held in LDS (8192 keys)

// position of key k (0..15) of a 16-key group in the V^T tile
__device__ __forceinline__ int vperm(int k) {
  return (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D, int G, int NW>
__global__ __launch_bounds__(64 * NW, (NW == 4 ? 2 : 1)) void prefill_kernel(PrefillParams p) {
  constexpr int NT = 64 * NW;         // threads
  constexpr int TQ = 32 * NW / G;     // tokens per work-group
  constexpr int QSTEPS = D / 16;      // MFMA k-steps over head_dim
  constexpr int DB = D / 32;          // 32-row blocks of O^T
  constexpr int KCH = kBK * D / 8 / NT;  // 16-byte K chunks per thread per tile
  constexpr int VCH = D * kBK / 8 / NT;  // 16-byte V chunks per thread per tile
  __shared__ __align__(16) uint16_t sK[2][kBK][D + kKPad];
  __shared__ __align__(16) uint16_t sV[2][D][kBK + kVPad];
  __shared__ int s_tab[kTabWin];

  const int kvh = blockIdx.x % p.hkv;
  const int item = blockIdx.x / p.hkv;
  if (item >= p.plan[0]) return;
  const int b = p.plan[1 + 2 * item];
  const int tile = p.plan[2 + 2 * item];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int row = lane & 31, kg = lane >> 5;

  const int q0 = p.qsl[b];
  const int q_len = p.qsl[b + 1] - q0;
  const int seq_len = p.seq_lens[b];
  const int ctx = seq_len - q_len;
  const int tok0 = tile * TQ;

  const int r = 32 * wave + row;
  const int tq = r / G, g = r - (r / G) * G;
  const int tok = tok0 + tq;
  const bool row_valid = tok < q_len;
  const int pos = ctx + min(tok, q_len - 1);
  const int wpos_lo = ctx + min(tok0 + (32 * wave) / G, q_len - 1);
  const int wpos_hi = ctx + min(tok0 + (32 * wave + 31) / G, q_len - 1);
  const int kend = ctx + min(tok0 + TQ, q_len);  // one past the last visible key

  bf16x8 qf[QSTEPS];
  if (row_valid) {
    const uint16_t* qrow = p.q + ((size_t)(q0 + tok) * p.hq + kvh * G + g) * D + 8 * kg;
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st)
      qf[st] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 16 * st));
  } else {
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st) qf[st] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  const int32_t* table = p.tables + (size_t)b * p.table_stride;
  const size_t head_elems = 16 * D;
  const size_t block_elems = (size_t)p.hkv * head_elems;
  const uint16_t* kbase = p.kc + kvh * head_elems;
  const uint16_t* vbase = p.vc + kvh * head_elems;

  // ---- staging: global -> registers -> LDS --------------------------------
  // Per-thread chunk geometry is fixed; only the tile's first block moves.
  // K chunk i: key kk = c / (D/8) of the tile, 8 dims at part*8.  V chunk i:
  // block bi of the tile, dim d, keys 8*half .. +7.
  int k_src[KCH], k_blk[KCH], k_dst[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int c = tid + NT * i;
    const int kk = c / (D / 8), part = c - kk * (D / 8);
    k_src[i] = (kk & 15) * D + part * 8;
    k_blk[i] = kk >> 4;
    k_dst[i] = kk * (D + kKPad) + part * 8;
  }
  int v_src[VCH], v_blk[VCH], v_key[VCH], v_dst[VCH];
#pragma unroll
  for (int i = 0; i < VCH; ++i) {
    const int c = tid + NT * i;
    const int bi = c / (2 * D);
    const int rem = c - bi * (2 * D);
    const int d = rem >> 1, half = rem & 1;
    v_src[i] = d * 16 + half * 8;
    v_blk[i] = bi;
    v_key[i] = bi * 16 + half * 8;
    v_dst[i] = d * (kBK + kVPad) + bi * 16;
  }
  int tab_base = 0;
  uint4 kr[KCH], vr[VCH];
  auto gload = [&](int k0) {
    const int tb = (k0 >> 4) - tab_base;
    if (k0 + kBK <= seq_len) {
      // whole tile inside the context: no per-key checks
#pragma unroll
      for (int i = 0; i < KCH; ++i)
        kr[i] = *reinterpret_cast<const uint4*>(kbase + (size_t)s_tab[tb + k_blk[i]] * block_elems +
                                                k_src[i]);
#pragma unroll
      for (int i = 0; i < VCH; ++i)
        vr[i] = *reinterpret_cast<const uint4*>(vbase + (size_t)s_tab[tb + v_blk[i]] * block_elems +
                                                v_src[i]);
      return;
    }
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int kpos = k0 + (k_src[i] / D) + 16 * k_blk[i];
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kpos < seq_len)
        v = *reinterpret_cast<const uint4*>(kbase + (size_t)s_tab[tb + k_blk[i]] * block_elems +
                                            k_src[i]);
      kr[i] = v;
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int kpos = k0 + v_key[i];
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kpos < seq_len) {
        v = *reinterpret_cast<const uint4*>(vbase + (size_t)s_tab[tb + v_blk[i]] * block_elems +
                                            v_src[i]);
        if (kpos + 8 > seq_len) {
          // keys past the context may hold anything (even NaN): zero them
          uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (kpos + e >= seq_len) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          v = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      vr[i] = v;
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* k_lds = &sK[buf][0][0];
    uint16_t* v_lds = &sV[buf][0][0];
#pragma unroll
    for (int i = 0; i < KCH; ++i) *reinterpret_cast<uint4*>(k_lds + k_dst[i]) = kr[i];
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      // keys 8*half .. +3 and +4 .. +7 of the block go to their permuted slots
      const int h8 = v_key[i] & 8;
      uint16_t* dst = v_lds + v_dst[i];
      *reinterpret_cast<uint2*>(dst + vperm(h8)) = make_uint2(vr[i].x, vr[i].y);
      *reinterpret_cast<uint2*>(dst + vperm(h8 + 4)) = make_uint2(vr[i].z, vr[i].w);
    }
  };

  float m = -INFINITY, l = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;

  // block-table window: entries [tab_base, tab_base + kTabWin) live in LDS.
  // It covers every block of the request: a 64-key tile can reach past the
  // last visible key, and those keys must still be read from their own
  // blocks (finite values times P = 0), never from a stand-in block.
  const int nblk = (seq_len + 15) >> 4;
  auto load_tab = [&](int base) {
    for (int i = tid; i < kTabWin; i += NT) s_tab[i] = (base + i < nblk) ? table[base + i] : 0;
  };
  load_tab(0);
  __syncthreads();
  gload(0);
  lstore(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < kend; k0 += kBK) {
    const bool more = k0 + kBK < kend;
    if (more && ((k0 + kBK) >> 4) >= tab_base + kTabWin) {
      // the next tile starts a new window (tiles never straddle one); every
      // thread is past its last use of the old entries
      tab_base += kTabWin;
      load_tab(tab_base);
      __syncthreads();
    }
    if (more) gload(k0 + kBK);
    if (k0 <= wpos_hi) {
      // ---- S^T = K Q^T over two 32-key halves --------------------------------
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
      const uint16_t* k_row0 = &sK[buf][row][8 * kg];
      const uint16_t* k_row1 = &sK[buf][32 + row][8 * kg];
      // two independent accumulation chains, operands fetched 4 steps ahead
#pragma unroll
      for (int s0 = 0; s0 < QSTEPS; s0 += 4) {
        uint4 fa[4], fb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          fa[u] = *reinterpret_cast<const uint4*>(k_row0 + 16 * (s0 + u));
          fb[u] = *reinterpret_cast<const uint4*>(k_row1 + 16 * (s0 + u));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[u]), qf[s0 + u], s[0], 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fb[u]), qf[s0 + u], s[1], 0, 0, 0);
        }
      }
      if (k0 + kBK - 1 > wpos_lo) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int key = k0 + 32 * kb + 8 * i + 4 * kg + j;
              if (key > pos) s[kb][4 * i + j] = -INFINITY;
            }
      }
      float mt = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mt = fmaxf(mt, s[kb][j]);
      mt = fmaxf(mt, shfl_xor(mt, 32)) * p.scale_log2;  // scale > 0 commutes with max
      if (__ballot(mt > m + kLazy) != 0) {
        const float m_new = fmaxf(m, mt);  // finite: key 0 is in the first tile
        const float alpha = fast_exp2(m - m_new);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        m = m_new;
      }
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          s[kb][j] = fast_exp2(__builtin_fmaf(s[kb][j], p.scale_log2, -m));
          rs += s[kb][j];
        }
      l += rs;

      // ---- O^T += V^T P^T, four 16-key steps ----------------------------------
#pragma unroll
      for (int ps = 0; ps < 4; ++ps) {
        const int kb = ps >> 1, ih = ps & 1;
        const f32x16& sp = s[kb];
        const bf16x8 pf = as_bf16x8(make_uint4(
            pack_bf16x2(sp[8 * ih + 0], sp[8 * ih + 1]), pack_bf16x2(sp[8 * ih + 2], sp[8 * ih + 3]),
            pack_bf16x2(sp[8 * ih + 4], sp[8 * ih + 5]), pack_bf16x2(sp[8 * ih + 6], sp[8 * ih + 7])));
        const int base = 32 * kb + 16 * ih + 8 * kg;
        uint4 fv[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
          fv[db] = *reinterpret_cast<const uint4*>(&sV[buf][32 * db + row][base]);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fv[db]), pf, acc[db], 0, 0, 0);
      }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  l += shfl_xor(l, 32);
  if (!row_valid) return;
  const float inv = 1.f / l;
  const int t = q0 + tok;
  const int h = kvh * G + g;
  uint16_t* orow = p.out + ((size_t)t * p.hq + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * kg;
      const f32x16& a = acc[db];
      *reinterpret_cast<uint2*>(orow + d) =
          make_uint2(pack_bf16x2(a[4 * i] * inv, a[4 * i + 1] * inv),
                     pack_bf16x2(a[4 * i + 2] * inv, a[4 * i + 3] * inv));
    }
  if (p.lse != nullptr && kg == 0) p.lse[(size_t)t * p.hq + h] = (m + fast_log2(l)) * kLn2;
}

template <int D, int G>
void launch_dg(const AttnArgs& a, hipStream_t stream) {
  constexpr int NW = PA_PREFILL_WAVES;
  PrefillParams p;
  p.q = (const uint16_t*)a.q;
  p.kc = (const uint16_t*)a.kc;
  p.vc = (const uint16_t*)a.vc;
  p.qsl = a.qsl;
  p.seq_lens = a.seq_lens;
  p.tables = a.tables;
  p.plan = a.plan;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.table_stride = a.table_stride;
  p.scale_log2 = a.scale * kLog2e;
  p.out = (uint16_t*)a.out;
  p.lse = a.lse;
  int shift = 0;
  while ((a.max_seq_len >> shift) >= kPlanBuckets) ++shift;
  trace_before(K_PLAN, stream);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, a.qsl, a.seq_lens, a.num_seqs,
                     decode_max_q(G), prefill_tile_tokens(G), shift, a.plan, a.plan_tmp,
                     a.plan_cap);
  trace_after(stream);
  trace_before(K_PREFILL, stream);
  hipLaunchKernelGGL((prefill_kernel<D, G, NW>), dim3(a.plan_cap * a.hkv), dim3(64 * NW), 0,
                     stream, p);
  trace_after(stream);
}

template <int D>
void launch_d(const AttnArgs& a, hipStream_t stream) {
  switch (a.hq / a.hkv) {
    case 1: launch_dg<D, 1>(a, stream); break;
    case 2: launch_dg<D, 2>(a, stream); break;
    case 4: launch_dg<D, 4>(a, stream); break;
    case 8: launch_dg<D, 8>(a, stream); break;
    default: launch_dg<D, 16>(a, stream); break;
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.d == 64) launch_d<64>(a, stream);
  else launch_d<128>(a, stream);
  return hipGetLastError();
}

}  // namespace pa
