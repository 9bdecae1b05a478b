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
// max needs one cross-lane exchange per tile.  Key tiles are 64 keys (four
// cache blocks).  A device-built work list (one entry per (request, query
// tile) of requests with more new tokens than the decode kernel packs) lets
// mixed batches launch without a host read of the metadata.
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

// Work list: plan[0] = item count, then (request, query tile) pairs.  Tiles of
// a request are listed last-first (the later tiles see more keys).
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ qsl,
                                                    int32_t num_seqs, int32_t dq,
                                                    int32_t tq, int32_t* __restrict__ plan,
                                                    int32_t cap) {
  __shared__ int s_scan[1024];
  __shared__ int s_base;
  const int tid = threadIdx.x;
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int c0 = 0; c0 < num_seqs; c0 += 1024) {
    const int b = c0 + tid;
    int n = 0;
    if (b < num_seqs) {
      const int ql = qsl[b + 1] - qsl[b];
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
        plan[1 + 2 * idx] = b;
        plan[2 + 2 * idx] = n - 1 - k;
      }
    }
    __syncthreads();
    if (tid == 1023) s_base = s_base + s_scan[1023];
    __syncthreads();
  }
  if (tid == 0) plan[0] = min(s_base, cap);
}

constexpr int kBK = 64;     // keys per tile
constexpr int kKPad = 8;    // bf16 padding per K row in LDS
constexpr int kVPad = 8;    // bf16 padding per V^T row in LDS

template <int D, int G>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
  constexpr int TQ = 128 / G;    // tokens per work-group
  constexpr int QSTEPS = D / 16; // MFMA k-steps over head_dim
  constexpr int DB = D / 32;     // 32-row blocks of O^T
  __shared__ __align__(16) uint16_t sK[kBK][D + kKPad];
  __shared__ __align__(16) uint16_t sV[D][kBK + kVPad];

  const int item = blockIdx.x, kvh = blockIdx.y;
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

  float m = -INFINITY, l = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < kend; k0 += kBK) {
    __syncthreads();  // the previous tile has been consumed
    // ---- stage K tile [64 keys][D] -------------------------------------
    constexpr int KCH = kBK * D / 8;
#pragma unroll
    for (int c = tid; c < KCH; c += 256) {
      const int key = c / (D / 8), part = c - key * (D / 8);
      const int kpos = k0 + key;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kpos < seq_len) {
        const int phys = table[kpos >> 4];
        v = *reinterpret_cast<const uint4*>(kbase + (size_t)phys * block_elems +
                                            (kpos & 15) * D + part * 8);
      }
      *reinterpret_cast<uint4*>(&sK[key][part * 8]) = v;
    }
    // ---- stage V^T tile [D][64 keys] -------------------------------------
    constexpr int VCH = D * kBK / 8;
#pragma unroll
    for (int c = tid; c < VCH; c += 256) {
      const int bi = c / (2 * D);
      const int rem = c - bi * (2 * D);
      const int d = rem >> 1, half = rem & 1;
      const int kpos = k0 + bi * 16 + half * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kpos < seq_len) {
        const int phys = table[kpos >> 4];
        v = *reinterpret_cast<const uint4*>(vbase + (size_t)phys * block_elems + d * 16 +
                                            half * 8);
        if (kpos + 8 > seq_len) {
          // keys past the context may hold anything (even NaN): zero them
          uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (kpos + e >= seq_len) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          v = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      *reinterpret_cast<uint4*>(&sV[d][bi * 16 + half * 8]) = v;
    }
    __syncthreads();
    if (k0 > wpos_hi) continue;  // every row of this wave is before the tile

    // ---- S^T = K Q^T over two 32-key halves --------------------------------
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
#pragma unroll
      for (int st = 0; st < QSTEPS; ++st) {
        const bf16x8 a = as_bf16x8(
            *reinterpret_cast<const uint4*>(&sK[32 * kb + row][16 * st + 8 * kg]));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb], 0, 0, 0);
      }
    }
    float sv[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sv[16 * kb + j] = s[kb][j] * p.scale_log2;
    if (k0 + kBK - 1 > wpos_lo) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = k0 + 32 * kb + 8 * i + 4 * kg + j;
            if (key > pos) sv[16 * kb + 4 * i + j] = -INFINITY;
          }
    }
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mt = fmaxf(mt, sv[i]);
    mt = fmaxf(mt, shfl_xor(mt, 32));
    const float m_new = fmaxf(m, mt);  // finite: key 0 is in the first tile
    const float alpha = fast_exp2(m - m_new);
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      sv[i] = fast_exp2(sv[i] - m_new);
      rs += sv[i];
    }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= alpha;

    // ---- O^T += V^T P^T, four 16-key steps ----------------------------------
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const int kb = ps >> 1, ih = ps & 1;
      const float* pp = &sv[16 * kb + 8 * ih];
      const bf16x8 pf = as_bf16x8(make_uint4(pack_bf16x2(pp[0], pp[1]), pack_bf16x2(pp[2], pp[3]),
                                             pack_bf16x2(pp[4], pp[5]), pack_bf16x2(pp[6], pp[7])));
      const int base = 32 * kb + 16 * ih + 4 * kg;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint2 lo = *reinterpret_cast<const uint2*>(&sV[32 * db + row][base]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&sV[32 * db + row][base + 8]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lo, hi), pf, acc[db], 0, 0, 0);
      }
    }
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
  trace_before(K_PLAN, stream);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, a.qsl, a.num_seqs,
                     decode_max_q(G), prefill_tile_tokens(G), a.plan, a.plan_cap);
  trace_after(stream);
  trace_before(K_PREFILL, stream);
  hipLaunchKernelGGL((prefill_kernel<D, G>), dim3(a.plan_cap, a.hkv), dim3(256), 0, stream, p);
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
