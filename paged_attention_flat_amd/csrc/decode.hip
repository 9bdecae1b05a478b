// Decode attention (bf16 cache, fp32 accumulation) for requests with few new
// tokens, with an optional split of the key axis.
//
// Method: "Inside the engine: kernels, CUDA graphs and the life of a request",
// sections "Never materialise the T x T matrix" (online softmax: running max m
// and denominator l, accumulator rescaled by e^(m_old - m_new)), "Prefill has a
// full grid; decode at batch 1 has almost none" (split-KV partials over block
// ranges, merged by a second kernel) and "Attention over a block table, not a
// contiguous tensor" (keys and values gathered through the block table).
//
// MI355X design.  One work-group = (request, KV head, split); its four waves
// walk disjoint pairs of 16-token blocks of the split's range and each keeps
// its own (m, l, acc) state, merged through LDS at the end.  All query heads
// of the KV head (group size G) and up to 16 / G new tokens are packed as the
// 16 columns of a 16x16x32 bf16 MFMA, so every K/V byte is read from HBM once
// per step:
//   S^T[key][col] = K[key][:] . Q[col][:]    A = K rows (16-byte loads),
//                                            B = Q (held in registers)
//   O^T[d][col]  += V^T[d][keys] P[keys][col] A = V (dim-major cache block:
//                                            8-byte loads of 4 keys),
//                                            B = P straight from the S^T
//                                            accumulator, no shuffles.
// A pair of blocks gives the 32-key contraction of the P.V product: MFMA
// slots 0-3 of a lane's key group carry keys 4g..4g+3 of the first block and
// slots 4-7 the same keys of the second, the order the S^T accumulator
// produces them in.  Row maxima use two cross-lane exchanges; exponentials
// are base 2 on log2(e)-prescaled scores.
#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* tables;
  int32_t hq, hkv, table_stride, splits, nt;
  float scale_log2;
  uint16_t* out;
  float* lse;
  float* part_out;
  float* part_lse;
};

constexpr int kWaves = 4;

template <int D, int G>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeParams p) {
  constexpr int DQ = 16 / G;       // new tokens per request packed in the columns
  constexpr int KSTEPS = D / 32;   // MFMA steps over head_dim for S^T
  constexpr int DB = D / 16;       // 16-row blocks of O^T
  constexpr int ACC_STRIDE = D + 4;

  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_acc[kWaves][16][ACC_STRIDE];

  const int b = blockIdx.x, kvh = blockIdx.y, split = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;

  const int q0 = p.qsl[b];
  const int q_len = p.qsl[b + 1] - q0;
  if (q_len <= 0 || q_len > DQ) return;  // empty request or a prefill row set
  const int seq_len = p.seq_lens[b];
  const int ctx = seq_len - q_len;
  const int nblocks = (seq_len + 15) >> 4;
  int bps = (nblocks + p.splits - 1) / p.splits;
  bps = (bps + 1) & ~1;  // whole pairs per split
  const int blk_lo = split * bps;
  const int blk_hi = min(nblocks, blk_lo + bps);

  const int qi = col / G, g = col - (col / G) * G;
  const bool col_valid = qi < q_len;
  const int qpos = ctx + min(qi, q_len - 1);

  // Q as the B operand: lane (col, kg) holds d = 32*st + 8*kg .. +8
  bf16x8 qf[KSTEPS];
  if (col_valid) {
    const uint16_t* qrow = p.q + ((size_t)(q0 + qi) * p.hq + kvh * G + g) * D;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
      qf[st] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 32 * st + 8 * kg));
  } else {
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) qf[st] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  const int32_t* table = p.tables + (size_t)b * p.table_stride;
  const size_t head_elems = 16 * D;
  const size_t block_elems = (size_t)p.hkv * head_elems;
  const uint16_t* kbase = p.kc + kvh * head_elems;
  const uint16_t* vbase = p.vc + kvh * head_elems;

  float m = -INFINITY, l = 0.f;
  f32x4 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int npairs = blk_hi > blk_lo ? (blk_hi - blk_lo + 1) >> 1 : 0;
  for (int pr = wave; pr < npairs; pr += kWaves) {
    const int j0 = blk_lo + 2 * pr;
    const bool has1 = j0 + 1 < blk_hi;
    const int phys0 = table[j0];
    const int phys1 = has1 ? table[j0 + 1] : phys0;
    const uint16_t* k0 = kbase + (size_t)phys0 * block_elems + col * D + 8 * kg;
    const uint16_t* k1 = kbase + (size_t)phys1 * block_elems + col * D + 8 * kg;
    const uint16_t* v0 = vbase + (size_t)phys0 * block_elems + col * 16 + 4 * kg;
    const uint16_t* v1 = vbase + (size_t)phys1 * block_elems + col * 16 + 4 * kg;

    bf16x8 ka[KSTEPS], kb[KSTEPS];
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      ka[st] = as_bf16x8(*reinterpret_cast<const uint4*>(k0 + 32 * st));
      kb[st] = as_bf16x8(*reinterpret_cast<const uint4*>(k1 + 32 * st));
    }
    uint2 va[DB], vb[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      va[db] = *reinterpret_cast<const uint2*>(v0 + db * 16 * 16);
      vb[db] = *reinterpret_cast<const uint2*>(v1 + db * 16 * 16);
    }

    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[st], qf[st], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[st], qf[st], s1, 0, 0, 0);
    }

    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = s0[i] * p.scale_log2;
      sv[4 + i] = s1[i] * p.scale_log2;
    }
    const int kp0 = 16 * j0 + 4 * kg;  // position of sv[0]
    if (16 * j0 + 31 > ctx) {
      // the pair reaches past the first new token: causal mask per column,
      // and keys past the context (tail of the last block, or a missing
      // second block) must not reach the P.V product even as NaN * 0
      uint32_t m0x = 0xffffffffu, m0y = 0xffffffffu, m1x = 0xffffffffu, m1y = 0xffffffffu;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pa = kp0 + i, pb = kp0 + 16 + i;
        if (pa > qpos) sv[i] = -INFINITY;
        if (!has1 || pb > qpos) sv[4 + i] = -INFINITY;
        const uint32_t half = (i & 1) ? 0xffff0000u : 0x0000ffffu;
        if (pa >= seq_len) { if (i < 2) m0x &= ~half; else m0y &= ~half; }
        if (!has1 || pb >= seq_len) { if (i < 2) m1x &= ~half; else m1y &= ~half; }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        va[db].x &= m0x; va[db].y &= m0y;
        vb[db].x &= m1x; vb[db].y &= m1y;
      }
    }

    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
    mt = fmaxf(mt, shfl_xor(mt, 16));
    mt = fmaxf(mt, shfl_xor(mt, 32));
    const float m_new = fmaxf(m, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float pv[8], rs = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = fast_exp2(sv[i] - m_use);
      rs += pv[i];
    }
    l = l * alpha + rs;
    m = m_new;

    const uint4 pbits = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                   pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
    const bf16x8 pf = as_bf16x8(pbits);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] *= alpha;
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va[db], vb[db]), pf,
                                                        acc[db], 0, 0, 0);
    }
  }

  // per-column denominator: sum the four key groups of the wave
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (kg == 0) {
    s_m[wave][col] = m;
    s_l[wave][col] = l;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_acc[wave][col][16 * db + 4 * kg + i] = acc[db][i];
  __syncthreads();

  // merge the waves: thread -> (column, run of D/16 dims)
  constexpr int RUN = D / 16;
  const int c = threadIdx.x >> 4;
  const int d0 = (threadIdx.x & 15) * RUN;
  const int cqi = c / G, cg = c - (c / G) * G;
  if (cqi >= q_len) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][c]);
  float wgt[kWaves], L = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    wgt[w] = (s_m[w][c] == -INFINITY) ? 0.f : fast_exp2(s_m[w][c] - M);
    L += wgt[w] * s_l[w][c];
  }
  float o[RUN];
#pragma unroll
  for (int k = 0; k < RUN; ++k) {
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) x += wgt[w] * s_acc[w][c][d0 + k];
    o[k] = x;
  }
  const int t = q0 + cqi;
  const int h = kvh * G + cg;
  if (p.splits == 1) {
    const float inv = 1.f / L;
    uint32_t packed[RUN / 2];
#pragma unroll
    for (int k = 0; k < RUN / 2; ++k) packed[k] = pack_bf16x2(o[2 * k] * inv, o[2 * k + 1] * inv);
    uint16_t* dst = p.out + ((size_t)t * p.hq + h) * D + d0;
    if constexpr (RUN == 8) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    } else {
      *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
    }
    if (p.lse != nullptr && d0 == 0) p.lse[(size_t)t * p.hq + h] = (M + fast_log2(L)) * kLn2;
  } else {
    const bool empty = (L == 0.f);
    const float inv = empty ? 0.f : 1.f / L;
    float* dst = p.part_out + (((size_t)split * p.nt + t) * p.hq + h) * D + d0;
#pragma unroll
    for (int k = 0; k < RUN; k += 4)
      *reinterpret_cast<float4*>(dst + k) =
          make_float4(o[k] * inv, o[k + 1] * inv, o[k + 2] * inv, o[k + 3] * inv);
    if (d0 == 0)
      p.part_lse[((size_t)split * p.nt + t) * p.hq + h] =
          empty ? -INFINITY : (M + fast_log2(L)) * kLn2;
  }
}

template <int D, int G>
void launch_dg(const AttnArgs& a, hipStream_t stream) {
  DecodeParams p;
  p.q = (const uint16_t*)a.q;
  p.kc = (const uint16_t*)a.kc;
  p.vc = (const uint16_t*)a.vc;
  p.qsl = a.qsl;
  p.seq_lens = a.seq_lens;
  p.tables = a.tables;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.table_stride = a.table_stride;
  p.splits = a.splits;
  p.nt = a.num_tokens;
  p.scale_log2 = a.scale * kLog2e;
  p.out = (uint16_t*)a.out;
  p.lse = a.lse;
  p.part_out = a.part_out;
  p.part_lse = a.part_lse;
  dim3 grid(a.num_seqs, a.hkv, a.splits);
  trace_before(a.splits > 1 ? K_DECODE_SPLIT : K_DECODE, stream);
  hipLaunchKernelGGL((decode_kernel<D, G>), grid, dim3(256), 0, stream, p);
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

hipError_t launch_decode_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.d == 64) launch_d<64>(a, stream);
  else launch_d<128>(a, stream);
  return hipGetLastError();
}

}  // namespace pa
