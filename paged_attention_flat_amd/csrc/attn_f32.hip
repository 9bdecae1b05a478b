// fp32 attention for every row of a flat step (decode and prefill rows
// alike), with the same optional split of the key axis as the bf16 decode
// path.  This is the full-precision path: vector ALU arithmetic, online
// softmax ("Inside the engine: kernels, CUDA graphs and the life of a
// request", section "Never materialise the T x T matrix") over chunks of 256
// keys gathered through the block table.
//
// One work-group = (flat row, KV head, split).  The row's request is found by
// binary search over query_start_loc, so prefill and decode rows need no
// host-side classification.  Per chunk: each thread scores one key for all G
// query heads of the KV head, one wave per head turns scores into
// probabilities and updates (m, l), then every thread accumulates its share
// of the G x D outputs over the chunk.
#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

struct F32Params {
  const float* q;
  const float* kc;
  const float* vc;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* tables;
  int32_t num_seqs, hq, hkv, table_stride, splits, nt;
  float scale_log2;
  float* out;
  float* lse;
  float* part_out;
  float* part_lse;
};

constexpr int kChunk = 256;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += shfl_xor(v, o);
  return v;
}

template <int D, int G>
__global__ __launch_bounds__(256) void attn_f32_kernel(F32Params p) {
  constexpr int OUTS = (G * D + 255) / 256;  // outputs per thread
  __shared__ __align__(16) float sq[G][D];
  __shared__ float sp[G][kChunk];
  __shared__ float s_m[G], s_l[G], s_alpha[G];
  __shared__ int s_phys[kChunk / 16];

  const int t = blockIdx.x, kvh = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (t >= p.qsl[p.num_seqs]) return;
  int lo = 0, hi = p.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int q0 = p.qsl[b];
  const int q_len = p.qsl[b + 1] - q0;
  const int seq_len = p.seq_lens[b];
  const int pos = seq_len - q_len + (t - q0);
  const int nblocks = (seq_len + 15) >> 4;
  const int bps = (nblocks + p.splits - 1) / p.splits;
  const int key_lo = split * bps * 16;
  const int key_hi = min((split + 1) * bps * 16, pos + 1);

  for (int i = tid; i < G * D; i += 256) {
    const int gg = i / D, d = i - gg * D;
    sq[gg][d] = p.q[((size_t)t * p.hq + kvh * G + gg) * D + d];
  }
  if (tid < G) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }
  float acc[OUTS];
#pragma unroll
  for (int k = 0; k < OUTS; ++k) acc[k] = 0.f;

  const int32_t* table = p.tables + (size_t)b * p.table_stride;
  const size_t head_elems = 16 * D;
  const size_t block_elems = (size_t)p.hkv * head_elems;
  const float* kbase = p.kc + kvh * head_elems;
  const float* vbase = p.vc + kvh * head_elems;

  for (int c0 = key_lo; c0 < key_hi; c0 += kChunk) {
    __syncthreads();
    if (tid < kChunk / 16) {
      const int kp = c0 + tid * 16;
      s_phys[tid] = kp < key_hi ? table[kp >> 4] : 0;
    }
    __syncthreads();
    // scores of key c0 + tid for the G heads
    const int key = c0 + tid;
    if (key < key_hi) {
      const float* krow = kbase + (size_t)s_phys[tid >> 4] * block_elems + (key & 15) * D;
      float sc[G];
#pragma unroll
      for (int gg = 0; gg < G; ++gg) sc[gg] = 0.f;
      for (int d = 0; d < D; d += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(krow + d);
#pragma unroll
        for (int gg = 0; gg < G; ++gg)
          sc[gg] += sq[gg][d] * kv.x + sq[gg][d + 1] * kv.y + sq[gg][d + 2] * kv.z +
                    sq[gg][d + 3] * kv.w;
      }
#pragma unroll
      for (int gg = 0; gg < G; ++gg) sp[gg][tid] = sc[gg] * p.scale_log2;
    } else {
#pragma unroll
      for (int gg = 0; gg < G; ++gg) sp[gg][tid] = -INFINITY;
    }
    __syncthreads();
    // softmax update, one wave per head
    for (int gg = wave; gg < G; gg += 4) {
      float mx = -INFINITY;
      for (int j = lane; j < kChunk; j += 64) mx = fmaxf(mx, sp[gg][j]);
      mx = wave_max(mx);
      const float m_old = s_m[gg];
      const float m_new = fmaxf(m_old, mx);
      const float alpha = fast_exp2(m_old - m_new);
      float sum = 0.f;
      for (int j = lane; j < kChunk; j += 64) {
        const float e = fast_exp2(sp[gg][j] - m_new);
        sp[gg][j] = e;
        sum += e;
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        s_alpha[gg] = alpha;
        s_m[gg] = m_new;
        s_l[gg] = s_l[gg] * alpha + sum;
      }
    }
    __syncthreads();
    const int nk = min(kChunk, key_hi - c0);
#pragma unroll
    for (int k = 0; k < OUTS; ++k) {
      const int o = tid + 256 * k;
      if (o < G * D) {
        const int gg = o / D, d = o - gg * D;
        float x = acc[k] * s_alpha[gg];
        for (int j = 0; j < nk; ++j) {
          const float v = vbase[(size_t)s_phys[j >> 4] * block_elems + d * 16 + (j & 15)];
          x += sp[gg][j] * v;
        }
        acc[k] = x;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < OUTS; ++k) {
    const int o = tid + 256 * k;
    if (o >= G * D) continue;
    const int gg = o / D, d = o - gg * D;
    const int h = kvh * G + gg;
    const float L = s_l[gg], M = s_m[gg];
    if (p.splits == 1) {
      p.out[((size_t)t * p.hq + h) * D + d] = acc[k] / L;
      if (p.lse != nullptr && d == 0) p.lse[(size_t)t * p.hq + h] = (M + fast_log2(L)) * kLn2;
    } else {
      const bool empty = (L == 0.f);
      p.part_out[(((size_t)split * p.nt + t) * p.hq + h) * D + d] = empty ? 0.f : acc[k] / L;
      if (d == 0)
        p.part_lse[((size_t)split * p.nt + t) * p.hq + h] =
            empty ? -INFINITY : (M + fast_log2(L)) * kLn2;
    }
  }
}

template <int D, int G>
void launch_dg(const AttnArgs& a, hipStream_t stream) {
  F32Params p;
  p.q = (const float*)a.q;
  p.kc = (const float*)a.kc;
  p.vc = (const float*)a.vc;
  p.qsl = a.qsl;
  p.seq_lens = a.seq_lens;
  p.tables = a.tables;
  p.num_seqs = a.num_seqs;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.table_stride = a.table_stride;
  p.splits = a.splits;
  p.nt = a.num_tokens;
  p.scale_log2 = a.scale * kLog2e;
  p.out = (float*)a.out;
  p.lse = a.lse;
  p.part_out = a.part_out;
  p.part_lse = a.part_lse;
  trace_before(a.splits > 1 ? K_F32_ATTN_SPLIT : K_F32_ATTN, stream);
  hipLaunchKernelGGL((attn_f32_kernel<D, G>), dim3(a.num_tokens, a.hkv, a.splits), dim3(256),
                     0, stream, p);
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

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream) {
  if (a.d == 64) launch_d<64>(a, stream);
  else launch_d<128>(a, stream);
  return hipGetLastError();
}

}  // namespace pa
