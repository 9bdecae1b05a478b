// Merge of split-KV partials: the second reduction kernel of the split-KV
// method ("Inside the engine: kernels, CUDA graphs and the life of a
// request", section "Prefill has a full grid; decode at batch 1 has almost
// none").  Each split s reports its normalised output o_s and log-sum-exp
// lse_s; with M = max_s lse_s the merged result is
//   lse = M + ln sum_s e^(lse_s - M),   out = sum_s e^(lse_s - lse) o_s,
// and a split with lse_s = -inf (it saw no key) weighs nothing: its o_s is
// never read.
//
// One wave per (row, query head): the lanes first reduce the split lse
// values, park the per-split weights in LDS, then each lane accumulates its
// head_dim / 64 output elements over the splits (coalesced rows of o_s).
// When called from the attention entry point the kernel also gets
// query_start_loc and skips rows of requests that the matrix-core prefill
// kernel already finalised.
#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kMaxSplits = 256;

struct CombineParams {
  const float* po;
  const float* pl;
  int32_t splits, nt, hq;
  void* out;
  float* lse;
  int32_t out_bf16;
  const int32_t* qsl;  // nullable: row filter for mixed batches
  int32_t num_seqs, dq;
};

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int PER = D / 64;
  __shared__ float s_w[4][kMaxSplits];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x;
  const int h = blockIdx.y * 4 + wave;
  if (h >= p.hq) return;
  if (p.qsl != nullptr) {
    if (t >= p.qsl[p.num_seqs]) return;
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.qsl[mid] <= t) lo = mid; else hi = mid - 1;
    }
    if (p.qsl[lo + 1] - p.qsl[lo] > p.dq) return;
  }
  const size_t row = (size_t)t * p.hq + h;
  const size_t split_stride = (size_t)p.nt * p.hq;
  float M = -INFINITY;
  for (int s = lane; s < p.splits; s += 64) M = fmaxf(M, p.pl[s * split_stride + row]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, shfl_xor(M, o));
  const int d0 = lane * PER;
  if (M == -INFINITY) {
    // no split saw a key
    for (int k = 0; k < PER; ++k) {
      if (p.out_bf16) reinterpret_cast<uint16_t*>(p.out)[row * D + d0 + k] = 0x7fc0;
      else reinterpret_cast<float*>(p.out)[row * D + d0 + k] = __builtin_nanf("");
    }
    if (p.lse != nullptr && lane == 0) p.lse[row] = -INFINITY;
    return;
  }
  float sum = 0.f;
  for (int s = lane; s < p.splits; s += 64) {
    const float x = p.pl[s * split_stride + row];
    const float w = (x == -INFINITY) ? 0.f : fast_exp2((x - M) * kLog2e);
    s_w[wave][s] = w;
    sum += w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += shfl_xor(sum, o);
  const float inv = 1.f / sum;
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  // s_w is written and read by the same wave only
  __builtin_amdgcn_wave_barrier();
  for (int s = 0; s < p.splits; ++s) {
    const float w = s_w[wave][s];
    if (w == 0.f) continue;
    const float* src = p.po + (s * split_stride + row) * D + d0;
    if constexpr (PER == 2) {
      const float2 v = *reinterpret_cast<const float2*>(src);
      acc[0] += w * v.x;
      acc[1] += w * v.y;
    } else {
      acc[0] += w * src[0];
    }
  }
  if (p.out_bf16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(p.out) + row * D + d0;
    if constexpr (PER == 2) {
      *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      dst[0] = (uint16_t)f32_to_bf16_bits(acc[0] * inv);
    }
  } else {
    float* dst = reinterpret_cast<float*>(p.out) + row * D + d0;
#pragma unroll
    for (int k = 0; k < PER; ++k) dst[k] = acc[k] * inv;
  }
  if (p.lse != nullptr && lane == 0) p.lse[row] = M + fast_log2(sum) * kLn2;
}

}  // namespace

hipError_t launch_combine(const float* po, const float* pl, int32_t splits, int32_t nt,
                          int32_t hq, int32_t d, void* out, float* lse, int32_t out_bf16,
                          const int32_t* qsl, int32_t num_seqs, int32_t dq,
                          hipStream_t stream) {
  CombineParams p;
  p.po = po;
  p.pl = pl;
  p.splits = splits;
  p.nt = nt;
  p.hq = hq;
  p.out = out;
  p.lse = lse;
  p.out_bf16 = out_bf16;
  p.qsl = qsl;
  p.num_seqs = num_seqs;
  p.dq = dq;
  dim3 grid(nt, (hq + 3) / 4);
  trace_before(K_COMBINE, stream);
  if (d == 64) hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(256), 0, stream, p);
  trace_after(stream);
  return hipGetLastError();
}

}  // namespace pa
