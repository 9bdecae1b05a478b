// Merge of split-KV partials: the second reduction kernel of the split-KV
// method ("Inside the engine: kernels, CUDA graphs and the life of a
// request", section "Prefill has a full grid; decode at batch 1 has almost
// none").  Each split s reports its normalised output o_s and log-sum-exp
// lse_s; with M = max_s lse_s the merged result is
//   lse = M + ln sum_s e^(lse_s - M),   out = sum_s e^(lse_s - lse) o_s,
// and a split with lse_s = -inf (it saw no key) weighs nothing: its o_s is
// never read.
//
// One work-group per (row, query head).  Its 256 threads first reduce the
// split lse values (one split per thread), then split the sum over o_s as
// (group of splits) x (4 consecutive dims): every thread has several
// independent 16-byte loads in flight, and the groups are folded through LDS.
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
  constexpr int QUADS = D / 4;          // float4 columns of a row
  constexpr int GROUPS = 256 / QUADS;   // split groups (8 for D=128, 16 for D=64)
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[8];
  __shared__ float4 s_acc[GROUPS][QUADS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x / p.hq;
  const int h = blockIdx.x - t * p.hq;
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

  const float x = tid < p.splits ? p.pl[tid * split_stride + row] : -INFINITY;
  float M = x;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, shfl_xor(M, o));
  if (lane == 0) s_red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  if (M == -INFINITY) {
    // no split saw a key
    for (int d = tid; d < D; d += 256) {
      if (p.out_bf16) reinterpret_cast<uint16_t*>(p.out)[row * D + d] = 0x7fc0;
      else reinterpret_cast<float*>(p.out)[row * D + d] = __builtin_nanf("");
    }
    if (p.lse != nullptr && tid == 0) p.lse[row] = -INFINITY;
    return;
  }
  const float w = (x == -INFINITY) ? 0.f : fast_exp2((x - M) * kLog2e);
  if (tid < kMaxSplits) s_w[tid] = w;
  float sum = w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += shfl_xor(sum, o);
  if (lane == 0) s_red[4 + wave] = sum;
  __syncthreads();
  sum = (s_red[4] + s_red[5]) + (s_red[6] + s_red[7]);

  const int quad = tid % QUADS, grp = tid / QUADS;
  const float* base = p.po + row * D + quad * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = grp; s < p.splits; s += GROUPS) {
    const float ws = s_w[s];
    if (ws == 0.f) continue;
    const float4 v = *reinterpret_cast<const float4*>(base + s * split_stride * D);
    acc.x += ws * v.x;
    acc.y += ws * v.y;
    acc.z += ws * v.z;
    acc.w += ws * v.w;
  }
  s_acc[grp][quad] = acc;
  __syncthreads();
  if (tid < QUADS) {
    float4 r = s_acc[0][tid];
#pragma unroll
    for (int g = 1; g < GROUPS; ++g) {
      const float4 v = s_acc[g][tid];
      r.x += v.x;
      r.y += v.y;
      r.z += v.z;
      r.w += v.w;
    }
    const float inv = 1.f / sum;
    if (p.out_bf16) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(p.out) + row * D + tid * 4;
      *reinterpret_cast<uint2*>(dst) =
          make_uint2(pack_bf16x2(r.x * inv, r.y * inv), pack_bf16x2(r.z * inv, r.w * inv));
    } else {
      float* dst = reinterpret_cast<float*>(p.out) + row * D + tid * 4;
      *reinterpret_cast<float4*>(dst) = make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
    }
    if (p.lse != nullptr && tid == 0) p.lse[row] = M + fast_log2(sum) * kLn2;
  }
}

// Zero fill for workspace initialisation (a kernel rather than a memset, so a
// captured HIP graph holds only kernel nodes).
__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, size_t n16,
                                                   uint8_t* __restrict__ tail, int ntail) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const int ntail = (int)(bytes - n16 * 16);
  const size_t blocks = (n16 + 255) / 256;
  trace_before(K_ZERO, stream);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, stream,
                     (uint4*)ptr, n16, (uint8_t*)ptr + n16 * 16, ntail);
  trace_after(stream);
  return hipGetLastError();
}

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
  dim3 grid(nt * hq);
  trace_before(K_COMBINE, stream);
  if (d == 64) hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(256), 0, stream, p);
  trace_after(stream);
  return hipGetLastError();
}

}  // namespace pa
