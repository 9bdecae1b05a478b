// KV write: scatter the step's new K and V rows into the paged cache through
// slot_mapping ("Model execution", section "Flattening a step": the KV write
// puts each new token's K and V at slot block_id * block_size + offset).
//
// One work-group handles 16 consecutive flat tokens of one KV head.  The K
// row of a token is a contiguous run in the token-major K block, copied in
// 16-byte pieces.  The V block is dim-major, so the 16 V rows are first staged
// in LDS and then written column by column: lanes that differ in the token
// index write neighbouring offsets of one dimension, which coalesce when the
// tokens fill consecutive slots of a block (the usual case for a prefill
// chunk).  The copy is a bit copy; the element type only fixes the width.
#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kTok = 16;

template <typename E>
__global__ __launch_bounds__(256) void kv_write_kernel(
    const E* __restrict__ key, const E* __restrict__ value, E* __restrict__ kc,
    E* __restrict__ vc, const int64_t* __restrict__ slots, int32_t nt,
    int32_t hkv, int32_t d, int64_t num_slots) {
  constexpr int kPad = 16 / sizeof(E);  // keeps LDS rows 16-byte aligned
  __shared__ __align__(16) E vrow[kTok][128 + kPad];
  __shared__ int64_t sslot[kTok];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTok;
  const int h = blockIdx.y;
  const int ntok = min(kTok, nt - t0);

  // The K/V loads do not depend on the slot, so they are issued together with
  // the slot load (one memory round trip before the stores).
  const int cpr = d * (int)sizeof(E) / 16;  // 16-byte pieces per row
  for (int c = tid; c < kTok * cpr; c += 256) {
    const int ti = c / cpr, part = c - ti * cpr;
    if (ti >= ntok) break;
    int64_t s = slots[t0 + ti];
    if (s >= num_slots) s = -1;  // out of the pool: dropped like a padded token
    const size_t src = ((size_t)(t0 + ti) * hkv + h) * d;
    const uint4 kv = reinterpret_cast<const uint4*>(key + src)[part];
    const uint4 vv = reinterpret_cast<const uint4*>(value + src)[part];
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

// FP8 (E4M3) cache: the same geometry with one byte per element.  Each
// value is divided by its KV head's scale (IEEE fp32 division), clamped to
// the largest finite E4M3 magnitude (448; the conversion would give NaN past
// it) and converted with round-to-nearest-even by the hardware instruction.
// Each thread quantises 8 consecutive dims of one token (one 8-byte K store);
// the V codes are staged in LDS and written dim-major like the 16-bit path.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  auto sat = [](float y) { return y > 448.f ? 448.f : (y < -448.f ? -448.f : y); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
  return (uint32_t)w;
}

template <typename E>
__device__ __forceinline__ float widen(E v);
template <>
__device__ __forceinline__ float widen<uint16_t>(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
template <>
__device__ __forceinline__ float widen<uint32_t>(uint32_t v) { return __uint_as_float(v); }

template <typename E>
__global__ __launch_bounds__(256) void kv_write_fp8_kernel(
    const E* __restrict__ key, const E* __restrict__ value, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, const int64_t* __restrict__ slots,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, int32_t nt,
    int32_t hkv, int32_t d, int64_t num_slots) {
  __shared__ __align__(16) uint8_t vrow[kTok][128 + 16];
  __shared__ int64_t sslot[kTok];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTok;
  const int h = blockIdx.y;
  const int ntok = min(kTok, nt - t0);
  const float ks = k_scale[h], vs = v_scale[h];
  const int cpr = d / 8;  // 8-element pieces per row
  for (int c = tid; c < kTok * cpr; c += 256) {
    const int ti = c / cpr, part = c - ti * cpr;
    if (ti >= ntok) break;
    int64_t s = slots[t0 + ti];
    if (s >= num_slots) s = -1;  // out of the pool: dropped like a padded token
    const size_t src = ((size_t)(t0 + ti) * hkv + h) * d + part * 8;
    float kf[8], vf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] = widen<E>(key[src + e]) / ks;
      vf[e] = widen<E>(value[src + e]) / vs;
    }
    if (part == 0) sslot[ti] = s;
    const uint2 vq = make_uint2(e4m3_pack4(vf[0], vf[1], vf[2], vf[3]),
                                e4m3_pack4(vf[4], vf[5], vf[6], vf[7]));
    *reinterpret_cast<uint2*>(&vrow[ti][part * 8]) = vq;
    if (s < 0) continue;
    const size_t blk = (size_t)(s >> 4), off = (size_t)(s & 15);
    uint8_t* kdst = kc + ((blk * hkv + h) * kTok + off) * d + part * 8;
    *reinterpret_cast<uint2*>(kdst) = make_uint2(e4m3_pack4(kf[0], kf[1], kf[2], kf[3]),
                                                 e4m3_pack4(kf[4], kf[5], kf[6], kf[7]));
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

}  // namespace

hipError_t launch_kv_write_fp8(const void* key, const void* value, void* kc, void* vc,
                               const int64_t* slots, const float* k_scale,
                               const float* v_scale, int32_t nt, int32_t hkv, int32_t d,
                               int32_t esize, int64_t num_blocks, hipStream_t stream) {
  dim3 grid((nt + kTok - 1) / kTok, hkv);
  trace_before(K_KV_WRITE_FP8, stream);
  if (esize == 2) {
    hipLaunchKernelGGL(kv_write_fp8_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       (const uint16_t*)key, (const uint16_t*)value, (uint8_t*)kc, (uint8_t*)vc,
                       slots, k_scale, v_scale, nt, hkv, d, num_blocks * kTok);
  } else {
    hipLaunchKernelGGL(kv_write_fp8_kernel<uint32_t>, grid, dim3(256), 0, stream,
                       (const uint32_t*)key, (const uint32_t*)value, (uint8_t*)kc, (uint8_t*)vc,
                       slots, k_scale, v_scale, nt, hkv, d, num_blocks * kTok);
  }
  trace_after(stream);
  return hipGetLastError();
}

hipError_t launch_kv_write(const void* key, const void* value, void* kc, void* vc,
                           const int64_t* slots, int32_t nt, int32_t hkv,
                           int32_t d, int32_t esize, int64_t num_blocks, hipStream_t stream) {
  dim3 grid((nt + kTok - 1) / kTok, hkv);
  trace_before(K_KV_WRITE, stream);
  if (esize == 2) {
    hipLaunchKernelGGL(kv_write_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       (const uint16_t*)key, (const uint16_t*)value, (uint16_t*)kc,
                       (uint16_t*)vc, slots, nt, hkv, d, num_blocks * kTok);
  } else {
    hipLaunchKernelGGL(kv_write_kernel<uint32_t>, grid, dim3(256), 0, stream,
                       (const uint32_t*)key, (const uint32_t*)value, (uint32_t*)kc,
                       (uint32_t*)vc, slots, nt, hkv, d, num_blocks * kTok);
  }
  trace_after(stream);
  return hipGetLastError();
}

}  // namespace pa
