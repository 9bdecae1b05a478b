// KV write: scatter the step's new K and V rows into the paged cache through
// slot_mapping ("Model execution", section "Flattening a step": the KV write
// puts each new token's K and V at slot block_id * block_size + offset).
//
// One work-group handles 16 consecutive flat tokens of one KV head
// (write_tokens: K rows copied in 16-byte pieces, V rows staged in LDS and
// written dim-major, so that they coalesce when the tokens fill consecutive
// slots of a block, the usual case for a prefill chunk).  The copy is a bit
// copy; the element type only fixes the width.
#include <type_traits>

#include "kv_write_body.h"

namespace pa {
namespace {

constexpr int kTok = kWriteTokens;

template <typename E>
__global__ __launch_bounds__(256) void kv_write_kernel(
    const E* __restrict__ key, const E* __restrict__ value, E* __restrict__ kc,
    E* __restrict__ vc, const int64_t* __restrict__ slots, int32_t nt,
    int32_t hkv, int32_t d, int64_t num_slots) {
  __shared__ __align__(16) E vrow[kTok][128 + 16 / sizeof(E)];
  __shared__ int64_t sslot[kTok];
  const int t0 = blockIdx.x * kTok;
  write_tokens<E>(key, value, kc, vc, slots, t0, min(kTok, nt - t0), blockIdx.y, hkv, d,
                  num_slots, vrow, sslot, threadIdx.x);
}

// FP8 (E4M3) cache: the same geometry with one byte per element.  Each
// value is divided by its KV head's scale (IEEE fp32 division), clamped to
// the largest finite E4M3 magnitude (448; the conversion would give NaN past
// it) and converted with round-to-nearest-even by the hardware instruction.
// Each thread quantises 8 consecutive dims of one token (one 8-byte K store);
// the V codes are staged in LDS and written dim-major like the 16-bit path.

template <typename E>
__device__ __forceinline__ float widen(E v);
template <>
__device__ __forceinline__ float widen<uint16_t>(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
template <>
__device__ __forceinline__ float widen<uint32_t>(uint32_t v) { return __uint_as_float(v); }

template <typename E>
__device__ __forceinline__ void write_tokens_fp8(const E* __restrict__ key,
                                                 const E* __restrict__ value,
                                                 uint8_t* __restrict__ kc,
                                                 uint8_t* __restrict__ vc,
                                                 const int64_t* __restrict__ slots, float ks,
                                                 float vs, int t0, int ntok, int h, int32_t hkv,
                                                 int32_t d, int64_t num_slots,
                                                 uint8_t (*vrow)[128 + 16], int64_t* sslot) {
  const int tid = threadIdx.x;
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

template <typename E>
__global__ __launch_bounds__(256) void kv_write_fp8_kernel(
    const E* __restrict__ key, const E* __restrict__ value, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, const int64_t* __restrict__ slots,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, int32_t nt,
    int32_t hkv, int32_t d, int64_t num_slots) {
  __shared__ __align__(16) uint8_t vrow[kTok][128 + 16];
  __shared__ int64_t sslot[kTok];
  const int t0 = blockIdx.x * kTok;
  const int h = blockIdx.y;
  write_tokens_fp8<E>(key, value, kc, vc, slots, k_scale[h], v_scale[h], t0,
                      min(kTok, nt - t0), h, hkv, d, num_slots, vrow, sslot);
}

// The KV write of the tokens of the matrix-core kernel's work list only: one
// work-group per (work item, KV head) writes the item's query tile (tq
// consecutive tokens of one request), 16 tokens at a time.  In a step that
// also has decode rows, the decode kernel writes those rows' tokens itself.
template <typename E, bool F8>
__global__ __launch_bounds__(256) void kv_write_plan_kernel(
    const E* __restrict__ key, const E* __restrict__ value, void* __restrict__ kc,
    void* __restrict__ vc, const int64_t* __restrict__ slots,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const int32_t* __restrict__ plan, const int32_t* __restrict__ qsl, int32_t tq,
    int32_t hkv, int32_t d, int64_t num_slots) {
  typedef typename std::conditional<F8, uint8_t, E>::type CE;
  __shared__ __align__(16) CE vrow[kTok][128 + 16 / sizeof(CE)];
  __shared__ int64_t sslot[kTok];
  const int item = blockIdx.x;
  if (item >= plan[0]) return;
  const int b = plan[1 + 2 * item], tile = plan[2 + 2 * item];
  const int q0 = qsl[b], q1 = qsl[b + 1];
  const int t_begin = q0 + tile * tq;
  const int t_end = min(q1, t_begin + tq);
  const int h = blockIdx.y;
  for (int t0 = t_begin; t0 < t_end; t0 += kTok) {
    if constexpr (F8)
      write_tokens_fp8<E>(key, value, (uint8_t*)kc, (uint8_t*)vc, slots, k_scale[h], v_scale[h],
                          t0, min(kTok, t_end - t0), h, hkv, d, num_slots, vrow, sslot);
    else
      write_tokens<E>(key, value, (E*)kc, (E*)vc, slots, t0, min(kTok, t_end - t0), h, hkv, d,
                      num_slots, vrow, sslot, threadIdx.x);
    __syncthreads();  // the staging is reused by the next 16 tokens
  }
}

// Rotary position embedding fused with the KV write.  Pairs are (i, i + d/2)
// of each head; row p of the cos/sin table holds cos of the d/2 angles, then
// their sin.  A work-group takes 16 tokens of one KV head: it rotates the new
// keys on their way into the cache (one read and one write of K), rotates the
// G query heads of that KV head in place, and writes V like kv_write.  Each
// thread owns 4 consecutive pairs of one row (two 4-element pieces, one per
// half of the head).  Arithmetic in fp32, one rounding to the element type.
template <typename E>
struct Piece4;  // four elements of E as one load / store
template <>
struct Piece4<uint16_t> {
  typedef uint2 T;
  // a read-once input row: non-temporal load
  static __device__ __forceinline__ T load(const uint16_t* p) {
    return load_stream8(reinterpret_cast<const uint2*>(p));
  }
  static __device__ __forceinline__ void get(T v, float* f) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
  }
  static __device__ __forceinline__ T put(const float* f) {
    return make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
  }
};
template <>
struct Piece4<uint32_t> {
  typedef uint4 T;
  static __device__ __forceinline__ T load(const uint32_t* p) {
    return load_stream16(reinterpret_cast<const uint4*>(p));
  }
  static __device__ __forceinline__ void get(T v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  static __device__ __forceinline__ T put(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};

// rotate the 4 pairs (lo[j], hi[j]) by the angles in c[j], s[j]
__device__ __forceinline__ void rotate4(float* lo, float* hi, const float4 c, const float4 s) {
  const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = lo[j], b = hi[j];
    lo[j] = a * cc[j] - b * ss[j];
    hi[j] = b * cc[j] + a * ss[j];
  }
}

template <typename E>
__global__ __launch_bounds__(256) void rope_kv_write_kernel(
    E* __restrict__ query, const E* __restrict__ key, const E* __restrict__ value,
    E* __restrict__ kc, E* __restrict__ vc, const int64_t* __restrict__ slots,
    const int64_t* __restrict__ positions, const float* __restrict__ cos_sin,
    int32_t max_position, int32_t nt, int32_t hq, int32_t hkv, int32_t d, int64_t num_slots) {
  typedef typename Piece4<E>::T P4;
  constexpr int kPad = 16 / sizeof(E);
  __shared__ __align__(16) E vrow[kTok][128 + kPad];
  __shared__ __align__(16) float scs[kTok][128];  // the tokens' cos | sin rows
  __shared__ int64_t sslot[kTok];
  __shared__ int spos[kTok];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTok;
  const int h = blockIdx.y;
  const int G = hq / hkv;
  const int ntok = min(kTok, nt - t0);
  if (tid < kTok) {
    int64_t s = -1;
    int p = -1;
    if (tid < ntok) {
      const int64_t pp = positions[t0 + tid];
      p = (pp >= 0 && pp < max_position) ? (int)pp : -1;  // outside the table: untouched
      s = slots[t0 + tid];
      if (s >= num_slots || p < 0) s = -1;
    }
    sslot[tid] = s;
    spos[tid] = p;
  }
  __syncthreads();
  // each token's cos / sin row is read from the table once per work-group
  // and serves its K row and the G query rows
  for (int c = tid; c < kTok * (d / 4); c += 256) {
    const int ti = c / (d / 4), part = c - ti * (d / 4);
    const int p = spos[ti];
    if (ti < ntok && p >= 0)
      *reinterpret_cast<float4*>(&scs[ti][4 * part]) =
          *reinterpret_cast<const float4*>(cos_sin + (size_t)p * d + 4 * part);
  }
  __syncthreads();
  const int half = d / 2, qpr = half / 4;  // 4-pair pieces per head row
  // K: rotate, write token-major into the cache
  for (int c = tid; c < kTok * qpr; c += 256) {
    const int ti = c / qpr, pc = c - ti * qpr;
    const int p = spos[ti];
    const int64_t s = sslot[ti];
    if (ti >= ntok || p < 0) continue;
    const size_t src = ((size_t)(t0 + ti) * hkv + h) * d + 4 * pc;
    float lo[4], hi[4];
    Piece4<E>::get(Piece4<E>::load(key + src), lo);
    Piece4<E>::get(Piece4<E>::load(key + src + half), hi);
    const float* row = &scs[ti][4 * pc];
    rotate4(lo, hi, *reinterpret_cast<const float4*>(row),
            *reinterpret_cast<const float4*>(row + half));
    if (s < 0) continue;
    const size_t blk = (size_t)(s >> 4), off = (size_t)(s & 15);
    E* kdst = kc + ((blk * hkv + h) * kTok + off) * d + 4 * pc;
    *reinterpret_cast<P4*>(kdst) = Piece4<E>::put(lo);
    *reinterpret_cast<P4*>(kdst + half) = Piece4<E>::put(hi);
  }
  // Q: the G query heads of this KV head, rotated in place
  for (int c = tid; c < kTok * G * qpr; c += 256) {
    const int ti = c / (G * qpr), rem = c - ti * (G * qpr);
    const int g = rem / qpr, pc = rem - g * qpr;
    const int p = spos[ti];
    if (ti >= ntok || p < 0) continue;
    E* qrow = query + ((size_t)(t0 + ti) * hq + h * G + g) * d + 4 * pc;
    float lo[4], hi[4];
    Piece4<E>::get(Piece4<E>::load(qrow), lo);
    Piece4<E>::get(Piece4<E>::load(qrow + half), hi);
    const float* row = &scs[ti][4 * pc];
    rotate4(lo, hi, *reinterpret_cast<const float4*>(row),
            *reinterpret_cast<const float4*>(row + half));
    *reinterpret_cast<P4*>(qrow) = Piece4<E>::put(lo);
    *reinterpret_cast<P4*>(qrow + half) = Piece4<E>::put(hi);
  }
  // V: staged in LDS, written dim-major (as kv_write)
  const int cpr = d * (int)sizeof(E) / 16;
  for (int c = tid; c < kTok * cpr; c += 256) {
    const int ti = c / cpr, part = c - ti * cpr;
    if (ti >= ntok) break;
    const size_t src = ((size_t)(t0 + ti) * hkv + h) * d;
    reinterpret_cast<uint4*>(&vrow[ti][0])[part] =
        load_stream16(reinterpret_cast<const uint4*>(value + src) + part);
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

hipError_t launch_rope_kv_write(void* query, const void* key, const void* value, void* kc,
                                void* vc, const int64_t* slots, const int64_t* positions,
                                const float* cos_sin, int32_t max_position, int32_t nt,
                                int32_t hq, int32_t hkv, int32_t d, int32_t esize,
                                int64_t num_blocks, hipStream_t stream) {
  dim3 grid((nt + kTok - 1) / kTok, hkv);
  trace_before(K_ROPE_KV_WRITE, stream);
  if (esize == 2) {
    hipLaunchKernelGGL(rope_kv_write_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       (uint16_t*)query, (const uint16_t*)key, (const uint16_t*)value,
                       (uint16_t*)kc, (uint16_t*)vc, slots, positions, cos_sin, max_position, nt,
                       hq, hkv, d, num_blocks * kTok);
  } else {
    hipLaunchKernelGGL(rope_kv_write_kernel<uint32_t>, grid, dim3(256), 0, stream,
                       (uint32_t*)query, (const uint32_t*)key, (const uint32_t*)value,
                       (uint32_t*)kc, (uint32_t*)vc, slots, positions, cos_sin, max_position, nt,
                       hq, hkv, d, num_blocks * kTok);
  }
  trace_after(stream);
  return hipGetLastError();
}

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

hipError_t launch_kv_write_plan(const AttnArgs& a, int32_t tq, hipStream_t stream) {
  dim3 grid(a.plan_cap, a.hkv);
  const int64_t num_slots = a.num_blocks * kTok;
  trace_before(a.cache_fp8 ? K_KV_WRITE_FP8 : K_KV_WRITE, stream);
  if (a.cache_fp8)
    hipLaunchKernelGGL((kv_write_plan_kernel<uint16_t, true>), grid, dim3(256), 0, stream,
                       (const uint16_t*)a.knew, (const uint16_t*)a.vnew, (void*)a.kc,
                       (void*)a.vc, a.slots, a.k_scale, a.v_scale, a.plan, a.qsl, tq, a.hkv, a.d,
                       num_slots);
  else
    hipLaunchKernelGGL((kv_write_plan_kernel<uint16_t, false>), grid, dim3(256), 0, stream,
                       (const uint16_t*)a.knew, (const uint16_t*)a.vnew, (void*)a.kc,
                       (void*)a.vc, a.slots, a.k_scale, a.v_scale, a.plan, a.qsl, tq, a.hkv, a.d,
                       num_slots);
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
