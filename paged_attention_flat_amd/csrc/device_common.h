// Device-side helpers for the gfx950 kernels: vector types for the matrix
// cores, bf16 packing, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 round-to-nearest-even (NaN stays NaN), as raw bits.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Pack two floats into one dword of two bf16 (lo in the low half), round to
// nearest even: a single v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint2 lo, uint2 hi) {
  uint4 v = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return __builtin_bit_cast(bf16x8, v);
}

// Eight E4M3 codes (bytes 0..7 of v) to eight bf16, exactly (every E4M3
// value is a bf16 value): four v_cvt_scalef32_pk_bf16_fp8 at scale 1.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint2 v) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
  return bf16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// E4M3 codes of four values already divided by their scale: clamped to the
// largest finite magnitude (448; the conversion gives NaN past it), then
// rounded to nearest even by the hardware conversion.  Every NaN, whatever
// its sign, encodes as the one code 0x7F (the test is on the bits, so it
// holds in translation units built without NaN semantics).
__device__ __forceinline__ float e4m3_sat(float y) {
  return y > 448.f ? 448.f : (y < -448.f ? -448.f : y);
}
__device__ __forceinline__ bool is_nan_bits(float y) {
  return (__float_as_uint(y) & 0x7fffffffu) > 0x7f800000u;
}
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(a), e4m3_sat(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(c), e4m3_sat(d), w, true);
  uint32_t u = (uint32_t)w;
  if (is_nan_bits(a)) u = (u & 0xffffff00u) | 0x0000007fu;
  if (is_nan_bits(b)) u = (u & 0xffff00ffu) | 0x00007f00u;
  if (is_nan_bits(c)) u = (u & 0xff00ffffu) | 0x007f0000u;
  if (is_nan_bits(d)) u = (u & 0x00ffffffu) | 0x7f000000u;
  return u;
}
__device__ __forceinline__ uint8_t e4m3_code(float y) {
  if (is_nan_bits(y)) return 0x7f;
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(y), 0.f, 0, false) & 0xff);
}

// Cache fragments of eight elements: raw bits as loaded (16 bytes of bf16 or
// 8 bytes of E4M3 codes) and their bf16 operand form.
template <bool F8>
struct Frag8;
template <>
struct Frag8<false> {
  typedef uint16_t elem;
  typedef uint4 raw;
  static __device__ __forceinline__ uint4 bits(raw r) { return r; }
};
template <>
struct Frag8<true> {
  typedef uint8_t elem;
  typedef uint2 raw;
  static __device__ __forceinline__ uint4 bits(raw r) {
    return __builtin_bit_cast(uint4, e4m3x8_to_bf16x8(r));
  }
};

// Cross-lane exchange inside a wave64 (ds_bpermute based).
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// 16-byte load with the non-temporal cache policy (data read once per step)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// the same for 8 bytes
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 load_stream8(const uint2* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// max / sum of v over lanes i and i ^ 32 with one VALU lane-half swap
// (v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; given v twice, the two results hold v of lane i
// and of lane i ^ 32 in some order)
__device__ __forceinline__ float max_xor32(float v) {
  const uint32_t b = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const uint32_t b = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// the same over lanes i and i ^ 16 (v_permlane16_swap exchanges the odd
// 16-lane rows of its first operand with the even rows of its second)
__device__ __forceinline__ float max_xor16(float v) {
  const uint32_t b = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const uint32_t b = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// threadIdx.x as a value the compiler cannot treat as the same on every pass
// of a persistent loop: a work unit's per-thread address arithmetic then
// stays inside the unit instead of being hoisted out of the loop and kept
// live (in registers) across the other kind of unit.  (Kernels without such
// a loop use threadIdx.x itself, which the compiler may rematerialise.)
__device__ __forceinline__ int unit_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float fast_log2(float x) {
  return __builtin_amdgcn_logf(x);
}

// Most wave totals a work-group's scan passes through LDS (1024 threads).
constexpr int kScanParts = 16;

// Inclusive prefix sum of v over the NT threads of a work-group (NT a
// multiple of 64, at most 1024), in thread order; `total` receives the
// work-group's sum.  Shuffles inside each wave, then the wave totals through
// `part` (kScanParts ints of LDS): two barriers, where a scan through LDS
// alone takes 2 log2(NT).  Every thread of the work-group calls it; `part`
// may be reused as soon as it returns.
template <int NT>
__device__ __forceinline__ int block_scan(int v, int* part, int& total) {
  static_assert(NT % 64 == 0 && NT / 64 <= kScanParts, "one wave total per part");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) part[wave] = v;
  __syncthreads();
  int base = 0, sum = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int p = part[i];
    base += i < wave ? p : 0;
    sum += p;
  }
  __syncthreads();
  total = sum;
  return v + base;
}

}  // namespace pa
