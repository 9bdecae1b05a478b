// Prefill attention body shared by the matrix-core kernel and the mixed
// prefill + decode kernel: the per-unit computation of a (work item, KV head)
// unit, its parameters and its shared memory.  The method and the MI355X
// design are described in prefill.hip.
#pragma once

#include "device_common.h"
#include "pa_internal.h"

namespace pa {

struct PrefillParams {
  const uint16_t* q;
  const void* kc;         // bf16 elements, or E4M3 codes (F8 kernels)
  const void* vc;
  const float* k_scale;   // F8 kernels: per-KV-head dequantisation scales
  const float* v_scale;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* tables;
  const int32_t* plan;
  int32_t hq, hkv, table_stride;
  float scale_log2;
  uint16_t* out;
  float* lse;
  // shared-prefix (cascade) stage: gathered decode rows of the sharers
  const int32_t* casc_count;  // [1] rows gathered
  const int32_t* vtok;        // [rows] flat token of each gathered row
  const int32_t* vpos;        // [rows] its position
  const int32_t* pre_blocks;  // the shared prefix's physical blocks
  int32_t pre_tokens;         // 16 * number of prefix blocks
  int32_t pre_splits;         // key ranges of the prefix (one partial each)
  int32_t pre_chunk;          // keys per range (a multiple of the key tile)
  int32_t pre_rows;           // row capacity of one range's partial arrays
  float* pre_out;             // [splits][rows][hq][D] fp32 normalised partials
  float* pre_lse;             // [splits][rows][hq] natural-log lse (-inf: no key)
};

constexpr int kKPad = 8;    // bf16 padding per K row in LDS
constexpr int kVPad = 8;    // bf16 padding per V^T row in LDS
constexpr float kLazy = 8.f;  // base-2 headroom before the running max moves
constexpr int kTabWin = 512;  // block-table entries held in LDS (8192 keys)
#ifndef PA_PREFILL_KEYS
#define PA_PREFILL_KEYS 64    // keys per K/V tile
#endif

// position of key k (0..15) of a 16-key group in the V^T tile
__device__ __forceinline__ int vperm(int k) {
  return (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// The matrix-core kernel's view of one call's arguments (host side; the
// shared-prefix fields are set by the prefix stage's launcher).
inline PrefillParams make_prefill_params(const AttnArgs& a) {
  PrefillParams p = {};
  p.q = (const uint16_t*)a.q;
  p.kc = a.kc;
  p.vc = a.vc;
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
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
  return p;
}

// CASC: the prefix stage of shared-prefix attention -- work-group tiles are
// consecutive gathered rows (decode tokens of the sharers, each with its own
// position), keys are the shared prefix blocks, and the result is a partial
// (normalised fp32 output and lse) merged later by the decode kernel.
// Shared memory of one prefill work-group: K tiles (double-buffered), V^T
// tiles (triple-buffered) and the block-table window.
template <int D, int kBK>
struct PrefillSmem {
  __align__(16) uint16_t sK[2][kBK][D + kKPad];
  __align__(16) uint16_t sV[3][D][kBK + kVPad];
  int s_tab[kTabWin];
};

// One prefill work unit = bx: (work item, KV head), KV head fastest (CASC:
// (row tile, prefix key range, KV head)), computed by the NW waves of the
// calling work-group (tid: the thread's index in it).  Every exit is
// work-group uniform.
template <int D, int G, int NW, int RG, int kBK, bool F8, bool CASC>
__device__ __forceinline__ void prefill_unit(const PrefillParams& p, int bx,
                                             PrefillSmem<D, kBK>& sm, const int tid) {
  typedef typename Frag8<F8>::elem CT;
  typedef typename Frag8<F8>::raw RT;
  constexpr int KB = kBK / 32;            // 32-key halves per tile
  constexpr int PS = kBK / 16;            // 16-key P.V steps per tile
  constexpr int NT = 64 * NW;             // threads
  constexpr int WROWS = 32 * RG;          // query rows per wave
  constexpr int TQ = WROWS * NW / G;      // tokens per work-group
  constexpr int QSTEPS = D / 16;          // MFMA k-steps over head_dim
  constexpr int DB = D / 32;              // 32-row blocks of O^T
  constexpr int KCH = kBK * D / 8 / NT;   // 16-byte K chunks per thread per tile
  constexpr int VCH = D * kBK / 8 / NT;   // 16-byte V chunks per thread per tile
  uint16_t (&sK)[2][kBK][D + kKPad] = sm.sK;
  uint16_t (&sV)[3][D][kBK + kVPad] = sm.sV;
  int (&s_tab)[kTabWin] = sm.s_tab;

  const int kvh = bx % p.hkv;
  const int item = bx / p.hkv;
  int b = 0, tile, q0, q_len, seq_len, ctx;
  int kbeg = 0, ksplit = 0;
  if constexpr (CASC) {
    // work-group = (row tile, prefix key range, KV head)
    ksplit = item % p.pre_splits;
    tile = item / p.pre_splits;
    kbeg = ksplit * p.pre_chunk;
    q_len = p.casc_count[0];  // rows gathered
    if (tile * TQ >= q_len) return;
    q0 = 0;
    seq_len = p.pre_tokens;
    ctx = 0;
  } else {
    if (item >= p.plan[0]) return;
    b = p.plan[1 + 2 * item];
    tile = p.plan[2 + 2 * item];
    q0 = p.qsl[b];
    q_len = p.qsl[b + 1] - q0;
    seq_len = p.seq_lens[b];
    ctx = seq_len - q_len;
  }
  const int lane = tid & 63, wave = tid >> 6;
  const int row = lane & 31, kg = lane >> 5;
  const int tok0 = tile * TQ;

  // row group rg of this wave: work-group rows WROWS*wave + 32*rg + row,
  // token-major over the G query heads of the KV head
  int tokr[RG], gr[RG], pos[RG];
  bool valid[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int r = WROWS * wave + 32 * rg + row;
    tokr[rg] = tok0 + r / G;
    gr[rg] = r - (r / G) * G;
    valid[rg] = tokr[rg] < q_len;
    // CASC: a row sees the prefix up to its own position; keys past the
    // prefix (zero-filled in the last tile) are masked like later positions
    if constexpr (CASC) pos[rg] = min(p.vpos[min(tokr[rg], q_len - 1)], seq_len - 1);
    else pos[rg] = ctx + min(tokr[rg], q_len - 1);
  }
  // smallest position among the wave's rows: a tile needs the per-row causal
  // mask only where it reaches past it.  Rows are token-major, so the wave's
  // first row has it; CASC rows carry unrelated positions: a wave minimum.
  int wpos_lo;
  if constexpr (CASC) {
    int mn = pos[0];
#pragma unroll
    for (int rg = 1; rg < RG; ++rg) mn = min(mn, pos[rg]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mn = min(mn, __shfl_xor(mn, off, 64));
    wpos_lo = mn;
  } else {
    wpos_lo = ctx + min(tok0 + (WROWS * wave) / G, q_len - 1);
  }
  const int kend = CASC ? min(seq_len, kbeg + p.pre_chunk)
                        : ctx + min(tok0 + TQ, q_len);  // one past the last key

  bf16x8 qf[RG][QSTEPS];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    if (valid[rg]) {
      const size_t qtok = CASC ? (size_t)p.vtok[tokr[rg]] : (size_t)(q0 + tokr[rg]);
      const uint16_t* qrow = p.q + (qtok * p.hq + kvh * G + gr[rg]) * D + 8 * kg;
#pragma unroll
      for (int st = 0; st < QSTEPS; ++st)
        qf[rg][st] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 16 * st));
    } else {
#pragma unroll
      for (int st = 0; st < QSTEPS; ++st) qf[rg][st] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }

  const int32_t* table = CASC ? p.pre_blocks : p.tables + (size_t)b * p.table_stride;
  const size_t head_elems = 16 * D;
  const size_t block_elems = (size_t)p.hkv * head_elems;
  // block ids are non-negative and a block holds < 2^32 elements: one
  // 32 x 32 -> 64-bit multiply-add per block instead of a signed 64-bit product
  const uint32_t block_elems32 = (uint32_t)block_elems;
  auto blk_off = [&](int id) -> uint64_t { return (uint64_t)(uint32_t)id * block_elems32; };
  const CT* kbase = static_cast<const CT*>(p.kc) + kvh * head_elems;
  const CT* vbase = static_cast<const CT*>(p.vc) + kvh * head_elems;
  // E4M3 cache: K's scale folds into the score scale, V's into the output;
  // the codes become bf16 exactly when a tile is staged into LDS
  const float scale_log2 = F8 ? p.scale_log2 * p.k_scale[kvh] : p.scale_log2;
  const float v_scale = F8 ? p.v_scale[kvh] : 1.f;

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
  int tab_base = (kbeg >> 4) / kTabWin * kTabWin;
  RT kr[KCH], vr[VCH];
  auto gload = [&](int k0) {
    const int tb = (k0 >> 4) - tab_base;
    if (k0 + kBK <= seq_len) {
      // whole tile inside the context: no per-key checks
#pragma unroll
      for (int i = 0; i < KCH; ++i)
        kr[i] = *reinterpret_cast<const RT*>(kbase + blk_off(s_tab[tb + k_blk[i]]) +
                                              k_src[i]);
#pragma unroll
      for (int i = 0; i < VCH; ++i)
        vr[i] = *reinterpret_cast<const RT*>(vbase + blk_off(s_tab[tb + v_blk[i]]) +
                                              v_src[i]);
      return;
    }
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int kpos = k0 + (k_src[i] / D) + 16 * k_blk[i];
      RT v = {};
      if (kpos < seq_len)
        v = *reinterpret_cast<const RT*>(kbase + blk_off(s_tab[tb + k_blk[i]]) +
                                         k_src[i]);
      kr[i] = v;
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int kpos = k0 + v_key[i];
      RT v = {};
      if (kpos < seq_len) {
        v = *reinterpret_cast<const RT*>(vbase + blk_off(s_tab[tb + v_blk[i]]) +
                                         v_src[i]);
        if (kpos + 8 > seq_len) {
          // keys past the context may hold anything (even NaN): zero them
          if constexpr (F8) {
            uint32_t w[2] = {v.x, v.y};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (kpos + e >= seq_len) w[e >> 2] &= ~(0xffu << (8 * (e & 3)));  // code 0 = +0
            v = make_uint2(w[0], w[1]);
          } else {
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (kpos + e >= seq_len) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
            v = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
      }
      vr[i] = v;
    }
  };
  auto lstore = [&](int kbuf, int vbuf) {
    uint16_t* k_lds = &sK[kbuf][0][0];
    uint16_t* v_lds = &sV[vbuf][0][0];
#pragma unroll
    for (int i = 0; i < KCH; ++i)
      *reinterpret_cast<uint4*>(k_lds + k_dst[i]) = Frag8<F8>::bits(kr[i]);
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      // keys 8*half .. +3 and +4 .. +7 of the block go to their permuted slots
      const int h8 = v_key[i] & 8;
      uint16_t* dst = v_lds + v_dst[i];
      const uint4 vv = Frag8<F8>::bits(vr[i]);
      *reinterpret_cast<uint2*>(dst + vperm(h8)) = make_uint2(vv.x, vv.y);
      *reinterpret_cast<uint2*>(dst + vperm(h8 + 4)) = make_uint2(vv.z, vv.w);
    }
  };

  // m: running max (base 2); l: denominator at m; m_prev, lpend, rescale:
  // the previous tile's max move and row sum, folded in by settle()
  float m[RG], l[RG], m_prev[RG], lpend[RG];
  bool rescale[RG];
  f32x16 acc[RG][DB];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    m[rg] = -INFINITY;
    l[rg] = 0.f;
    m_prev[rg] = -INFINITY;
    lpend[rg] = 0.f;
    rescale[rg] = false;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[rg][i][j] = 0.f;
  }

  // block-table window: entries [tab_base, tab_base + kTabWin) live in LDS.
  // It covers every block of the request: a 64-key tile can reach past the
  // last visible key, and those keys must still be read from their own
  // blocks (finite values times P = 0), never from a stand-in block.
  const int nblk = (seq_len + 15) >> 4;
  auto load_tab = [&](int base) {
    for (int i = tid; i < kTabWin; i += NT) s_tab[i] = (base + i < nblk) ? table[base + i] : 0;
  };
  load_tab(tab_base);
  __syncthreads();
  gload(kbeg);
  lstore(0, 0);
  __syncthreads();

  // A moved max of the previous tile: acc holds every P.V up to two tiles
  // back and l every row sum up to two tiles back, both at the old max; the
  // previous tile's row sum is at the new one.  The rescale (and its one
  // exponential) runs only on tiles where the max moved: the branch is
  // wave-uniform.  CASC rows that have seen no key yet keep a factor of 1.
  auto settle = [&]() {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      if (rescale[rg]) {
        const float alpha =
            (CASC && m[rg] == -INFINITY) ? 1.f : fast_exp2(m_prev[rg] - m[rg]);
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[rg][db] *= alpha;
        l[rg] = l[rg] * alpha + lpend[rg];
      } else {
        l[rg] += lpend[rg];
      }
    }
  };

  // O^T += V^T P^T over a tile: four 16-key steps; each V^T fragment read
  // from LDS feeds the MFMAs of every row group of the wave
  // (the fragments of the first step, fv0, are read by the caller ahead of
  // time, so the first MFMAs do not wait for LDS)
  auto vfrag = [&](uint4 (&f)[DB], int vbuf, int ps) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
      f[db] = *reinterpret_cast<const uint4*>(&sV[vbuf][32 * db + row][16 * ps + 8 * kg]);
  };
  auto pv = [&](int vbuf, const bf16x8 (&pf)[RG][PS], const uint4 (&fv0)[DB]) {
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) {
      uint4 fv[DB];
      if (ps == 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db) fv[db] = fv0[db];
      } else {
        vfrag(fv, vbuf, ps);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          acc[rg][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fv[db]), pf[rg][ps],
                                                                acc[rg][db], 0, 0, 0);
    }
  };

  // Software pipeline per wave: iteration `it` computes S of tile it, then
  // issues the P.V products of tile it-1 (P kept in registers, V^T still in
  // its LDS buffer) in the same basic block as the softmax of tile it, so the
  // MFMAs run while the exponentials issue.  K is double-buffered in LDS, V
  // triple-buffered (tile it-1 is still read while tile it+1 is stored).
  // Tiles past a row's position are computed anyway (masked: P = 0), which
  // keeps the loop body branch-free.  Before the first tile, P = 0 against
  // the finite V^T of tile 0.
  bf16x8 pprev[RG][PS];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) pprev[rg][ps] = as_bf16x8(make_uint4(0, 0, 0, 0));
  int vprev = 0;
  int it = 0;
  for (int k0 = kbeg; k0 < kend; k0 += kBK, ++it) {
    const int kbuf = it & 1, vbuf = it % 3;
    const bool more = k0 + kBK < kend;
    settle();
    if (more && ((k0 + kBK) >> 4) >= tab_base + kTabWin) {
      // the next tile starts a new window (tiles never straddle one); every
      // thread is past its last use of the old entries
      tab_base += kTabWin;
      load_tab(tab_base);
      __syncthreads();
    }
    if (more) gload(k0 + kBK);
    // ---- S^T = K Q^T: every K fragment feeds all row groups ------------------
    // The K fragments of the next group of MFMAs are read from LDS while the
    // current group runs (the fences keep the compiler from pairing each read
    // with the MFMA right after it, which exposes the LDS latency every time).
    f32x16 s[RG][KB];
    constexpr int SG = 2;                    // k-steps per group
    constexpr int NG = QSTEPS / SG;          // groups per tile
    static_assert(QSTEPS % SG == 0 && NG % 2 == 0, "k-steps split into an even number of groups");
    uint4 fka[KB][SG], fkb[KB][SG];
    uint4 fv0[DB];
    auto kfrag = [&](uint4 (&f)[KB][SG], int g) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int u = 0; u < SG; ++u)
          f[kb][u] = *reinterpret_cast<const uint4*>(
              &sK[kbuf][32 * kb + row][8 * kg + 16 * (SG * g + u)]);
    };
    auto kmfma = [&](const uint4 (&f)[KB][SG], int g) {
#pragma unroll
      for (int u = 0; u < SG; ++u)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int rg = 0; rg < RG; ++rg)
            s[rg][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                as_bf16x8(f[kb][u]), qf[rg][SG * g + u],
                (g == 0 && u == 0) ? f32x16{} : s[rg][kb], 0, 0, 0);
    };
    kfrag(fka, 0);
#pragma unroll
    for (int g = 0; g < NG; g += 2) {
      if (g + 1 < NG) kfrag(fkb, g + 1);
      __builtin_amdgcn_sched_barrier(0);
      kmfma(fka, g);
      __builtin_amdgcn_sched_barrier(0);
      if (g + 1 < NG) {
        if (g + 2 < NG) kfrag(fka, g + 2);
        // the first V^T fragments of the P.V below load during the last group
        if (g + 2 >= NG) vfrag(fv0, vprev, 0);
        __builtin_amdgcn_sched_barrier(0);
        kmfma(fkb, g + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (k0 + kBK - 1 > wpos_lo) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int key = k0 + 32 * kb + 8 * i + 4 * kg + j;
              if (key > pos[rg]) s[rg][kb][4 * i + j] = -INFINITY;
            }
    }
    float m_new[RG];
    bool move[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      // row max: 2 * KB independent chains of three-input maxima (8 values
      // per chain, 4 instructions), then the chains
      float mx[2 * KB];
#pragma unroll
      for (int u = 0; u < 2 * KB; ++u) {
        const f32x16& sv = s[rg][u >> 1];
        const int o = 8 * (u & 1);
        float c = fmaxf(fmaxf(sv[o], sv[o + 1]), sv[o + 2]);
        c = fmaxf(fmaxf(c, sv[o + 3]), sv[o + 4]);
        c = fmaxf(fmaxf(c, sv[o + 5]), sv[o + 6]);
        mx[u] = fmaxf(c, sv[o + 7]);
      }
#pragma unroll
      for (int w = 2 * KB; w > 1; w >>= 1)
#pragma unroll
        for (int u = 0; u < w / 2; ++u) mx[u] = fmaxf(mx[u], mx[u + w / 2]);
      float mt = mx[0];
      mt = max_xor32(mt) * scale_log2;  // scale > 0 commutes with max
      move[rg] = __ballot(mt > m[rg] + kLazy) != 0;
      // finite once the wave has met key 0, which every row sees
      m_new[rg] = move[rg] ? fmaxf(m[rg], mt) : m[rg];
    }
    // exponent reference: CASC rows that have seen no key yet (m = -inf)
    // take 0, so their masked scores give P = 0 rather than NaN
    float m_ref[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
      m_ref[rg] = (CASC && m_new[rg] == -INFINITY) ? 0.f : m_new[rg];

    // ---- P.V of the previous tile, interleaved with this tile's softmax -----
    pv(vprev, pprev, fv0);
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      float ps4[4];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          s[rg][kb][j] = fast_exp2(__builtin_fmaf(s[rg][kb][j], scale_log2, -m_ref[rg]));
          // the first four values seed the partial sums (no 0 + x)
          if (kb == 0 && j < 4) ps4[j] = s[rg][kb][j];
          else ps4[j & 3] += s[rg][kb][j];
        }
      const float rs = (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
        const f32x16& sp = s[rg][ps >> 1];
        const int o = 8 * (ps & 1);
        pprev[rg][ps] = as_bf16x8(make_uint4(
            pack_bf16x2(sp[o + 0], sp[o + 1]), pack_bf16x2(sp[o + 2], sp[o + 3]),
            pack_bf16x2(sp[o + 4], sp[o + 5]), pack_bf16x2(sp[o + 6], sp[o + 7])));
      }
      // folded into acc and l by settle() at the top of the next iteration,
      // after the previous tile's P.V (accumulated at the old max) is in
      m_prev[rg] = m[rg];
      rescale[rg] = move[rg];
      lpend[rg] = rs;
      m[rg] = m_new[rg];
    }
    // Issue order of the block above: each P.V MFMA followed by about ten
    // VALU instructions of the softmax, and the V^T fragments of the next
    // 16-key step read from LDS right after that step's first MFMA.  Left to
    // itself the scheduler issues the MFMAs ahead of the exponentials, which
    // then run with the matrix core idle (long prefill: 1-2 % faster in A/Bs
    // on three boxes; identical results).
#pragma unroll
    for (int ps = 0; ps < PS; ++ps)
#pragma unroll
      for (int j = 0; j < RG * DB; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // ten VALU
        if (j == 0 && ps + 1 < PS) __builtin_amdgcn_sched_group_barrier(0x100, DB, 0);  // LDS reads
      }
    vprev = vbuf;
    // unconditional: after the last tile it stores stale registers into
    // buffers nothing reads again (keeps the loop body one basic block)
    lstore(kbuf ^ 1, (it + 1) % 3);
    __syncthreads();
  }
  settle();
  {
    uint4 fv0[DB];
    vfrag(fv0, vprev, 0);
    pv(vprev, pprev, fv0);
  }

#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const float lt = sum_xor32(l[rg]);
    if (!valid[rg]) continue;
    const float inv = v_scale / lt;
    const int h = kvh * G + gr[rg];
    if constexpr (CASC) {
      // the partial of gathered row tokr over this key range: fp32,
      // normalised; a row that saw no key here gives o = 0, lse = -inf
      const size_t prow_i = ((size_t)ksplit * p.pre_rows + tokr[rg]) * p.hq + h;
      const float cinv = lt > 0.f ? inv : 0.f;
      float* prow = p.pre_out + prow_i * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x16& a = acc[rg][db];
          *reinterpret_cast<float4*>(prow + 32 * db + 8 * i + 4 * kg) =
              make_float4(a[4 * i] * cinv, a[4 * i + 1] * cinv, a[4 * i + 2] * cinv,
                          a[4 * i + 3] * cinv);
        }
      if (kg == 0) p.pre_lse[prow_i] = lt > 0.f ? (m[rg] + fast_log2(lt)) * kLn2 : -INFINITY;
      continue;
    }
    const int t = q0 + tokr[rg];
    uint16_t* orow = p.out + ((size_t)t * p.hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * db + 8 * i + 4 * kg;
        const f32x16& a = acc[rg][db];
        *reinterpret_cast<uint2*>(orow + d) =
            make_uint2(pack_bf16x2(a[4 * i] * inv, a[4 * i + 1] * inv),
                       pack_bf16x2(a[4 * i + 2] * inv, a[4 * i + 3] * inv));
      }
    if (p.lse != nullptr && kg == 0)
      p.lse[(size_t)t * p.hq + h] = (m[rg] + fast_log2(lt)) * kLn2;
  }
}

}  // namespace pa
