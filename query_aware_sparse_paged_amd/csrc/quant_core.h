// 2-bit quantised KV pages for grouped-query heads (page 16, head_dim 128):
// KIVI-style codes (2 bits, groups of 32: SCBench notes, the method table)
// for every page outside a full-precision residual region of the last R
// logical pages (SparseEngine article, decode-hook paragraph: a quantised
// region managed together with a residual one).  Scoring and selection are
// unchanged (the summaries come from the full-precision keys); only the
// attention reads a selected page back from its codes.
//
// Quantiser (per token, 32 consecutive channels of the key or the value): m =
// the group minimum and s = (max - min) / 3, both stored as binary16; code =
// round-half-even((x - m) / s) clamped to 0..3, each step in binary32 with m
// and s as stored (s = 0: code 0).  Read back as m + code * s.
//
// A quantised page-head is 1536 bytes (against 8192 in bf16), packed so that
// each lane of the attention reads its MFMA fragments' codes as one 8-byte
// load (two words w0, w1) and turns each pair of codes into a pair of bf16
// operands 4 + c with one rotate and one and-or: pair p (< 16) lives in
// word p / 8, rotated left by a = 2 (p % 8) from the position where its first
// code sits at bits 5-6 and its second at bits 21-22.
//   [   0, 512) key codes:   token t, lane group kg (< 4) at byte 32 t + 8 kg;
//                            pair p = 4 i + k holds channels 32 i + 8 kg + 2 k
//                            and + 1 (i, k < 4)
//   [ 512, 768) key pairs:   token t, group i: binary16 (m, s) at 16 t + 4 i
//   [ 768,1280) value codes: channel n (< 16) of each block, lane group kg at
//                            byte 8 (4 n + kg); pair p = 2 i + h holds tokens
//                            4 kg + 2 h and + 1 of channel 16 i + n (i < 8)
//   [1280,1536) value pairs: token t, group g (channels 32 g ...): at 16 t + 4 g
// The attention then needs no per-element dequantisation: with A' = 4 + c
// as the MFMA operand, q . (m + c s) over a group = (m - 4 s) sum(q) +
// s (q . A'), and sum_t p_t (m + c s) = sum_t p_t (m - 4 s) + (p s) . A'.
#pragma once

#include <hip/hip_fp16.h>

#include "attend_core.h"

namespace qasp {
namespace quant {

constexpr int kPageHeadBytes = 1536, kKeyPairs = 512, kValCodes = 768, kValPairs = 1280;

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
  return __half2float(__ushort_as_half((unsigned short)(h & 0xffffu)));
}

// (m, s) of a group as binary16 patterns, and its m, s as binary32.
__device__ __forceinline__ uint32_t group_pair(float mn, float mx, float &m, float &s) {
  const float st = __fdiv_rn(mx - mn, 3.0f);
  const __half m16 = __float2half_rn(mn), s16 = __float2half_rn(st);
  m = __half2float(m16);
  s = __half2float(s16);
  return (uint32_t)__half_as_ushort(m16) | ((uint32_t)__half_as_ushort(s16) << 16);
}

__device__ __forceinline__ uint32_t rotl(uint32_t x, int a) { return a == 0 ? x : (x << a) | (x >> (32 - a)); }

// bf16 operands 4 + c of pair p (< 16) of a lane's code words (4 + c has
// exponent 2 and the code in the two leading fraction bits).  mask and base
// are 0x00600060 and 0x40804080 held in registers (see CodeConsts), so the
// and-or is one instruction.
__device__ __forceinline__ uint32_t pair_operands(uint2 w, int p, uint32_t mask, uint32_t base) {
  const uint32_t x = p < 8 ? w.x : w.y;
  const uint32_t r = __builtin_amdgcn_alignbit(x, x, 2 * (p % 8));  // rotate right
  return (r & mask) | base;
}

// The two constants of pair_operands, made opaque so that they stay in
// registers (as literals they would split the and-or into two instructions).
struct CodeConsts {
  uint32_t mask, base;
  __device__ __forceinline__ CodeConsts() : mask(0x00600060u), base(0x40804080u) {
    asm volatile("" : "+v"(mask), "+v"(base));
  }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// a, b as a bf16 pair (round to nearest even) and the pair of what remains.
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
  const float ra = a - __uint_as_float(hi << 16), rb = b - __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){ra, rb}, bf16x2_t));
}

__device__ __forceinline__ uint32_t code_of(float x, float m, float s) {
  if (s == 0.f) return 0u;
  const float c = rintf(__fdiv_rn(x - m, s));
  return (uint32_t)fminf(fmaxf(c, 0.f), 3.f);
}

// Quantises page-head (phys, g) from the bf16 pools (keys [t][d], values
// [dv][t]).  Called by every thread of a block of at least 256 threads (it
// holds two block barriers); sm: 256 floats of LDS.  Phase A computes the
// (m, s) pair of every group (16 tokens x 4 key + 4 value groups) into LDS and
// memory; phase B writes the code words (each word is written by one thread).
__device__ inline void quantize_page_head(const uint16_t *__restrict__ k_pool, const uint16_t *__restrict__ v_pool,
                                   uint8_t *__restrict__ qpool, int phys, int g, int Hkv, float *sm) {
  constexpr int PS = 16, D = 128, DV = 128;
  float *sh_m = sm, *sh_s = sm + 8 * PS;  // [token][group: 4 key, 4 value]
  const int tid = threadIdx.x;
  const size_t ph = (size_t)phys * Hkv + g;
  const uint16_t *kp = k_pool + ph * PS * D;   // [t][d]
  const uint16_t *vp = v_pool + ph * DV * PS;  // [dv][t]
  uint8_t *dst = qpool + ph * kPageHeadBytes;
  if (tid < 8 * PS) {
    const int t = tid / 8, grp = tid % 8;
    // min / max in channel order, the first of equal values kept (so the
    // sign of a zero minimum is that of the first zero)
    float mn = 0.f, mx = 0.f;
    for (int e = 0; e < 32; e++) {
      const uint16_t bits = grp < 4 ? kp[t * D + 32 * grp + e] : vp[(32 * (grp - 4) + e) * PS + t];
      const float x = __uint_as_float((uint32_t)bits << 16);
      if (e == 0 || x < mn) mn = x;
      if (e == 0 || x > mx) mx = x;
    }
    float m, s;
    const uint32_t pair = group_pair(mn, mx, m, s);
    sh_m[tid] = m;
    sh_s[tid] = s;
    *(uint32_t *)(dst + (grp < 4 ? kKeyPairs + 16 * t + 4 * grp : kValPairs + 16 * t + 4 * (grp - 4))) = pair;
  }
  __syncthreads();
  if (tid < 128) {  // key codes: item (t, kg, word h) -> 16 codes (groups 2h, 2h + 1), one word
    const int t = tid / 8, kg = (tid / 2) % 4, h = tid % 2;
    uint32_t w = 0;
    for (int pp = 0; pp < 8; pp++) {  // pair 8 h + pp: group i = 2 h + pp / 4, k = pp % 4
      const int i = 2 * h + pp / 4, k = pp % 4;
      const float m = sh_m[t * 8 + i], s = sh_s[t * 8 + i];
      const float x0 = __uint_as_float((uint32_t)kp[t * D + 32 * i + 8 * kg + 2 * k] << 16);
      const float x1 = __uint_as_float((uint32_t)kp[t * D + 32 * i + 8 * kg + 2 * k + 1] << 16);
      w |= rotl(code_of(x0, m, s) << 5 | code_of(x1, m, s) << 21, 2 * pp);
    }
    *(uint32_t *)(dst + 32 * t + 8 * kg + 4 * h) = w;
  } else if (tid < 256) {  // value codes: item (n, kg, word h) -> 16 codes (blocks 4h .. 4h + 3), one word
    const int item = tid - 128, n = item / 8, kg = (item / 2) % 4, h = item % 2;
    uint32_t w = 0;
    for (int pp = 0; pp < 8; pp++) {  // pair 8 h + pp: block i = 4 h + pp / 2, tokens 4 kg + 2 (pp % 2) + 0/1
      const int i = 4 * h + pp / 2, dv = 16 * i + n, grp = 4 + dv / 32;
      const int t0 = 4 * kg + 2 * (pp % 2), t1 = t0 + 1;
      const float x0 = __uint_as_float((uint32_t)vp[dv * PS + t0] << 16);
      const float x1 = __uint_as_float((uint32_t)vp[dv * PS + t1] << 16);
      w |= rotl(code_of(x0, sh_m[t0 * 8 + grp], sh_s[t0 * 8 + grp]) << 5 |
                    code_of(x1, sh_m[t1 * 8 + grp], sh_s[t1 * 8 + grp]) << 21,
                2 * pp);
    }
    *(uint32_t *)(dst + kValCodes + 8 * (4 * n + kg) + 4 * h) = w;
  }
  __syncthreads();
}

// The page of sequence b that leaves the residual region at this step: when
// the step's token opened a new page, page P - 1 - residual_pages; else -1.
__device__ __forceinline__ int leaving_page(int L, int residual_pages) {
  constexpr int PS = 16;
  if (L < 1 || (L - 1) % PS != 0) return -1;
  const int j = (L + PS - 1) / PS - 1 - residual_pages;
  return j >= 0 ? j : -1;
}

// One quantised page-head's fragments for a wave lane.
// (the pairs are loaded separately: see the attention loop)
struct QPage {
  uint2 kc;      // key code words: token l % 16, channels 32 i + 8 (l / 16) ...
  uint2 vc;      // value code words: channels 16 i + l % 16, tokens 4 (l / 16) ...

  __device__ __forceinline__ void load(const uint8_t *ph, int lane) {
    const int n = lane & 15, kg = lane >> 4;
    kc = *(const uint2 *)(ph + 32 * n + 8 * kg);
    vc = *(const uint2 *)(ph + kValCodes + 8 * (4 * n + kg));
  }
};

// Key or value pairs (at byte offset off) of tokens 4 (l / 16) + r, groups 0..3.
__device__ __forceinline__ void load_pairs(uint4 *pr, const uint8_t *ph, int off, int lane) {
#pragma unroll
  for (int r = 0; r < 4; r++) pr[r] = *(const uint4 *)(ph + off + 16 * ((lane >> 4) * 4 + r));
}

__device__ __forceinline__ uint32_t dw(const uint4 &v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// Sum of head column l % 16's query over each group of 32 channels (every
// lane of the column gets it).
__device__ __forceinline__ void query_group_sums(const uint4 *bq, float *qs) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint32_t w = dw(bq[i], k);
      a += __uint_as_float(w << 16) + __uint_as_float(w & 0xffff0000u);
    }
    a += __shfl_xor(a, 16, kWave);
    a += __shfl_xor(a, 32, kWave);
    qs[i] = a;
  }
}

// Softmax attention of the wave's head columns over one quantised page
// (logical id j; vp: its value pairs).  bacc[g] accumulates, in the scale of
// st, this lane's tokens' share of the zero-point part of the output channels
// of value group g (summed over the lanes of a column and added to st.acc by
// the caller).
__device__ __forceinline__ void attend_qpage(attend::WaveState &st, float *bacc, const QPage &pg, const uint4 *kp,
                                             const uint4 *vp, const uint4 *bq, const float *qs, int j, int L,
                                             bool is_static, int sink_end, int win_begin, float scale_log2,
                                             const CodeConsts &cc, int lane) {
  constexpr int PS = 16;
  const int kg = lane >> 4;
  // S^T: per group, (m - 4 s) sum(q) + s (A' q)
  float sv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint4 a = make_uint4(pair_operands(pg.kc, 4 * i, cc.mask, cc.base),
                               pair_operands(pg.kc, 4 * i + 1, cc.mask, cc.base),
                               pair_operands(pg.kc, 4 * i + 2, cc.mask, cc.base),
                               pair_operands(pg.kc, 4 * i + 3, cc.mask, cc.base));
    const floatx4 o = mfma16x16x32(a, bq[i], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const uint32_t pair = dw(kp[r], i);
      const float m = half_bits_to_f32(pair), sc = half_bits_to_f32(pair >> 16);
      sv[r] = fmaf(fmaf(-4.f, sc, m), qs[i], fmaf(sc, o[r], sv[r]));
    }
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int pos = j * PS + 4 * kg + r;
    const bool ok = (pos < L) & (!is_static | (pos < sink_end) | (pos >= win_begin));
    sv[r] = ok ? sv[r] * scale_log2 : -INFINITY;
    tmax = fmaxf(tmax, sv[r]);
  }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
  const float m_new = fmaxf(st.m, tmax);
  float alpha = 1.f;
  float p[4];
  if (m_new == -INFINITY) {
#pragma unroll
    for (int r = 0; r < 4; r++) p[r] = 0.f;
  } else {
    alpha = __builtin_amdgcn_exp2f(st.m - m_new);
#pragma unroll
    for (int r = 0; r < 4; r++) p[r] = sv[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[r] - m_new);
  }
  float psum = (p[0] + p[1]) + (p[2] + p[3]);
  psum += __shfl_xor(psum, 16, kWave);
  psum += __shfl_xor(psum, 32, kWave);
  st.l = st.l * alpha + psum;
  st.m = m_new;
  // per value group g: weights p s as bf16 hi + lo, and the zero-point part
  uint2 bh[4], bl[4];
#pragma unroll
  for (int g = 0; g < 4; g++) {
    float w4[4], z = 0.f;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const uint32_t pair = dw(vp[r], g);
      const float m = half_bits_to_f32(pair), sc = half_bits_to_f32(pair >> 16);
      w4[r] = p[r] * sc;
      z = fmaf(p[r], fmaf(-4.f, sc, m), z);
    }
    split2(w4[0], w4[1], bh[g].x, bl[g].x);
    split2(w4[2], w4[3], bh[g].y, bl[g].y);
    bacc[g] = fmaf(bacc[g], alpha, z);
  }
  // once the running maxima stop moving, alpha is exactly 1 in every lane:
  // then the accumulators need no rescaling (a wave-uniform test)
  if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
    for (int i = 0; i < 8; i++) st.acc[i] *= alpha;
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint2 a =
        make_uint2(pair_operands(pg.vc, 2 * i, cc.mask, cc.base), pair_operands(pg.vc, 2 * i + 1, cc.mask, cc.base));
    st.acc[i] = mfma16x16x16(a, bh[i / 2], st.acc[i]);
    st.acc[i] = mfma16x16x16(a, bl[i / 2], st.acc[i]);
  }
}


// Attention of one wave over its npg (<= 64) pages of a unit, lane i holding
// the i-th page's logical id (my_j) and physical page (my_phys), ascending:
// the pages below q_end from the quantised pool (code words one page ahead,
// each page's pairs at its start), the others from the bf16 pools, one at a
// time.  bq: the q columns of the wave's heads.
__device__ __forceinline__ void attend_wave_quant(attend::WaveState &st, const uint4 *bq, int npg, int my_j,
                                                  int my_phys, int q_end, const uint8_t *__restrict__ qpool,
                                                  const uint16_t *__restrict__ k_pool,
                                                  const uint16_t *__restrict__ v_pool, int Hkv, int g, int L,
                                                  bool is_static, int sink_end, int win_begin, float scale_log2,
                                                  int lane) {
  constexpr int PS = 16, D = 128, DV = 128;
  const int n_q = __popcll(__ballot(lane < npg && my_j < q_end));  // the wave's first n_q pages
  if (n_q > 0) {
    auto base = [&](int it) {
      return qpool + ((size_t)__shfl(my_phys, min(it, n_q - 1), kWave) * Hkv + g) * kPageHeadBytes;
    };
    float qs[4], bacc[4] = {0.f, 0.f, 0.f, 0.f};
    query_group_sums(bq, qs);
    // code words one page ahead; the pairs are loaded at the start of their
    // page (the value pairs are waited on only after the key work)
    const CodeConsts cc;
    QPage cur, nxt;
    cur.load(base(0), lane);
    for (int it = 0; it < n_q; it++) {
      uint4 kp[4], vp[4];
      load_pairs(kp, base(it), kKeyPairs, lane);
      load_pairs(vp, base(it), kValPairs, lane);
      nxt.load(base(it + 1), lane);  // past the end: the last page again (unused)
      attend_qpage(st, bacc, cur, kp, vp, bq, qs, __shfl(my_j, it, kWave), L, is_static, sink_end, win_begin,
                   scale_log2, cc, lane);
      cur = nxt;
    }
    // output channels 16 i + 4 (l / 16) + r belong to value group i / 2; the
    // lanes of a column hold their own tokens' shares
#pragma unroll
    for (int gr = 0; gr < 4; gr++) {
      bacc[gr] += __shfl_xor(bacc[gr], 16, kWave);
      bacc[gr] += __shfl_xor(bacc[gr], 32, kWave);
    }
#pragma unroll
    for (int i = 0; i < 8; i++) st.acc[i] += bacc[i / 2];
  }
  // the remaining (residual) pages from the bf16 pools, one at a time (a
  // handful per wave; no prefetch stages, which keeps the registers low)
  const attend::PageWork<PS, D, DV> pw{k_pool, v_pool, bq, Hkv, g, L, sink_end, win_begin, is_static, scale_log2};
  for (int it = n_q; it < npg; it++) {
    const attend::PageRegs<D, DV> pr = pw.load(__shfl(my_phys, it, kWave), lane);
    pw.compute(st, true, __shfl(my_j, it, kWave), pr.k, pr.v, lane);
  }
}

}  // namespace quant
}  // namespace qasp
