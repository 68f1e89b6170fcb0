// Device building blocks of the sparse paged attention (grouped-query
// heads, page 16, head_dim 128): one wave attends its group's heads over a
// list of page-heads with online softmax.
//
// Per page-head a wave
//   - loads the 16x128 key tile straight into the A operand of 4 MFMAs
//     (16x16x32): lane (token m = l%16, k block l/16) reads 16 contiguous
//     bytes of key row m, so the 64 lanes read the page-head's 4 KiB once;
//   - S^T = K q^T puts token 4*(l/16)+r of head l%16 in lane l, register r;
//   - online softmax in the exp2 domain per head (running max m, sum l);
//   - O^T += V^T P with 16x16x16 MFMAs: the value tile is stored transposed
//     ([dv][token], tokens fastest), so lane (dv = l%16, l/16) reads 4
//     consecutive tokens as 8 contiguous bytes, and P^T comes straight from
//     the S^T registers.  P is split into bf16 hi + lo parts (two MFMAs) so
//     the weights keep ~16 significant bits.
// Two page-heads are in flight while one is computed: three register stages
// rotate through an unrolled loop, every prefetch is issued (past the end the
// last page is loaded again and computed fully masked), so the compiler's
// load-wait counts stay static.
#pragma once

#include "common.h"

namespace qasp {
namespace attend {

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16),
                    f32_to_bf16_rne(c) | (f32_to_bf16_rne(d) << 16));
}
__device__ __forceinline__ float bf16_round_f32(float a) { return __uint_as_float(f32_to_bf16_rne(a) << 16); }

// q^T as the B operand: column n = head n of the group (qg = its first row).
template <int D>
__device__ __forceinline__ void load_q_columns(uint4 *bq, const uint16_t *qg, int G, int lane) {
  const int n = lane & 15, kg = lane >> 4;
  const uint32_t keep = n < G ? ~0u : 0u;  // unconditional loads (row clamped), then masked
  const uint16_t *qh = qg + (size_t)(n < G ? n : 0) * D + 8 * kg;
#pragma unroll
  for (int i = 0; i < D / 32; i++) {
    const uint4 v = *(const uint4 *)(qh + 32 * i);
    bq[i] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
  }
}

struct WaveState {
  float m, l;        // running max (log2 units) and sum, per head column
  floatx4 acc[8];    // O^T rows dv = 16 i + 4 (l/16) + r, column l % 16
};

__device__ __forceinline__ void init_state(WaveState &st) {
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int i = 0; i < 8; i++) st.acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
}

// One page-head's fragments for a wave (keys as MFMA A operands, values as
// V^T fragments), held in registers.
template <int D, int DV>
struct PageRegs {
  uint4 k[D / 32];
  uint2 v[DV / 16];
};

// Loading and computing one page-head for a wave (the two halves of the
// pipelined loops below).  L, sink_end and win_begin bound the tokens of the
// unit (their values are read).  With CAUSAL the head columns are draft
// queries with their own ends: column l % 16 scores only tokens before Lq and,
// for a static head, at or after winq (its own window) or before sink_end;
// the unit bounds still decide which value entries are read.
template <int PS, int D, int DV, bool CAUSAL = false>
struct PageWork {
  static_assert(PS == 16 && D == 128 && DV == 128, "tile shapes");
  const uint16_t *__restrict__ k_pool;
  const uint16_t *__restrict__ v_pool;
  const uint4 *bq;
  int Hkv, g, L, sink_end, win_begin;
  bool is_static;
  float scale_log2;
  int Lq, winq;  // per lane, CAUSAL only

  __device__ __forceinline__ void load(int phys, uint4 *kk, uint2 *vv, int lane) const {
    const int n = lane & 15, kg = lane >> 4;
    const size_t ph = (size_t)phys * Hkv + g;
    const uint16_t *kp = k_pool + (ph * PS + n) * D + 8 * kg;
    const uint16_t *vp = v_pool + ph * DV * PS + (size_t)n * PS + 4 * kg;
#pragma unroll
    for (int i = 0; i < D / 32; i++) kk[i] = *(const uint4 *)(kp + 32 * i);
#pragma unroll
    for (int i = 0; i < DV / 16; i++) vv[i] = *(const uint2 *)(vp + 16 * i * PS);
  }
  __device__ __forceinline__ PageRegs<D, DV> load(int phys, int lane) const {
    PageRegs<D, DV> r;
    load(phys, r.k, r.v, lane);
    return r;
  }

  // page with logical id j; real = false computes it fully masked
  __device__ __forceinline__ void compute(WaveState &st, bool real, int j, const uint4 *kt, const uint2 *vt,
                                          int lane) const {
    const int kg = lane >> 4;
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D / 32; i++) s = mfma16x16x32(kt[i], bq[i], s);
    float sv[4];
    float tmax = -INFINITY;
    uint32_t keep[2] = {0u, 0u};  // value bits of the attended tokens 4kg + r
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int pos = j * PS + 4 * kg + r;
      const bool ok = real & (pos < L) & (!is_static | (pos < sink_end) | (pos >= win_begin));
      bool use = ok;
      if constexpr (CAUSAL) use = ok & (pos < Lq) & (!is_static | (pos < sink_end) | (pos >= winq));
      sv[r] = use ? s[r] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, sv[r]);
      keep[r >> 1] |= ok ? (0xffffu << (16 * (r & 1))) : 0u;
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
    const uint2 ph = pack_bf16x4(p[0], p[1], p[2], p[3]);
    const uint2 pl = pack_bf16x4(p[0] - bf16_round_f32(p[0]), p[1] - bf16_round_f32(p[1]),
                                 p[2] - bf16_round_f32(p[2]), p[3] - bf16_round_f32(p[3]));
    // values of tokens that are not attended are zeroed: a zero weight times
    // a stale non-finite pool entry would still be NaN
#pragma unroll
    for (int i = 0; i < DV / 16; i++) {
      const uint2 v = make_uint2(vt[i].x & keep[0], vt[i].y & keep[1]);
      st.acc[i] *= alpha;
      st.acc[i] = mfma16x16x16(v, ph, st.acc[i]);
      st.acc[i] = mfma16x16x16(v, pl, st.acc[i]);
    }
  }
};

// Attends npg page-heads.  Lane i (< npg) holds the i-th page's logical id
// (my_j) and physical page (my_phys).  Tokens t of a page are used when
// t < L and, for a static head, t < sink_end or t >= win_begin.  When pre is
// set, first already holds page 0 (loaded by the caller earlier).
template <int PS, int D, int DV, bool CAUSAL>
__device__ __forceinline__ void attend_pages(WaveState &st, const PageWork<PS, D, DV, CAUSAL> &pw, int npg, int my_j,
                                             int my_phys, int lane, bool pre = false,
                                             PageRegs<D, DV> first = PageRegs<D, DV>()) {
  if (npg <= 0) return;
  uint4 kA[D / 32], kB[D / 32], kC[D / 32];
  uint2 vA[DV / 16], vB[DV / 16], vC[DV / 16];
  auto load_page = [&](int it, uint4 *kk, uint2 *vv) {
    pw.load(__shfl(my_phys, min(it, npg - 1), kWave), kk, vv, lane);
  };
  auto compute_page = [&](int it, const uint4 *kt, const uint2 *vt) {
    pw.compute(st, it < npg, __shfl(my_j, min(it, npg - 1), kWave), kt, vt, lane);
  };
  // page it computes from (kc, vc) after prefetching page it+2 into (kn, vn)
  auto page_step = [&](int it, const uint4 *kc, const uint2 *vc, uint4 *kn, uint2 *vn) {
    load_page(it + 2, kn, vn);
    compute_page(it, kc, vc);
  };
  if (pre) {
#pragma unroll
    for (int i = 0; i < D / 32; i++) kA[i] = first.k[i];
#pragma unroll
    for (int i = 0; i < DV / 16; i++) vA[i] = first.v[i];
  } else {
    load_page(0, kA, vA);
  }
  load_page(1, kB, vB);
  for (int it = 0; it < npg; it += 3) {
    page_step(it, kA, vA, kC, vC);
    page_step(it + 1, kB, vB, kA, vA);
    page_step(it + 2, kC, vC, kB, vB);
  }
}

// Attends a wave's npg page-heads of any number: one page per lane in chunks
// of 64 (attend_pages holds a chunk's ids in the lanes).  page_at(i) returns
// (logical id, physical page) of the wave's i-th page; pre / first as in
// attend_pages, for the first chunk.
template <int PS, int D, int DV, bool CAUSAL, typename PageAt>
__device__ __forceinline__ void attend_list(WaveState &st, const PageWork<PS, D, DV, CAUSAL> &pw, int npg, int lane,
                                            PageAt page_at, bool pre = false,
                                            PageRegs<D, DV> first = PageRegs<D, DV>()) {
  const int n0 = min(npg, kWave);
  int2 jp = make_int2(0, 0);
  if (lane < n0) jp = page_at(lane);
  attend_pages<PS, D, DV>(st, pw, n0, jp.x, jp.y, lane, pre, first);
  // more than 64 pages for this wave (a selection of more than 64 pages per
  // wave of the block): the following chunks, without the preloaded page
  for (int c0 = kWave; c0 < npg; c0 += kWave) {
    const int nc = min(npg - c0, kWave);
    int2 jc = make_int2(0, 0);
    if (lane < nc) jc = page_at(c0 + lane);
    attend_pages<PS, D, DV>(st, pw, nc, jc.x, jc.y, lane);
  }
}

// LDS footprint of merge_waves for W waves and G heads (floats).
__host__ __device__ constexpr int merge_lds_floats(int W, int G, int DV) { return 2 * W * G + W * G * (DV + 4); }

// Merges the W waves' states of the block through LDS (sm: merge_lds_floats
// floats).  emit(h, dv, a, lsum, M) is called once per (head, channel) with
// the combined unnormalised accumulator a, sum lsum and max M.
template <int W, int DV, typename Emit>
__device__ __forceinline__ void merge_waves(float *sm, const WaveState &st, int G, Emit emit) {
  constexpr int ROW = DV + 4;
  float *sm_m = sm, *sm_l = sm + W * G, *sm_acc = sm + 2 * W * G;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int n = lane & 15, kg = lane >> 4;
  if (n < G) {
    if (kg == 0) {
      sm_m[wave * G + n] = st.m;
      sm_l[wave * G + n] = st.l;
    }
    float *row = sm_acc + ((size_t)wave * G + n) * ROW;
#pragma unroll
    for (int i = 0; i < DV / 16; i++)
#pragma unroll
      for (int r = 0; r < 4; r++) row[16 * i + 4 * kg + r] = st.acc[i][r];
  }
  __syncthreads();
  for (int item = threadIdx.x; item < G * DV; item += W * kWave) {
    const int h = item / DV, dv = item % DV;
    float M = sm_m[h];
#pragma unroll
    for (int w = 1; w < W; w++) M = fmaxf(M, sm_m[w * G + h]);
    float a = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; w++) {
        const float f = __builtin_amdgcn_exp2f(sm_m[w * G + h] - M);  // exp2(-inf) = 0
        a += f * sm_acc[((size_t)w * G + h) * ROW + dv];
        lsum += f * sm_l[w * G + h];
      }
    }
    emit(h, dv, a, lsum, M);
  }
}

}  // namespace attend
}  // namespace qasp
