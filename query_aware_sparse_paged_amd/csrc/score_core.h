// Device building blocks of score_pages: the per-page upper bound on q.k
// from the page summaries, on MFMA.
//
// For query head h and page j with summary (lo, hi):
//     U_h(j) = sum_d max(q_d lo_d, q_d hi_d) = q_h^- . lo_j + q_h^+ . hi_j
// (q^- keeps the negative channels of q, q^+ the positive ones), and the
// page's score is max over the heads h that share the KV head.  The split
// form is one dot product of length 2*D between [q^-, q^+] and the summary
// row [lo, hi], so a 16-page group against up to 16 heads is a chain of
// 16x16x32 bf16 MFMAs.  Each MFMA starts from zero and its 32-product result
// is added in fp64, so the only fp32 rounding is inside one MFMA.  Alongside,
// chained MFMAs on absolute values give S_h(j) = sum_d |q_d| |x_d|, from
// which a rigorous bound on the error of the fp32 score follows:
//     |U_fp32 - U| <= 33 * 2^-23 * S * 1.01 + 2^-50
// The product of two bf16 values (8-bit significands) is exact in fp32, so an
// MFMA rounds only in its additions: at most 32 of them, each on a partial
// sum bounded by that step's share of S, with unit roundoff taken as 2^-23 so
// that a faithful rather than nearest rounding is covered; the exact fp64
// conversions, the fp64 additions and the final rounding to fp32 add less than
// 2^-23 S; the absolute term covers flushed subnormal operands and products
// when |q|, |k| <= 2^64.  The selection uses this bound to decide which pages
// it must re-score exactly.
#pragma once

#include "common.h"

namespace qasp {
namespace score {

constexpr float kErrRel = 33.0f * 1.1920928955078125e-07f * 1.01f;  // 33 * 2^-23 * 1.01
constexpr float kErrAbs = 8.8817841970012523e-16f;                   // 2^-50

__device__ __forceinline__ uint4 map4(uint4 v, int mode) {
  // mode 0: negative part, 1: positive part, 2: absolute value
  uint4 r;
  if (mode == 0) {
    r.x = bf16x2_negative_part(v.x); r.y = bf16x2_negative_part(v.y);
    r.z = bf16x2_negative_part(v.z); r.w = bf16x2_negative_part(v.w);
  } else if (mode == 1) {
    r.x = bf16x2_positive_part(v.x); r.y = bf16x2_positive_part(v.y);
    r.z = bf16x2_positive_part(v.z); r.w = bf16x2_positive_part(v.w);
  } else {
    r.x = bf16x2_abs(v.x); r.y = bf16x2_abs(v.y); r.z = bf16x2_abs(v.z); r.w = bf16x2_abs(v.w);
  }
  return r;
}

// A operands of one wave: row m = head m of the group, k = [q^-, q^+] and its
// absolute value.  Lane l holds row l % 16, k block l / 16.
// ABS: also keep |q'| for the contraction on absolute values.
template <int D, bool ABS = true>
struct QOperands {
  static constexpr int KSTEPS = 2 * D / 32;
  uint4 aq[KSTEPS], aa[ABS ? KSTEPS : 1];
};

// qg: the group's first q row; heads m >= G (or an inactive group) get zeros.
template <int D, bool ABS = true>
__device__ __forceinline__ void load_q_operands(QOperands<D, ABS> &op, const uint16_t *qg, int G, bool active,
                                                int lane) {
  // active is uniform over the wave (q may be null when it is false); inside,
  // every lane loads (row clamped) and masks, so no per-lane branch
  // serialises the loads
  const int m = lane & 15, kg = lane >> 4;
  const uint16_t *qh = qg + (size_t)(m < G ? m : 0) * D;
  const uint32_t keep = m < G ? ~0u : 0u;
#pragma unroll
  for (int i = 0; i < QOperands<D, ABS>::KSTEPS; i++) {
    const int k0 = 32 * i + 8 * kg;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (active) v = *(const uint4 *)(qh + (k0 < D ? k0 : k0 - D));
    v = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
    op.aq[i] = map4(v, k0 < D ? 0 : 1);
    if (ABS) op.aa[i] = map4(op.aq[i], 2);
  }
}

// Summary rows of physical page `phys` (>= 0) for KV head g, in the B-operand
// layout: lane l holds page column l % 16 ... the caller passes the lane's page.
template <int D>
__device__ __forceinline__ void load_group(uint4 *dst, const uint16_t *summ, int phys, int Hkv, int g, int lane) {
  const uint16_t *sp = summ + summ_record(phys, g, Hkv) * (2 * D) + 8 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 2 * D / 32; i++) dst[i] = *(const uint4 *)(sp + 32 * i);
}

// Scores of a 16-page group: on return every lane of page column l % 16 holds
// the group score (max over the G heads, fp64 sum of the MFMA steps) and the
// largest S of its heads.
template <int D>
__device__ __forceinline__ void score_group(const QOperands<D> &op, const uint4 *cur, int G, int lane,
                                            double &best, float &bound) {
  const int kg = lane >> 4;
  double u64[4] = {0.0, 0.0, 0.0, 0.0};
  floatx4 sa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < QOperands<D>::KSTEPS; i++) {
    const floatx4 ui = mfma16x16x32(op.aq[i], cur[i], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int r = 0; r < 4; r++) u64[r] += (double)ui[r];
    sa = mfma16x16x32(op.aa[i], map4(cur[i], 2), sa);
  }
  // lane (n, kg) holds heads 4kg + r of page n
  best = -INFINITY;
  bound = 0.f;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    if (4 * kg + r < G) {
      best = fmax(best, u64[r]);
      bound = fmaxf(bound, sa[r]);
    }
  }
  best = fmax(best, __shfl_xor(best, 16, kWave));
  best = fmax(best, __shfl_xor(best, 32, kWave));
  bound = fmaxf(bound, __shfl_xor(bound, 16, kWave));
  bound = fmaxf(bound, __shfl_xor(bound, 32, kWave));
}

// Candidate scoring order by physical page: positions [s0, n) of order[]
// (LDS) receive the candidates s0 .. n-1 sorted into 256 equal ranges of the
// pool by their physical page phys[i] (LDS), a counting sort in rounds of 4T
// (bucket of page p: (p * bucket_mul) >> 32).  The order inside a bucket is
// whatever the LDS atomics give; callers use the order only to schedule
// loads, so no result depends on it.  cnt: 256 ints of LDS, zero on entry
// and on return.  Called by all T threads of the block; ends with a barrier
// when it sorted anything.
template <int T>
__device__ void bucket_order(int32_t *order, const int32_t *phys, int s0, int n, uint32_t bucket_mul, int *cnt) {
  constexpr int NB = 256;
  static_assert(T >= NB && T % kWave == 0, "one bucket per thread or more");
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  for (int i0 = s0; i0 < n; i0 += 4 * T) {
    int bk[4], rk[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int i = i0 + r * T + tid;
      bk[r] = i < n ? min((int)__umulhi((uint32_t)phys[i], bucket_mul), NB - 1) : 0;
      rk[r] = i < n ? atomicAdd(&cnt[bk[r]], 1) : 0;
    }
    __syncthreads();
    if (wave == 0) {  // exclusive scan of the bucket counts, in place (4 per lane)
      int c[4], t = 0;
#pragma unroll
      for (int x = 0; x < 4; x++) {
        c[x] = cnt[4 * lane + x];
        t += c[x];
      }
      int e = wave_incl_sum(t) - t;
#pragma unroll
      for (int x = 0; x < 4; x++) {
        cnt[4 * lane + x] = e;
        e += c[x];
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int i = i0 + r * T + tid;
      if (i < n) order[i0 + cnt[bk[r]] + rk[r]] = i;
    }
    __syncthreads();
    for (int x = tid; x < NB; x += T) cnt[x] = 0;
    if (i0 + 4 * T < n) __syncthreads();  // the next round counts again
  }
}

// The host-side multiplier of bucket_order for a pool of pool_pages pages.
__host__ __device__ inline uint32_t bucket_multiplier(int pool_pages) {
  const unsigned long long m = (256ull << 32) / (unsigned long long)(pool_pages > 0 ? pool_pages : 1);
  return m > 0xffffffffull ? 0xffffffffu : (uint32_t)m;
}

// One wave's share of a unit's scoring: the wave's groups 0 .. my_groups-1
// (16 candidates each; cand_of(gi) is this lane's candidate in its gi-th
// group, -1 if none, phys_of(c) that candidate's physical page), the next
// group's summaries in flight while the current one is computed.  bs[0]
// already holds group 0, whose lane candidate is c_cur (page phys_cur).
// emit(c, best, bound) runs on the lanes with kg = 0 for every candidate.
template <int D, typename CandOf, typename PhysOf, typename Emit>
__device__ __forceinline__ void score_groups(const QOperands<D> &op, uint4 (&bs)[2][2 * D / 32], const uint16_t *summ,
                                             int Hkv, int g, int G, int my_groups, int c_cur, int phys_cur, int lane,
                                             CandOf cand_of, PhysOf phys_of, Emit emit) {
  constexpr int KSTEPS = 2 * D / 32;
  const int kg = lane >> 4;
  for (int gi = 0; gi < my_groups; gi += 2) {
#pragma unroll
    for (int half = 0; half < 2; half++) {
      uint4 *cur = bs[half];
      // prefetch: summaries of the next group (page 0 past the last)
      const int c_next = cand_of(gi + half + 1);
      const int phys_next = phys_of(c_next);
      load_group<D>(bs[half ^ 1], summ, max(phys_next, 0), Hkv, g, lane);
      if (phys_cur < 0) {
#pragma unroll
        for (int i = 0; i < KSTEPS; i++) cur[i] = make_uint4(0, 0, 0, 0);
      }
      double best;
      float bound;
      score_group<D>(op, cur, G, lane, best, bound);
      if (kg == 0 && c_cur >= 0) emit(c_cur, best, bound);
      phys_cur = phys_next;
      c_cur = c_next;
    }
  }
}

// The stored score of a candidate page: fp32 value and error bound; an
// overflow becomes (0, inf) so that selection re-scores the page exactly.
// With the runner-up head's value (second) and the leading head (arg), the
// leader is certified when it beats the runner-up by more than twice the
// error bound of every head's value.
__device__ __forceinline__ qasp_score make_score(double best, float bound, double second = INFINITY,
                                                 int arg = -1, float rel = kErrRel) {
  const float v = (float)best;
  const float err = rel * bound + kErrAbs;
  qasp_score sc;
  sc.reserved = 0;
  if (isfinite(v) && isfinite(err)) {
    sc.value = v == 0.f ? 0.f : v;  // no -0
    sc.err = err;
    sc.head = best - second > 2.0 * (double)err ? arg : -1;
  } else {
    sc.value = 0.f;
    sc.err = INFINITY;
    sc.head = -1;
  }
  return sc;
}

}  // namespace score
}  // namespace qasp
