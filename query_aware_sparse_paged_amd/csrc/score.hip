// score_pages: the per-page upper bound on q.k from the page summaries.
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
//     |U_fp32 - U| <= 65 * 2^-23 * S * 1.01 + 2^-50
// (per MFMA at most one rounding per product and per addition, unit roundoff
// taken as 2^-23 so that a faithful rather than nearest rounding is covered;
// the fp64 additions and the final rounding to fp32 add less than 2^-23 S;
// the absolute term covers flushed subnormal operands and products when
// |q|, |k| <= 2^64).  The selection step uses this bound to decide which
// pages it must re-score exactly.
//
// Candidates are the pages between the sink and the local window; every
// other slot of a row gets value -inf, err 0.
#include "common.h"
#include "launch.h"

namespace qasp {

namespace {

constexpr int kScoreWaves = 4;
constexpr int kScoreGroupsPerWave = 4;   // 16-page groups per wave
constexpr int kScorePagesPerBlock = kScoreWaves * kScoreGroupsPerWave * 16;

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

}  // namespace

// Grouped-query scoring, head_dim D (128).  Grid: (page blocks, Hkv, B);
// block = 4 waves; wave w scores kScoreGroupsPerWave groups of 16 consecutive
// logical pages, loading group i+1 while it computes group i.  Lane l: page
// column n = l % 16, k block kg = l / 16.
template <int D>
__global__ __launch_bounds__(256) void score_gqa_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ summ,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    qasp_score *__restrict__ scores, int pt_stride, int max_pages, int Hq, int Hkv, int G,
    int ps, int n_sink, int n_local, uint64_t static_mask) {
  constexpr int K2 = 2 * D;
  constexpr int KSTEPS = K2 / 32;
  constexpr int GPW = kScoreGroupsPerWave;
  constexpr int PTR = (GPW * 16 + kWave - 1) / kWave;  // page-table registers per lane
  const int b = blockIdx.z, g = blockIdx.y;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int n = lane & 15, kg = lane >> 4;
  const bool is_static = head_is_static(static_mask, g);
  const int L = seq_lens[b];
  const int P = num_pages_of(L, ps);
  const int cand_lo = min(n_sink, P), cand_hi = max(cand_lo, P - n_local);
  qasp_score *row = scores + ((size_t)b * Hkv + g) * max_pages;
  const int wave_first = (blockIdx.x * kScoreWaves + wave) * GPW * 16;
  if (wave_first >= max_pages) return;

  // physical page of each of the wave's pages (-1: not a candidate)
  int phys_r[PTR];
#pragma unroll
  for (int r = 0; r < PTR; r++) {
    const int j = wave_first + kWave * r + lane;
    phys_r[r] = (!is_static && j >= cand_lo && j < cand_hi) ? page_table[(size_t)b * pt_stride + j] : -1;
  }
  auto phys_of = [&](int grp) {
    const int idx = grp * 16 + n;
    return __shfl(phys_r[idx / kWave], idx % kWave, kWave);
  };
  uint4 bs[2][KSTEPS];
  auto load_group = [&](int grp, uint4 *dst) {
    const int phys = phys_of(grp);
    const uint16_t *sp = summ + ((size_t)(phys < 0 ? 0 : phys) * Hkv + g) * K2 + 8 * kg;
#pragma unroll
    for (int i = 0; i < KSTEPS; i++) dst[i] = phys >= 0 ? *(const uint4 *)(sp + 32 * i) : make_uint4(0, 0, 0, 0);
  };
  load_group(0, bs[0]);

  // A operands: row m = head g*G + m of [q^-, q^+] and of its absolute value.
  uint4 aq[KSTEPS], aa[KSTEPS];
  {
    const int m = n;
    const uint16_t *qh = q + ((size_t)b * Hq + (size_t)g * G + m) * D;
#pragma unroll
    for (int i = 0; i < KSTEPS; i++) {
      const int k0 = 32 * i + 8 * kg;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < G && !is_static) v = *(const uint4 *)(qh + (k0 < D ? k0 : k0 - D));
      aq[i] = map4(v, k0 < D ? 0 : 1);
      aa[i] = map4(aq[i], 2);
    }
  }

  constexpr float kErrRel = 65.0f * 1.1920928955078125e-07f * 1.01f;  // 65 * 2^-23 * 1.01
  constexpr float kErrAbs = 8.8817841970012523e-16f;                   // 2^-50
#pragma unroll
  for (int grp = 0; grp < GPW; grp++) {
    const int j0 = wave_first + grp * 16;
    if (j0 >= max_pages) break;
    if (grp + 1 < GPW) load_group(grp + 1, bs[(grp + 1) & 1]);
    const uint4 *cur = bs[grp & 1];
    double u64[4] = {0.0, 0.0, 0.0, 0.0};
    floatx4 sa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KSTEPS; i++) {
      const floatx4 ui = mfma16x16x32(aq[i], cur[i], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; r++) u64[r] += (double)ui[r];
      sa = mfma16x16x32(aa[i], map4(cur[i], 2), sa);
    }
    // lane (n, kg) holds heads 4kg + r of page j0 + n
    double best = -INFINITY;
    float bound = 0.f;
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
    const int j = j0 + n;
    const bool is_cand = phys_of(grp) >= 0;  // cross-lane read: outside the divergent branch
    if (kg == 0 && j < max_pages) {
      qasp_score sc;
      if (is_cand) {
        const float v = (float)best;
        const float err = kErrRel * bound + kErrAbs;
        if (isfinite(v) && isfinite(err)) {
          sc.value = v == 0.f ? 0.f : v;  // no -0
          sc.err = err;
        } else {                           // overflowed: let selection re-score it
          sc.value = 0.f;
          sc.err = INFINITY;
        }
      } else {
        sc.value = -INFINITY;
        sc.err = 0.f;
      }
      row[j] = sc;
    }
  }
}

hipError_t launch_score_pages(const qasp_layout &lay, const qasp_batch &bat,
                              const qasp_policy &pol, const uint16_t *q, const uint16_t *summ,
                              qasp_score *scores, hipStream_t stream) {
  if (bat.batch == 0 || bat.max_pages == 0) return hipSuccess;
  const int G = bat.num_q_heads / lay.num_kv_heads;
  dim3 grid((bat.max_pages + kScorePagesPerBlock - 1) / kScorePagesPerBlock, lay.num_kv_heads,
            bat.batch);
  if (lay.head_dim_k == 128) {
    hipLaunchKernelGGL(score_gqa_kernel<128>, grid, dim3(256), 0, stream, q, summ, bat.page_table,
                       bat.seq_lens, scores, bat.pt_stride, bat.max_pages, bat.num_q_heads,
                       lay.num_kv_heads, G, lay.page_size, pol.n_sink_pages, pol.n_local_pages,
                       pol.static_head_mask);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qasp
