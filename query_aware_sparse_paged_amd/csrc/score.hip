// score_pages kernel: fp32 page scores with rigorous error bounds (see
// score_core.h) for every candidate page of every query-aware head.
// Candidates are the pages between the sink and the local window; every
// other slot of a row gets value -inf, err 0.
#include "launch.h"
#include "quant_core.h"
#include "score_core.h"

namespace qasp {

namespace {
constexpr int kScoreWaves = 4;
#ifndef QASP_SCORE_GROUPS_PER_WAVE
#define QASP_SCORE_GROUPS_PER_WAVE 4
#endif
constexpr int kScoreGroupsPerWave = QASP_SCORE_GROUPS_PER_WAVE;   // 16-page groups per wave
constexpr int kScorePagesPerBlock = kScoreWaves * kScoreGroupsPerWave * 16;
}  // namespace

// Grid: (page blocks, Hkv, B); block = 4 waves; wave w scores
// kScoreGroupsPerWave groups of 16 consecutive logical pages, loading group
// i+1 while it computes group i.  With qpool, the row's first block also
// quantises page-head (leaving page, g) of a step whose token opened a new
// page (2-bit pages: the page that leaves the residual region; no block of
// this kernel reads it, the attention launch after it does).
template <int D>
__global__ __launch_bounds__(256) void score_gqa_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ summ,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    qasp_score *__restrict__ scores, int pt_stride, int max_pages, int Hq, int Hkv, int G,
    int ps, int n_sink, int n_local, uint64_t static_mask, TokenAppend ap, uint8_t *__restrict__ qpool,
    int residual_pages, const uint16_t *__restrict__ qk_pool, const uint16_t *__restrict__ qv_pool) {
  constexpr int KSTEPS = 2 * D / 32;
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
  // the step's token (page L-1 is not a candidate here), by the row's first block
  if (ap.k_new != nullptr && blockIdx.x == 0 && L > 0)
    ap.run(b, g, g + 1, page_table[(size_t)b * pt_stride + (L - 1) / ps], (L - 1) % ps, threadIdx.x, blockDim.x);
  if (qpool != nullptr && blockIdx.x == 0) {  // block-uniform; every thread takes part (barriers inside)
    __shared__ float qsm[256];
    const int jl = quant::leaving_page(L, residual_pages);
    if (jl >= 0) quant::quantize_page_head(qk_pool, qv_pool, qpool, page_table[(size_t)b * pt_stride + jl], g, Hkv, qsm);
  }
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
  // every lane issues its loads (non-candidates read page 0 and are zeroed
  // afterwards), so the wait counts stay static
  uint4 bs[2][KSTEPS];
  score::load_group<D>(bs[0], summ, max(phys_of(0), 0), Hkv, g, lane);
  score::QOperands<D> op;
  score::load_q_operands<D>(op, q + ((size_t)b * Hq + (size_t)g * G) * D, G, !is_static, lane);

#pragma unroll
  for (int grp = 0; grp < GPW; grp++) {
    const int j0 = wave_first + grp * 16;
    if (grp + 1 < GPW) score::load_group<D>(bs[(grp + 1) & 1], summ, max(phys_of(grp + 1), 0), Hkv, g, lane);
    uint4 *cur = bs[grp & 1];
    const bool is_cand = phys_of(grp) >= 0;  // cross-lane read: outside divergent code
    if (!is_cand) {
#pragma unroll
      for (int i = 0; i < KSTEPS; i++) cur[i] = make_uint4(0, 0, 0, 0);
    }
    double best;
    float bound;
    score::score_group<D>(op, cur, G, lane, best, bound);
    const int j = j0 + n;
    if (kg == 0 && j < max_pages) row[j] = is_cand ? score::make_score(best, bound) : qasp_score{-INFINITY, 0.f, -1, 0};
  }
}

hipError_t launch_score_pages(const qasp_layout &lay, const qasp_batch &bat,
                              const qasp_policy &pol, const uint16_t *q, const uint16_t *summ,
                              qasp_score *scores, hipStream_t stream, const TokenAppend &ap, uint8_t *qpool,
                              int residual_pages, const uint16_t *k_pool, const uint16_t *v_pool) {
  if (bat.batch == 0 || bat.max_pages == 0) return hipSuccess;
  const int G = bat.num_q_heads / lay.num_kv_heads;
  dim3 grid((bat.max_pages + kScorePagesPerBlock - 1) / kScorePagesPerBlock, lay.num_kv_heads,
            bat.batch);
  if (lay.head_dim_k == 128) {
    hipLaunchKernelGGL(score_gqa_kernel<128>, grid, dim3(256), 0, stream, q, summ, bat.page_table,
                       bat.seq_lens, scores, bat.pt_stride, bat.max_pages, bat.num_q_heads,
                       lay.num_kv_heads, G, lay.page_size, pol.n_sink_pages, pol.n_local_pages,
                       pol.static_head_mask, ap, qpool, residual_pages, k_pool, v_pool);
  } else if (lay.head_dim_k == 576) {
    return launch_score_mla(lay, bat, pol, q, summ, scores, stream, ap);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qasp
