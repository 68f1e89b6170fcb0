// 2-bit quantised KV pages: the bulk and in-step quantiser kernels and the
// attention over quantised pages (the layout, the quantiser and the
// per-wave attention are in quant_core.h).
#include "launch.h"
#include "quant_core.h"
#include "select_core.h"

namespace qasp {
namespace quant {

// One block per (logical page, sequence) (bulk: every page below P -
// residual_pages) or per sequence (step: the page leaving the residual region).
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t *__restrict__ k_pool,
                                                       const uint16_t *__restrict__ v_pool, uint8_t *__restrict__ qpool,
                                                       const int32_t *__restrict__ page_table,
                                                       const int32_t *__restrict__ seq_lens, int pt_stride, int Hkv,
                                                       int residual_pages, int step_mode) {
  constexpr int PS = 16;
  __shared__ float sm[16 * PS];
  const int b = blockIdx.y;
  const int L = seq_lens[b];
  const int P = (L + PS - 1) / PS;
  const int j = step_mode ? leaving_page(L, residual_pages) : (int)blockIdx.x;
  if (j < 0 || j >= P - residual_pages) return;  // block-uniform
  const int phys = page_table[(size_t)b * pt_stride + j];
  for (int g = 0; g < Hkv; g++) quantize_page_head(k_pool, v_pool, qpool, phys, g, Hkv, sm);
}

}  // namespace quant

// LDS of the selecting form of decode_quant_gqa_kernel (bytes): the
// selection's keys (8 bytes per page), which the quantiser before and the wave
// merge after reuse, two bit maps, the list.
struct SelectQuantLds {
  size_t bits, list, total;
  __host__ __device__ SelectQuantLds(int max_pages, int max_sel, int W, int G) {
    const size_t keys = (size_t)max_pages * 8, merge = (size_t)attend::merge_lds_floats(W, G, 128) * 4;
    size_t m = keys > merge ? keys : merge;
    if (m < 256 * 4) m = 256 * 4;  // the quantiser's staging
    bits = (m + 15) & ~(size_t)15;
    list = bits + 2 * (size_t)((max_pages + 31) / 32) * 4;
    total = list + (size_t)max_sel * 4;
  }
};

// Sparse paged attention with quantised pages: as decode_gqa_kernel (block
// (split, g, b), waves take every WAVES-th selected page), except that a
// wave's pages below P - residual_pages (its first ones: the list is
// ascending) are read from the quantised pool, the rest from the bf16 pools.
// SELECT: the kernel chain's selection inside the same launch, as in
// select_decode_gqa_kernel: block (unit, split) in the XCD-contiguous order
// of a one-dimensional grid; every block selects its unit's pages from the
// stored scores (the first split also writes sel / sel_count), then attends
// its split of the list.  Otherwise sel / sel_count are read.
template <int WAVES, bool SELECT>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4))) void
decode_quant_gqa_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_pool, const uint16_t *__restrict__ v_pool,
    const uint8_t *__restrict__ qpool, const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    int32_t *__restrict__ sel, int32_t *__restrict__ sel_count, float *__restrict__ partial,
    float2 *__restrict__ partial_ml, float *__restrict__ out, int pt_stride, int max_sel, int Hq, int Hkv, int G,
    int splits, int pps, float scale_log2, int sink_tokens, int window_tokens, uint64_t static_mask,
    int residual_pages, uint8_t *__restrict__ qpool_w, const uint16_t *__restrict__ k_pool_q,
    const uint16_t *__restrict__ v_pool_q, const qasp_score *__restrict__ scores, const uint16_t *__restrict__ summ,
    int max_pages, int n_sink, int n_local, int top_k) {
  constexpr int PS = 16, D = 128, DV = 128;
  extern __shared__ __attribute__((aligned(16))) float lds[];  // 16-byte aligned: the list is written from 16-byte key loads
  int split, g, b;
  if constexpr (SELECT) {
    const int item = xcd_contiguous_item(blockIdx.x, gridDim.x);
    split = item % splits;
    g = (item / splits) % Hkv;
    b = item / (splits * Hkv);
  } else {
    split = blockIdx.x;
    g = blockIdx.y;
    b = blockIdx.z;
  }
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int unit = b * Hkv + g;
  const int L = seq_lens[b];
  if (qpool_w != nullptr) {
    // the unit is not split: its block alone reads page-head (leaving page, g),
    // so it quantises it first (the barriers inside order the reads below)
    const int jl = quant::leaving_page(L, residual_pages);
    if (jl >= 0)  // block-uniform
      quant::quantize_page_head(k_pool_q, v_pool_q, qpool_w, page_table[(size_t)b * pt_stride + jl], g, Hkv, lds);
  }
  const int q_end = (L + PS - 1) / PS - residual_pages;  // pages below are quantised
  const bool is_static = head_is_static(static_mask, g);
  const int sink_end = is_static ? min(sink_tokens, L) : 0;
  const int win_begin = is_static ? max(0, L - window_tokens) : 0;
  const size_t head0 = (size_t)b * Hq + (size_t)g * G;
  const int32_t *list = sel + (size_t)unit * max_sel;
  int count;
  if constexpr (SELECT) {
    __shared__ sel::SelShared<WAVES> sh;
    const SelectQuantLds lay(max_pages, max_sel, WAVES, G);
    uint32_t *bits = (uint32_t *)((char *)lds + lay.bits);
    int32_t *lds_list = (int32_t *)((char *)lds + lay.list);
    __syncthreads();  // the quantiser above is done with the LDS
    count = sel::select_unit<D, WAVES>(sh, (uint64_t *)lds, bits, (max_pages + 31) / 32, scores + (size_t)unit * max_pages,
                                       L, PS, is_static, n_sink, n_local, top_k, sink_tokens, window_tokens, q + head0 * D,
                                       G, summ, page_table + (size_t)b * pt_stride, Hkv, g,
                                       split == 0 ? sel + (size_t)unit * max_sel : nullptr, lds_list, max_sel);
    if (split == 0 && threadIdx.x == 0) sel_count[unit] = count;
    __syncthreads();  // the list is complete; the keys are dead
    list = lds_list;
  } else {
    count = sel_count[unit];
  }
  const int first = split * pps, last = min(first + pps, count);
  const int npg = max(0, (last - first - wave + WAVES - 1) / WAVES);
  int my_j = 0, my_phys = 0;
  if (lane < npg) {
    my_j = list[first + wave + WAVES * lane];
    my_phys = page_table[(size_t)b * pt_stride + my_j];
  }
  uint4 bq[D / 32];
  attend::load_q_columns<D>(bq, q + head0 * D, G, lane);
  attend::WaveState st;
  attend::init_state(st);
  quant::attend_wave_quant(st, bq, npg, my_j, my_phys, q_end, qpool, k_pool, v_pool, Hkv, g, L, is_static, sink_end,
                           win_begin, scale_log2, lane);
  attend::merge_waves<WAVES, DV>(lds, st, G, [&](int h, int dv, float a, float lsum, float M) {
    if (splits == 1) {
      out[(head0 + h) * DV + dv] = lsum > 0.f ? a / lsum : 0.f;
    } else {
      const size_t ps_idx = (head0 + h) * splits + split;
      partial[ps_idx * DV + dv] = a;
      if (dv == 0) partial_ml[ps_idx] = make_float2(M, lsum);
    }
  });
}

hipError_t launch_quantize(const qasp_layout &lay, const qasp_batch &bat, int residual_pages, bool step_mode,
                           const uint16_t *k_pool, const uint16_t *v_pool, uint8_t *qpool, hipStream_t stream) {
  if (bat.batch == 0 || bat.max_pages == 0) return hipSuccess;
  dim3 grid(step_mode ? 1 : bat.max_pages, bat.batch);
  hipLaunchKernelGGL(quant::quantize_kernel, grid, dim3(256), 0, stream, k_pool, v_pool, qpool, bat.page_table,
                     bat.seq_lens, bat.pt_stride, lay.num_kv_heads, residual_pages, step_mode ? 1 : 0);
  return hipGetLastError();
}

// the selecting form runs 8 waves (two per SIMD: the selection needs more than
// the 128 registers of four waves per SIMD)
constexpr int kSelectQuantWaves = 8;

size_t select_quant_lds_bytes(const qasp_layout &lay, const qasp_batch &bat, int max_sel) {
  const int G = bat.num_q_heads / lay.num_kv_heads;
  return SelectQuantLds(bat.max_pages > 0 ? bat.max_pages : 1, max_sel, kSelectQuantWaves, G).total +
         sizeof(sel::SelShared<kSelectQuantWaves>);
}

// scores != nullptr: the blocks select first (sel / sel_count, then written,
// receive the selection); else sel / sel_count are the given selection.
hipError_t launch_decode_quant_gqa(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                                   int residual_pages, const uint16_t *q, const uint16_t *k_pool,
                                   const uint16_t *v_pool, const uint8_t *qpool, const int32_t *sel,
                                   const int32_t *sel_count, int max_sel, float scale, float *out,
                                   const Workspace &ws, hipStream_t stream, const qasp_score *scores,
                                   const uint16_t *summ, bool quantised_before) {
  constexpr int W = 16;  // 16 waves per block, four per SIMD: a quantised page is short work, latency needs hiding
  if (bat.batch == 0) return hipSuccess;
  const int G = bat.num_q_heads / lay.num_kv_heads;
  const float scale_log2 = scale * 1.4426950408889634f;
  const int pps = (max_sel + ws.splits - 1) / ws.splits;
  const size_t lds = (size_t)std::max(attend::merge_lds_floats(W, G, 128), 256) * sizeof(float);
  dim3 grid(ws.splits, lay.num_kv_heads, bat.batch);
  // the page-head leaving the residual region: quantised by the scoring kernel
  // before (quantised_before), else, with one block per unit, by the block
  // itself, otherwise by the in-step quantiser launched first
  const bool fold = !quantised_before && ws.splits == 1;
  if (!quantised_before && !fold) {
    hipError_t e = launch_quantize(lay, bat, residual_pages, true, k_pool, v_pool, (uint8_t *)qpool, stream);
    if (e != hipSuccess) return e;
  }
  if (scores != nullptr) {
    const int mp = bat.max_pages > 0 ? bat.max_pages : 1;
    constexpr int WS = kSelectQuantWaves;
    const size_t slds = SelectQuantLds(mp, max_sel, WS, G).total;
    hipLaunchKernelGGL((decode_quant_gqa_kernel<WS, true>), dim3((unsigned)ws.splits * lay.num_kv_heads * bat.batch),
                       dim3(WS * 64), slds, stream, q, k_pool, v_pool, qpool, bat.page_table, bat.seq_lens,
                       (int32_t *)sel, (int32_t *)sel_count, ws.partial, ws.partial_ml, out, bat.pt_stride, max_sel,
                       bat.num_q_heads, lay.num_kv_heads, G, ws.splits, pps, scale_log2, pol.sink_tokens,
                       pol.window_tokens, pol.static_head_mask, residual_pages, fold ? (uint8_t *)qpool : nullptr,
                       k_pool, v_pool, scores, summ, mp, pol.n_sink_pages, pol.n_local_pages, pol.top_k);
  } else {
    hipLaunchKernelGGL((decode_quant_gqa_kernel<W, false>), grid, dim3(W * 64), lds, stream, q, k_pool, v_pool,
                       qpool, bat.page_table, bat.seq_lens, (int32_t *)sel, (int32_t *)sel_count, ws.partial,
                       ws.partial_ml, out, bat.pt_stride, max_sel, bat.num_q_heads, lay.num_kv_heads, G, ws.splits,
                       pps, scale_log2, pol.sink_tokens, pol.window_tokens, pol.static_head_mask, residual_pages,
                       fold ? (uint8_t *)qpool : nullptr, k_pool, v_pool, nullptr, nullptr, 0, 0, 0, 0);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ws.splits == 1) return e;
  return launch_merge_splits(ws, bat.batch, bat.num_q_heads, lay.head_dim_v, out, stream);
}

}  // namespace qasp
