// select_topk kernel: sink + local + top-k pages per (sequence, KV head), and
// the static A-shape page sets (sink tokens + local window; SCBench notes,
// notes.yuuk.io, "Tri-shape" paragraph).  The certified top-k with exact
// re-scoring is in select_core.h.  One block per (KV head, sequence).
#include "launch.h"
#include "select_core.h"

namespace qasp {

template <int D, int THREADS>
__global__ __launch_bounds__(THREADS) void select_topk_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ summ,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    const qasp_score *__restrict__ scores, int32_t *__restrict__ sel,
    int32_t *__restrict__ sel_count, int pt_stride, int max_pages,
    int max_sel, int Hq, int Hkv, int G, int ps, int n_sink, int n_local, int top_k,
    int sink_tokens, int window_tokens, uint64_t static_mask) {
  constexpr int NW = THREADS / kWave;
  extern __shared__ uint64_t dyn[];
  __shared__ sel::SelShared<NW> sh;
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int unit = b * Hkv + g;
  const int nwords = (max_pages + 31) / 32;
  uint64_t *keys64 = dyn;                                  // [max_pages]
  uint32_t *keys32 = (uint32_t *)dyn;                      // aliases keys64 until the band step
  uint32_t *sel_bits = (uint32_t *)(dyn + max_pages);      // [nwords]
  uint32_t *band_bits = sel_bits + nwords;                 // [nwords] (candidate index)

  const int L = seq_lens[b];
  const int P = num_pages_of(L, ps);
  const bool is_static = head_is_static(static_mask, g);
  const int cand_lo = min(n_sink, P), cand_hi = max(cand_lo, P - n_local);
  const int n = cand_hi - cand_lo;
  const int k = top_k;
  const bool ranked = !is_static && k > 0 && k < n;

  // issue the score loads first: eight per thread in flight
  constexpr int kLoadUnroll = 8;
  const qasp_score *row = scores + (size_t)unit * max_pages + cand_lo;
  float e_loc = 0.f;
  uint32_t k_min = ~0u, k_max = 0;
  if (ranked) {
    for (int i0 = 0; i0 < n; i0 += kLoadUnroll * THREADS) {
      qasp_score sc[kLoadUnroll];
#pragma unroll
      for (int u = 0; u < kLoadUnroll; u++) {
        const int i = i0 + u * THREADS + tid;
        sc[u] = i < n ? row[i] : qasp_score{-INFINITY, 0.f, -1, 0};
      }
#pragma unroll
      for (int u = 0; u < kLoadUnroll; u++) {
        const int i = i0 + u * THREADS + tid;
        if (i < n) {
          const uint32_t o = sel::f32_order(sc[u].value);
          keys32[i] = o;
          k_min = min(k_min, o);
          k_max = max(k_max, o);
          e_loc = fmaxf(e_loc, sc[u].err);
        }
      }
    }
  }
  for (int w = tid; w < nwords; w += THREADS) {
    sel_bits[w] = 0;
    band_bits[w] = 0;
  }
  for (int w = tid; w < NW * 256; w += THREADS) (&sh.hist[0][0])[w] = 0;
  if (tid == 0) sh.nlist = 0;
  __syncthreads();

  bool fast = false;
  uint32_t uk_fast = 0;
  if (is_static) {
    const int sink_end = min(sink_tokens, L);
    const int win_begin = max(0, L - window_tokens);
    for (int j = tid; j < P; j += THREADS) {
      const int a = j * ps, e = min(a + ps, L);
      if (a < sink_end || e > win_begin) atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
    }
  } else {
    if (ranked) {
      sel::block_max_min_max(e_loc, k_min, k_max, sh);
      fast = sel::select_candidates<D, NW>(sh, keys32, keys64, sel_bits, band_bits, n, k, cand_lo, e_loc, k_min,
                                           k_max, q + ((size_t)b * Hq + (size_t)g * G) * D, G, summ,
                                           page_table + (size_t)b * pt_stride, Hkv, g, row, nullptr, &uk_fast);
    }
    if (!fast)
      for (int j = tid; j < P; j += THREADS)
        if (j < cand_lo || j >= cand_hi || (!ranked && k > 0)) atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  // without pages in doubt the list comes straight from the keys
  int32_t *sel_row = sel + (size_t)unit * max_sel;
  const int count = fast ? sel::emit_by_threshold(sh, keys32, n, uk_fast, cand_lo, cand_hi, P, sel_row, nullptr, max_sel)
                         : sel::emit_selection(sh, sel_bits, nwords, sel_row, nullptr, max_sel);
  if (tid == 0) sel_count[unit] = count;
}

hipError_t launch_select_topk(const qasp_layout &lay, const qasp_batch &bat,
                              const qasp_policy &pol, const uint16_t *q, const uint16_t *summ,
                              const qasp_score *scores, int32_t *sel, int32_t *sel_count,
                              int max_sel, hipStream_t stream) {
  if (bat.batch == 0) return hipSuccess;
  const int G = bat.num_q_heads / lay.num_kv_heads;
  const int mp = bat.max_pages > 0 ? bat.max_pages : 1;
  const size_t lds = (size_t)mp * 8 + 2 * (size_t)((mp + 31) / 32) * 4;
  dim3 grid(lay.num_kv_heads, bat.batch);
#define QASP_SELECT_ARGS                                                                        \
  q, summ, bat.page_table, bat.seq_lens, scores, sel, sel_count, bat.pt_stride, mp, max_sel,    \
      bat.num_q_heads, lay.num_kv_heads, G, lay.page_size, pol.n_sink_pages, pol.n_local_pages,  \
      pol.top_k, pol.sink_tokens, pol.window_tokens, pol.static_head_mask
  // more threads for long sequences (the passes walk every candidate)
  const bool wide = mp > 2048;
  if (lay.head_dim_k == 128) {
    if (wide)
      hipLaunchKernelGGL((select_topk_kernel<128, 512>), grid, dim3(512), lds, stream, QASP_SELECT_ARGS);
    else
      hipLaunchKernelGGL((select_topk_kernel<128, 256>), grid, dim3(256), lds, stream, QASP_SELECT_ARGS);
  } else if (lay.head_dim_k == 576) {
    if (wide)
      hipLaunchKernelGGL((select_topk_kernel<576, 512>), grid, dim3(512), lds, stream, QASP_SELECT_ARGS);
    else
      hipLaunchKernelGGL((select_topk_kernel<576, 256>), grid, dim3(256), lds, stream, QASP_SELECT_ARGS);
  } else {
    return hipErrorInvalidValue;
  }
#undef QASP_SELECT_ARGS
  return hipGetLastError();
}

}  // namespace qasp
