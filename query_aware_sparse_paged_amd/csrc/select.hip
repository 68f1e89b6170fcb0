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
  extern __shared__ __attribute__((aligned(16))) uint64_t dyn[];  // 16-byte aligned: the list is written from 16-byte key loads
  __shared__ sel::SelShared<NW> sh;
  const int g = blockIdx.x, b = blockIdx.y;
  const int unit = b * Hkv + g;
  const int nwords = (max_pages + 31) / 32;
  const int count = sel::select_unit<D, NW>(
      sh, dyn, (uint32_t *)(dyn + max_pages), nwords, scores + (size_t)unit * max_pages, seq_lens[b], ps,
      head_is_static(static_mask, g), n_sink, n_local, top_k, sink_tokens, window_tokens,
      q + ((size_t)b * Hq + (size_t)g * G) * D, G, summ, page_table + (size_t)b * pt_stride, Hkv, g,
      sel + (size_t)unit * max_sel, nullptr, max_sel);
  if (threadIdx.x == 0) sel_count[unit] = count;
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
