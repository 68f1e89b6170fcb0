// Page-summary kernels: bulk build and append-with-update.
//
// A page summary is the elementwise minimum and maximum of the keys of the
// page's valid tokens (the per-page key metadata a decode-time query-aware
// page selector reads; SparseEngine article, blog.ontle.kr/blog/332, the
// decode-hook paragraph on Quest).  min/max are taken in a total order
// (-0 below +0) on 16-bit order keys, two channels per dword.
#include "common.h"
#include "launch.h"

namespace qasp {

// Elementwise min / max of two bf16 pairs packed in dwords.
__device__ __forceinline__ void minmax_bf16x2(uint32_t v, uint32_t &lo, uint32_t &hi) {
  int v0 = bf16_order_key(v & 0xffffu), v1 = bf16_order_key(v >> 16);
  int l0 = bf16_order_key(lo & 0xffffu), l1 = bf16_order_key(lo >> 16);
  int h0 = bf16_order_key(hi & 0xffffu), h1 = bf16_order_key(hi >> 16);
  lo = bf16_from_order_key(min(v0, l0)) | (bf16_from_order_key(min(v1, l1)) << 16);
  hi = bf16_from_order_key(max(v0, h0)) | (bf16_from_order_key(max(v1, h1)) << 16);
}

// One block per (logical page, sequence); threads stride over
// (KV head, channel pair).  Consecutive threads read consecutive dwords of a
// token row, so each token row of a page-head is one contiguous read.
__global__ __launch_bounds__(256) void build_summaries_kernel(
    const uint32_t *__restrict__ k_pool, uint32_t *__restrict__ summ,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    int pt_stride, int ps, int num_kv_heads, int head_dim_k) {
  const int b = blockIdx.y, j = blockIdx.x;
  const int L = seq_lens[b];
  if (j >= num_pages_of(L, ps)) return;
  const int phys = page_table[(size_t)b * pt_stride + j];
  const int valid = min(ps, L - j * ps);
  const int words = head_dim_k / 2;
  for (int item = threadIdx.x; item < num_kv_heads * words; item += blockDim.x) {
    const int g = item / words, w = item % words;
    const size_t ph = (size_t)phys * num_kv_heads + g;
    const uint32_t *kp = k_pool + ph * ps * words + w;
    uint32_t lo = kp[0], hi = lo;
    for (int t = 1; t < valid; t++) minmax_bf16x2(kp[(size_t)t * words], lo, hi);
    const size_t sr = summ_record(phys, g, num_kv_heads);
    summ[sr * 2 * words + w] = lo;
    summ[sr * 2 * words + words + w] = hi;
  }
}

// One block per sequence: writes the new token at position seq_lens[b] +
// pos_offset and folds its key into the page summary (slot 0 starts it).
__global__ __launch_bounds__(256) void append_kv_kernel(TokenAppend ap, const int32_t *__restrict__ page_table,
                                                        const int32_t *__restrict__ seq_lens, int pos_offset,
                                                        int pt_stride) {
  const int b = blockIdx.x;
  const int pos = seq_lens[b] + pos_offset;
  if (pos < 0) return;
  const int phys = page_table[(size_t)b * pt_stride + pos / ap.ps];
  ap.run(b, 0, ap.num_kv_heads, phys, pos % ap.ps, threadIdx.x, blockDim.x);
}

hipError_t launch_build_summaries(const qasp_layout &lay, const qasp_batch &bat,
                                  const uint16_t *k_pool, uint16_t *summ, hipStream_t stream) {
  if (bat.batch == 0 || bat.max_pages == 0) return hipSuccess;
  dim3 grid(bat.max_pages, bat.batch);
  hipLaunchKernelGGL(build_summaries_kernel, grid, dim3(256), 0, stream,
                     (const uint32_t *)k_pool, (uint32_t *)summ, bat.page_table, bat.seq_lens,
                     bat.pt_stride, lay.page_size, lay.num_kv_heads, lay.head_dim_k);
  return hipGetLastError();
}

TokenAppend token_append(const qasp_layout &lay, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                         uint16_t *v_pool, uint16_t *summ) {
  return TokenAppend{(const uint32_t *)k_new, lay.v_from_k ? nullptr : v_new, (uint32_t *)k_pool,
                     lay.v_from_k ? nullptr : v_pool, (uint32_t *)summ, lay.num_kv_heads, lay.head_dim_k,
                     lay.head_dim_v, lay.page_size};
}

hipError_t launch_append_kv(const qasp_layout &lay, const qasp_batch &bat, int pos_offset,
                            const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                            uint16_t *v_pool, uint16_t *summ, hipStream_t stream) {
  if (bat.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kv_kernel, dim3(bat.batch), dim3(256), 0, stream,
                     token_append(lay, k_new, v_new, k_pool, v_pool, summ), bat.page_table, bat.seq_lens,
                     pos_offset, bat.pt_stride);
  return hipGetLastError();
}

}  // namespace qasp
