// Kernels of the multi-query decode step (nq draft tokens per sequence, as a
// speculative-decoding check of multi-token-prediction drafts needs: the
// llama.cpp draft-head fix article on aikeizai.jp, the section on why it
// matters).  The step reuses the scoring, selection and attention kernels on
// a regrouped query: the group of KV head g holds its G heads for each of the
// nq draft queries (nq * G head columns), so one selection serves every draft
// query and each selected page is read once for all of them.
//   append_drafts_kernel : writes the nq draft tokens (positions L - nq ...
//                          L - 1) and folds their keys into the summaries.
//   swap_rows_kernel     : exchanges two middle dimensions of a
//                          [B][X][Y][chunk] array (the query into the grouped
//                          order, the output back to the caller's order).
#include "common.h"
#include "launch.h"

namespace qasp {

// One block per sequence.  Token i of b is row b * nq + i of k_new / v_new
// ([B][nq][Hkv][D] and [B][nq][Hkv][Dv]).  Every token runs the same
// item -> thread mapping, so the thread that wrote a summary word for token
// i is the one that reads it back for token i + 1 (program order, no
// barrier).  Tokens at negative positions (L < nq) are skipped.
__global__ __launch_bounds__(256) void append_drafts_kernel(TokenAppend ap, const int32_t *__restrict__ page_table,
                                                            const int32_t *__restrict__ seq_lens, int nq,
                                                            int pt_stride) {
  const int b = blockIdx.x;
  const int L = seq_lens[b];
  for (int i = 0; i < nq; i++) {
    const int pos = L - nq + i;
    if (pos < 0) continue;
    const int phys = page_table[(size_t)b * pt_stride + pos / ap.ps];
    ap.run(b * nq + i, 0, ap.num_kv_heads, phys, pos % ap.ps, threadIdx.x, blockDim.x);
  }
}

// dst[b][y][x][:] = src[b][x][y][:], chunks of `chunk` 16-byte words; one
// block per (b, x, y).
__global__ __launch_bounds__(128) void swap_rows_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                        int X, int Y, int chunk) {
  const int b = blockIdx.y, x = blockIdx.x / Y, y = blockIdx.x % Y;
  const uint4 *s = src + (((size_t)b * X + x) * Y + y) * chunk;
  uint4 *d = dst + (((size_t)b * Y + y) * X + x) * chunk;
  for (int c = threadIdx.x; c < chunk; c += blockDim.x) d[c] = s[c];
}

hipError_t launch_append_drafts(const qasp_layout &lay, const qasp_batch &bat, int nq, const uint16_t *k_new,
                                const uint16_t *v_new, uint16_t *k_pool, uint16_t *v_pool, uint16_t *summ,
                                hipStream_t stream) {
  if (bat.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(append_drafts_kernel, dim3(bat.batch), dim3(256), 0, stream,
                     token_append(lay, k_new, v_new, k_pool, v_pool, summ), bat.page_table, bat.seq_lens, nq,
                     bat.pt_stride);
  return hipGetLastError();
}

hipError_t launch_swap_rows(const void *src, void *dst, int batch, int X, int Y, size_t chunk_bytes,
                            hipStream_t stream) {
  if (batch == 0 || X == 0 || Y == 0) return hipSuccess;
  const int chunk = (int)(chunk_bytes / 16);
  hipLaunchKernelGGL(swap_rows_kernel, dim3(X * Y, batch), dim3(chunk >= 128 ? 128 : 64), 0, stream,
                     (const uint4 *)src, (uint4 *)dst, X, Y, chunk);
  return hipGetLastError();
}

}  // namespace qasp
