// Kernels of the multi-query decode step (nq draft tokens per sequence, as a
// speculative-decoding check of multi-token-prediction drafts needs: the
// llama.cpp draft-head fix article on aikeizai.jp, the section on why it
// matters).  The step reuses the scoring, selection and attention kernels on
// a regrouped query: the group of KV head g holds its G heads for each of the
// nq draft queries (nq * G head columns), so one selection serves every draft
// query and each selected page is read once for all of them.
//   prepare_drafts_kernel : the query into the grouped order, and the nq
//                           draft tokens (positions L - nq ... L - 1)
//                           written with their keys folded into the
//                           summaries.
// The attention kernels write the output straight into the caller's
// [B][nq][Hq][Dv] order.
#include "common.h"
#include "launch.h"

namespace qasp {

// One block per (KV head g, sequence b), 128 threads:
//   - copies the group's query rows into the grouped order: row r = i*G + h of
//     unit (b, g) is head g*G + h of draft i;
//   - when k_new is given, writes draft i's key row and value column at
//     position L - nq + i (token i of b is row b * nq + i of k_new / v_new,
//     [B][nq][Hkv][D] and [B][nq][Hkv][Dv]) and folds the keys into the page
//     summaries: thread w < D/2 owns summary word w and carries the page's
//     running min / max over the drafts in registers (a draft in slot 0
//     starts a page), writing each page's words once.
// Drafts at negative positions (L < nq) are skipped.
__global__ __launch_bounds__(128) void prepare_drafts_kernel(TokenAppend ap, const uint4 *__restrict__ q,
                                                             uint4 *__restrict__ q_grouped,
                                                             const int32_t *__restrict__ page_table,
                                                             const int32_t *__restrict__ seq_lens, int nq, int G,
                                                             int pt_stride) {
  const int g = blockIdx.x, b = blockIdx.y, Hkv = ap.num_kv_heads;
  const int row16 = ap.head_dim_k / 8;  // 16-byte words per query row
  for (int x = threadIdx.x; x < nq * G * row16; x += blockDim.x) {
    const int r = x / row16, c = x % row16, i = r / G, h = r % G;
    q_grouped[(((size_t)b * Hkv + g) * nq * G + r) * row16 + c] =
        q[(((size_t)b * nq + i) * Hkv * G + (size_t)g * G + h) * row16 + c];
  }
  if (!ap.k_new) return;
  const int L = seq_lens[b], ps = ap.ps, words = ap.head_dim_k / 2;
  const int i0 = max(0, nq - L);  // first draft with a position
  for (int w = threadIdx.x; w < words; w += blockDim.x) {
    uint32_t lo = 0, hi = 0;
    int cur_phys = -1;
    for (int i = i0; i < nq; i++) {
      const int pos = L - nq + i, t = pos % ps;
      const int phys = page_table[(size_t)b * pt_stride + pos / ps];
      const size_t ph = (size_t)phys * Hkv + g;
      const uint32_t kv = ap.k_new[(((size_t)b * nq + i) * Hkv + g) * words + w];
      ap.k_pool[(ph * ps + t) * words + w] = kv;
      if (!ap.summ) continue;
      if (phys != cur_phys) {
        if (cur_phys >= 0) {
          uint32_t *sp = ap.summ + ((size_t)cur_phys * Hkv + g) * 2 * words;
          sp[w] = lo;
          sp[words + w] = hi;
        }
        cur_phys = phys;
        if (t == 0) {
          lo = hi = kv;
          continue;
        }
        const uint32_t *sp = ap.summ + ph * 2 * words;
        lo = sp[w];
        hi = sp[words + w];
      }
      const int v0 = bf16_order_key(kv & 0xffffu), v1 = bf16_order_key(kv >> 16);
      lo = bf16_from_order_key(min(v0, bf16_order_key(lo & 0xffffu))) |
           (bf16_from_order_key(min(v1, bf16_order_key(lo >> 16))) << 16);
      hi = bf16_from_order_key(max(v0, bf16_order_key(hi & 0xffffu))) |
           (bf16_from_order_key(max(v1, bf16_order_key(hi >> 16))) << 16);
    }
    if (ap.summ && cur_phys >= 0) {
      uint32_t *sp = ap.summ + ((size_t)cur_phys * Hkv + g) * 2 * words;
      sp[w] = lo;
      sp[words + w] = hi;
    }
  }
  if (!ap.v_pool) return;
  const int DV = ap.head_dim_v;
  for (int x = threadIdx.x; x < (nq - i0) * DV; x += blockDim.x) {
    const int i = i0 + x / DV, dv = x % DV;
    const int pos = L - nq + i;
    const int phys = page_table[(size_t)b * pt_stride + pos / ps];
    ap.v_pool[(((size_t)phys * Hkv + g) * DV + dv) * ps + pos % ps] =
        ap.v_new[(((size_t)b * nq + i) * Hkv + g) * DV + dv];
  }
}

hipError_t launch_prepare_drafts(const qasp_layout &lay, const qasp_batch &bat, int nq, const uint16_t *q,
                                 uint16_t *q_grouped, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                                 uint16_t *v_pool, uint16_t *summ, hipStream_t stream) {
  if (bat.batch == 0) return hipSuccess;
  const int G = bat.num_q_heads / lay.num_kv_heads;
  hipLaunchKernelGGL(prepare_drafts_kernel, dim3(lay.num_kv_heads, bat.batch), dim3(128), 0, stream,
                     token_append(lay, k_new, v_new, k_pool, v_pool, summ), (const uint4 *)q, (uint4 *)q_grouped,
                     bat.page_table, bat.seq_lens, nq, G, bat.pt_stride);
  return hipGetLastError();
}

}  // namespace qasp
