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

constexpr int kDraftsMax = 16;  // drafts per sequence (at most one page of 16 tokens)

// One block per (KV head g, sequence b), 128 threads:
//   - copies the group's query rows into the grouped order: row r = i*G + h of
//     unit (b, g) is head g*G + h of draft i;
//   - when k_new is given, writes draft i's key row and value column at
//     position L - nq + i (token i of b is row b * nq + i of k_new / v_new,
//     [B][nq][Hkv][D] and [B][nq][Hkv][Dv]) and folds the keys into the page
//     summaries.  The drafts span at most two pages (nq <= page size), whose
//     physical pages are read once; thread t loads key word t and value
//     channel t of every draft first (needs D/2 <= 128 and Dv <= 128 threads),
//     and thread w < D/2 carries summary word w's
//     running min / max over the drafts of a page in registers (a draft in
//     slot 0 starts a page), writing each page's words once.
// Drafts at negative positions (L < nq) are skipped.
__global__ __launch_bounds__(128) void prepare_drafts_kernel(TokenAppend ap, const uint4 *__restrict__ q,
                                                             uint4 *__restrict__ q_grouped,
                                                             const int32_t *__restrict__ page_table,
                                                             const int32_t *__restrict__ seq_lens, int nq, int G,
                                                             int pt_stride) {
  const int g = blockIdx.x, b = blockIdx.y, Hkv = ap.num_kv_heads, tid = threadIdx.x;
  const int words = ap.head_dim_k / 2, DV = ap.head_dim_v;
  // every draft's key word / value entry of this thread, loaded before the
  // length is known (the rows exist whatever the length)
  uint32_t kv[kDraftsMax];
  uint16_t vv[kDraftsMax];
  if (ap.k_new != nullptr) {
#pragma unroll
    for (int d = 0; d < kDraftsMax; d++) {
      kv[d] = d < nq && tid < words ? ap.k_new[(((size_t)b * nq + d) * Hkv + g) * words + tid] : 0u;
      vv[d] = d < nq && tid < DV && ap.v_new ? ap.v_new[(((size_t)b * nq + d) * Hkv + g) * DV + tid] : 0;
    }
  }
  const int L = seq_lens[b], ps = ap.ps;
  const bool writes = ap.k_new != nullptr && L > 0;
  const int i0 = max(0, nq - L);  // first draft with a position
  const int p0 = L - nq + i0;     // its position
  const int j0 = p0 / ps, t0 = p0 % ps;
  int phys0 = 0, phys1 = 0;
  if (writes) {
    phys0 = page_table[(size_t)b * pt_stride + j0];
    phys1 = page_table[(size_t)b * pt_stride + (L - 1) / ps];
  }
  const int row16 = ap.head_dim_k / 8;  // 16-byte words per query row
  for (int x = tid; x < nq * G * row16; x += blockDim.x) {
    const int r = x / row16, c = x % row16, i = r / G, h = r % G;
    q_grouped[(((size_t)b * Hkv + g) * nq * G + r) * row16 + c] =
        q[(((size_t)b * nq + i) * Hkv * G + (size_t)g * G + h) * row16 + c];
  }
  if (!writes) return;
  // drafts i0 ... nq - 1 are written (loops over compile-time indices keep
  // kv / vv in registers)
  if (tid < words) {
    const int w = tid;
    uint32_t lo = 0, hi = 0;
    if (ap.summ && t0 != 0) {  // the first page already holds tokens
      const uint32_t *sp = ap.summ + summ_record(phys0, g, Hkv) * 2 * words;
      lo = sp[w];
      hi = sp[words + w];
    }
#pragma unroll
    for (int i = 0; i < kDraftsMax; i++) {
      if (i >= nq) break;
      if (i < i0) continue;
      const int pos = L - nq + i, t = pos % ps;
      const size_t ph = (size_t)(pos / ps == j0 ? phys0 : phys1) * Hkv + g;
      const uint32_t k = kv[i];
      ap.k_pool[(ph * ps + t) * words + w] = k;
      if (!ap.summ) continue;
      if (t == 0) {
        if (i > i0) {  // the drafts cross into the second page: the first page is complete
          uint32_t *sp = ap.summ + summ_record(phys0, g, Hkv) * 2 * words;
          sp[w] = lo;
          sp[words + w] = hi;
        }
        lo = hi = k;
        continue;
      }
      const int v0 = bf16_order_key(k & 0xffffu), v1 = bf16_order_key(k >> 16);
      lo = bf16_from_order_key(min(v0, bf16_order_key(lo & 0xffffu))) |
           (bf16_from_order_key(min(v1, bf16_order_key(lo >> 16))) << 16);
      hi = bf16_from_order_key(max(v0, bf16_order_key(hi & 0xffffu))) |
           (bf16_from_order_key(max(v1, bf16_order_key(hi >> 16))) << 16);
    }
    if (ap.summ) {
      uint32_t *sp = ap.summ + summ_record((L - 1) / ps == j0 ? phys0 : phys1, g, Hkv) * 2 * words;
      sp[w] = lo;
      sp[words + w] = hi;
    }
  }
  if (!ap.v_pool || tid >= DV) return;
#pragma unroll
  for (int i = 0; i < kDraftsMax; i++) {
    if (i >= nq) break;
    if (i < i0) continue;
    const int pos = L - nq + i;
    const size_t ph = (size_t)(pos / ps == j0 ? phys0 : phys1) * Hkv + g;
    ap.v_pool[(ph * DV + tid) * ps + pos % ps] = vv[i];
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
