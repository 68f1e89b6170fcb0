// One whole decode step for grouped-query heads in a single kernel, used when
// every (sequence, KV head) unit can have a block of its own (units >= CUs):
//   append   the current token's key/value and its page summary (head g only);
//   score    every candidate page from the summaries (score_core.h);
//   select   sink + local + certified top-k, exact on ties (select_core.h);
//   attend   softmax attention over the selected pages (attend_core.h).
// The scores and the selection stay in LDS: no round trip through HBM and no
// kernel boundary between the steps.  Each unit's data is touched by its own
// block only, so no inter-block synchronisation is needed.
#include "attend_core.h"
#include "launch.h"
#include "quant_core.h"
#include "score_core.h"
#include "select_core.h"

namespace qasp {

// Dynamic LDS layout of the fused kernel (bytes).
struct FusedLds {
  size_t keys, phys, order, bits, list, merge, total;
  __host__ __device__ FusedLds(int max_pages, int max_sel, int G) {
    const int nwords = (max_pages + 31) / 32;
    keys = 0;                                                       // uint64 [max_pages]
    phys = keys + (size_t)max_pages * 8;                            // int32 [max_pages]: pages of the sequence
    order = phys + (size_t)max_pages * 4;                           // int32 [max_pages]: scoring order
    bits = order + (size_t)max_pages * 4;                           // 2 x uint32 [nwords]
    list = bits + (size_t)2 * nwords * 4;                           // int32 [max_sel]
    merge = (list + (size_t)max_sel * 4 + 15) & ~(size_t)15;        // float merge area
    total = merge + (size_t)attend::merge_lds_floats(kFusedWaves, G, 128) * 4;
  }
};

// The (sequence, KV head) unit of block i of the one-dimensional grid.
// Blocks are dispatched in index order, block i to shader engine i % 32
// (XCD i % 8, engine (i / 8) % 4 of it, 8 CUs each), each waiting for a free
// CU of its engine, and a block that waits holds up those behind it.
//  - One round (lpt false: no more units than CUs): block i takes sequence
//    i % B and the (i / B)-th head of the dispatch order (query-aware heads
//    first), so consecutive blocks take different sequences and a sequence's
//    heads share an XCD.
//  - Several rounds (lpt): the query-aware units come first, ranked by
//    length (longest first, ties by sequence index) and dealt to the engines
//    in a snake (rows of 32 blocks alternately left to right and right to
//    left), so every engine gets the same mix of long and short units and
//    the engines free their CUs at about the same pace; the static units,
//    all of about the same size, follow.  Needs B <= T and both unit counts
//    multiples of 32 (otherwise the one-round order).
// sm: 2T ints of LDS.  Every thread of the block returns the same unit.
template <int T>
__device__ __forceinline__ int2 unit_for_block(int i, const int32_t *seq_lens, int B, int Hkv, uint64_t static_mask,
                                               bool lpt, int *sm) {
  constexpr int kEngines = 32;
  const uint64_t all = Hkv >= 64 ? ~0ull : ((1ull << Hkv) - 1);
  const uint64_t qa = all & ~static_mask, st = all & static_mask;
  const int n_qa = __popcll(qa);
  const int nq = B * n_qa, ns = B * (Hkv - n_qa);
  if (!lpt || B > T || nq % kEngines != 0 || ns % kEngines != 0)
    return make_int2(i % B, head_in_dispatch_order(static_mask, Hkv, i / B));
  auto nth_head = [](uint64_t mask, int h) {
    for (; h > 0; h--) mask &= mask - 1;  // drop the h lowest set bits
    return __ffsll((long long)mask) - 1;
  };
  if (i >= nq) {  // block-uniform: a static unit, in sequence order (no ranking)
    const int item = i - nq;
    return make_int2(item % B, nth_head(st, item / B));
  }
  const int tid = threadIdx.x;
  const int len = tid < B ? seq_lens[tid] : 0;
  if (tid < B) sm[tid] = len;
  __syncthreads();
  if (tid < B) {
    int rank = 0;
#pragma unroll 8
    for (int u = 0; u < B; u++) {
      const int lu = sm[u];
      rank += lu > len || (lu == len && u < tid);
    }
    sm[T + rank] = tid;  // sequence of each rank
  }
  __syncthreads();
  const int row = i / kEngines, j = i % kEngines;
  const int item = row * kEngines + (row & 1 ? kEngines - 1 - j : j);  // rank among the query-aware units
  const int b = sm[T + item / n_qa];
  const int g = nth_head(qa, item % n_qa);
  __syncthreads();  // sm is free again
  return make_int2(b, g);
}

// CAUSAL: the multi-query form (n_draft draft queries x G / n_draft heads as
// the group's columns, query rows already in that order, drafts already
// appended): column n scores the tokens up to its draft's position and, for a
// static head, its own window of window_q tokens (window_tokens is then the
// drafts' union); the output goes to [B][n_draft][Hq / n_draft][DV].
// SEL_ONLY: append, score and select only (the selection is written out for
// another attention kernel; out is not touched).
// QUANT: 2-bit quantised pages (qpool) below the last residual_pages of the
// sequence: the block quantises the page-head that leaves the residual region
// at this step (no other block reads it), then each wave attends its pages,
// the quantised ones from their codes (at most 64 pages per wave).
// The n_draft draft tokens of sequence b, KV head g, appended by one wave
// (lane = key word; values two per lane) at positions L - n_draft ...: key
// rows, value columns and the page summaries (the running min / max of a
// page's drafts in registers; a draft in slot 0 starts a page).  Drafts go in
// chunks of four, each chunk's loads issued together.  draft_k
// [B][n_draft][Hkv][128], draft_v [B][n_draft][Hkv][128]; summ may be null.
__device__ __forceinline__ void append_drafts_wave(const uint16_t *__restrict__ draft_k,
                                                   const uint16_t *__restrict__ draft_v, uint16_t *__restrict__ k_pool,
                                                   uint16_t *__restrict__ v_pool, uint16_t *__restrict__ summ,
                                                   const int32_t *__restrict__ pt_row, int L, int n_draft, int b,
                                                   int g, int Hkv, int lane) {
  constexpr int PS = 16, D = 128, DV = 128;
  const int i0 = max(0, n_draft - L);  // drafts at negative positions are not written
  uint32_t lo = 0, hi = 0;
  int cur_page = -1;
  size_t cur_sr = 0;  // summary record of the current page
  for (int c0 = i0; c0 < n_draft; c0 += 4) {
    uint32_t kv[4];
    uint16_t va[4], vb[4];
    int phys[4];
#pragma unroll
    for (int d = 0; d < 4; d++) {
      const int i = min(c0 + d, n_draft - 1);
      const size_t row = ((size_t)b * n_draft + i) * Hkv + g;
      kv[d] = ((const uint32_t *)draft_k)[row * (D / 2) + lane];
      va[d] = draft_v[row * DV + lane];
      vb[d] = draft_v[row * DV + lane + kWave];
      phys[d] = pt_row[(L - n_draft + i) / PS];
    }
#pragma unroll
    for (int d = 0; d < 4; d++) {
      const int i = c0 + d;
      if (i >= n_draft) break;
      const int pos = L - n_draft + i, t = pos % PS, page = pos / PS;
      const size_t ph = (size_t)phys[d] * Hkv + g;
      ((uint32_t *)k_pool)[(ph * PS + t) * (D / 2) + lane] = kv[d];
      v_pool[(ph * DV + lane) * PS + t] = va[d];
      v_pool[(ph * DV + lane + kWave) * PS + t] = vb[d];
      if (summ == nullptr) continue;
      if (page != cur_page) {
        if (cur_page >= 0) {
          uint32_t *sp = (uint32_t *)summ + cur_sr * D;
          sp[lane] = lo;
          sp[D / 2 + lane] = hi;
        }
        cur_page = page;
        cur_sr = summ_record(phys[d], g, Hkv);
        if (t == 0) {
          lo = hi = kv[d];
          continue;
        }
        const uint32_t *sp = (const uint32_t *)summ + cur_sr * D;
        lo = sp[lane];
        hi = sp[D / 2 + lane];
      }
      const int v0 = bf16_order_key(kv[d] & 0xffffu), v1 = bf16_order_key(kv[d] >> 16);
      lo = bf16_from_order_key(min(v0, bf16_order_key(lo & 0xffffu))) |
           (bf16_from_order_key(min(v1, bf16_order_key(lo >> 16))) << 16);
      hi = bf16_from_order_key(max(v0, bf16_order_key(hi & 0xffffu))) |
           (bf16_from_order_key(max(v1, bf16_order_key(hi >> 16))) << 16);
    }
  }
  if (summ != nullptr && cur_page >= 0) {
    uint32_t *sp = (uint32_t *)summ + cur_sr * D;
    sp[lane] = lo;
    sp[D / 2 + lane] = hi;
  }
  __threadfence_block();
}

// Up to four draft tokens of one (sequence, KV head), appended by one wave in
// three parts so that their latency hides under the scoring: the rows are
// loaded in the prologue, the first page's summary once the page list is in
// LDS, and the stores (with the summaries' min / max carried across the
// drafts of a page) go after the scoring.  Needs L >= n_draft.
struct DeferredDrafts {
  static constexpr int PS = 16, D = 128, DV = 128;
  uint32_t kv[4], lo = 0, hi = 0;
  uint16_t va[4], vb[4];

  __device__ __forceinline__ void load_rows(const uint16_t *draft_k, const uint16_t *draft_v, int b, int g, int Hkv,
                                            int n_draft, int lane) {
#pragma unroll
    for (int d = 0; d < 4; d++) {
      const size_t row = ((size_t)b * n_draft + min(d, n_draft - 1)) * Hkv + g;
      kv[d] = ((const uint32_t *)draft_k)[row * (D / 2) + lane];
      va[d] = draft_v[row * DV + lane];
      vb[d] = draft_v[row * DV + lane + kWave];
    }
  }
  __device__ __forceinline__ void load_summary(const uint16_t *summ, const int32_t *page_phys, int L, int n_draft,
                                               int g, int Hkv, int lane) {
    const int p0 = L - n_draft;
    if (summ == nullptr || p0 % PS == 0) return;
    const uint32_t *sp = (const uint32_t *)summ + summ_record(page_phys[p0 / PS], g, Hkv) * D;
    lo = sp[lane];
    hi = sp[D / 2 + lane];
  }
  __device__ __forceinline__ void store(uint16_t *k_pool, uint16_t *v_pool, uint16_t *summ, const int32_t *page_phys,
                                        int L, int n_draft, int g, int Hkv, int lane) {
    int cur_page = (L - n_draft) / PS;
    bool started = (L - n_draft) % PS != 0;  // lo / hi hold the first page's summary
#pragma unroll
    for (int d = 0; d < 4; d++) {
      if (d >= n_draft) break;
      const int pos = L - n_draft + d, t = pos % PS, page = pos / PS;
      const size_t ph = (size_t)page_phys[page] * Hkv + g;
      ((uint32_t *)k_pool)[(ph * PS + t) * (D / 2) + lane] = kv[d];
      v_pool[(ph * DV + lane) * PS + t] = va[d];
      v_pool[(ph * DV + lane + kWave) * PS + t] = vb[d];
      if (summ == nullptr) continue;
      if (t == 0) {
        if (started) {  // the first page is complete
          uint32_t *sp = (uint32_t *)summ + summ_record(page_phys[cur_page], g, Hkv) * D;
          sp[lane] = lo;
          sp[D / 2 + lane] = hi;
        }
        cur_page = page;
        started = true;
        lo = hi = kv[d];
        continue;
      }
      const int v0 = bf16_order_key(kv[d] & 0xffffu), v1 = bf16_order_key(kv[d] >> 16);
      lo = bf16_from_order_key(min(v0, bf16_order_key(lo & 0xffffu))) |
           (bf16_from_order_key(min(v1, bf16_order_key(lo >> 16))) << 16);
      hi = bf16_from_order_key(max(v0, bf16_order_key(hi & 0xffffu))) |
           (bf16_from_order_key(max(v1, bf16_order_key(hi >> 16))) << 16);
    }
    if (summ != nullptr) {
      uint32_t *sp = (uint32_t *)summ + summ_record(page_phys[cur_page], g, Hkv) * D;
      sp[lane] = lo;
      sp[D / 2 + lane] = hi;
    }
    __threadfence_block();
  }
};

template <int D, int DV, int PS, int W, bool CAUSAL = false, bool SEL_ONLY = false, bool QUANT = false>
__global__ __launch_bounds__(W * 64) void fused_step_gqa_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    uint16_t *__restrict__ k_pool, uint16_t *__restrict__ v_pool, uint16_t *__restrict__ summ,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens, float *__restrict__ out,
    int32_t *__restrict__ sel_out, int32_t *__restrict__ sel_count_out, int pt_stride, int max_pages,
    int max_sel, int Hq, int Hkv, int G, int n_sink, int n_local, int top_k, int sink_tokens,
    int window_tokens, uint64_t static_mask, float scale_log2, uint32_t bucket_mul, int lpt, int n_draft,
    int window_q, const uint16_t *__restrict__ draft_k, const uint16_t *__restrict__ draft_v,
    uint8_t *__restrict__ qpool, int residual_pages) {
  static_assert(D == 128 && DV == 128, "append and staging assume 128 channels");
  static_assert(!(QUANT && (CAUSAL || SEL_ONLY)), "quantised pages: one-token attention");
  constexpr int NW = W, T = W * kWave;
  constexpr int KSTEPS = 2 * D / 32;
  extern __shared__ __attribute__((aligned(16))) uint64_t dyn[];  // 16-byte aligned: the list is written from 16-byte key loads
  __shared__ sel::SelShared<NW> sh;
  __shared__ uint32_t sh_kmin, sh_kmax;
  __shared__ int sh_emax;
  const FusedLds lay(max_pages, max_sel, G);
  uint64_t *keys64 = dyn;
  uint32_t *keys32 = (uint32_t *)dyn;
  const int nwords = (max_pages + 31) / 32;
  uint32_t *sel_bits = (uint32_t *)((char *)dyn + lay.bits);
  uint32_t *band_bits = sel_bits + nwords;
  int32_t *list = (int32_t *)((char *)dyn + lay.list);
  int32_t *page_phys = (int32_t *)((char *)dyn + lay.phys);
  int32_t *order = (int32_t *)((char *)dyn + lay.order);
  float *merge_area = (float *)((char *)dyn + lay.merge);

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  __shared__ int rank_sm[2 * T];
  const int2 bg = unit_for_block<T>(blockIdx.x, seq_lens, gridDim.x / Hkv, Hkv, static_mask, lpt != 0, rank_sm);
  const int b = bg.x, g = bg.y;
  const int n_col = lane & 15, kg = lane >> 4;
  const int unit = b * Hkv + g;
  const int L = seq_lens[b];
  const int P = num_pages_of(L, PS);
  const int32_t *pt_row = page_table + (size_t)b * pt_stride;
  const bool is_static = head_is_static(static_mask, g);
  const int cand_lo = min(n_sink, P), cand_hi = max(cand_lo, P - n_local);
  const int n = cand_hi - cand_lo;
  const int k = top_k;
  const bool ranked = !is_static && k > 0 && k < n;
  const size_t head0 = (size_t)b * Hq + (size_t)g * G;
  // a static head's selection is known without scores: the pages holding sink
  // tokens, [0, st_sink), and those holding window tokens, [st_win, P)
  // (st_win >= st_sink, so the two ranges do not overlap); list position i
  // is page static_page(i)
  int st_sink = 0, st_win = 0, st_count = 0;
  if (is_static) {
    const int sink_end = min(sink_tokens, L), win_begin = max(0, L - window_tokens);
    st_sink = (sink_end + PS - 1) / PS;
    st_win = max(st_sink, win_begin < L ? win_begin / PS : P);
    st_count = min(st_sink + (P - st_win), max_sel);
  }
  auto static_page = [&](int i) { return i < st_sink ? i : st_win + (i - st_sink); };

  for (int w = tid; w < nwords; w += T) {
    sel_bits[w] = 0;
    band_bits[w] = 0;
  }
  for (int w = tid; w < NW * 256; w += T) (&sh.hist[0][0])[w] = 0;
  if (tid == 0) {
    sh.nlist = 0;
    sh_kmin = ~0u;
    sh_kmax = 0u;
    sh_emax = 0;
  }
  // ---- the sequence's physical pages and the group's q rows to LDS (the
  // scoring, the exact re-scoring and the attention read them there); every
  // load of a round is issued before its results are stored
  const bool q_in_lds = (size_t)G * D * 2 <= sel::kQStageBytes;
  // (CAUSAL) deferred draft append: block-uniform
  const bool defer_drafts = CAUSAL && draft_k != nullptr && n_draft <= 4 && L >= n_draft &&
                            (L - n_draft) / PS >= cand_hi;
  DeferredDrafts drafts;
  {
    const int nq = q_in_lds ? G * D / 2 : 0;  // q words
    const uint32_t *qsrc = (const uint32_t *)(q + head0 * D);
    // CAUSAL: q is the caller's [B][n_draft][Hq / n_draft][D]; group row r is
    // head r % (G / n_draft) of draft r / (G / n_draft)
    auto q_word = [&](int wq) {
      if constexpr (CAUSAL) {
        const int per_query = G / n_draft, r = wq / (D / 2);
        const size_t row = ((size_t)b * n_draft + r / per_query) * (Hq / n_draft) + (size_t)g * per_query +
                           r % per_query;
        return ((const uint32_t *)q)[row * (D / 2) + wq % (D / 2)];
      } else {
        return qsrc[wq];
      }
    };
    // CAUSAL: the drafts' append by the last wave.  Up to four drafts whose
    // pages are no candidates: deferred (rows loaded now, stores after the
    // scoring, before the barrier that precedes any read of those pages).
    // Otherwise: written here, before the barrier below, so the scoring sees
    // their summaries.
    if constexpr (CAUSAL) {
      if (draft_k != nullptr && wave == W - 1) {
        if (defer_drafts)
          drafts.load_rows(draft_k, draft_v, b, g, Hkv, n_draft, lane);
        else
          append_drafts_wave(draft_k, draft_v, k_pool, v_pool, summ, pt_row, L, n_draft, b, g, Hkv, lane);
      }
    }
    constexpr int kPtPerRound = 8;  // page-table entries per thread a round (one round up to 4096 pages)
    for (int r0 = 0; r0 < P || r0 < kPtPerRound * nq; r0 += kPtPerRound * T) {  // and 1 q word per thread
      int v[kPtPerRound];
#pragma unroll
      for (int r = 0; r < kPtPerRound; r++) {
        const int j = r0 + r * T + tid;
        v[r] = j < P ? pt_row[j] : 0;
      }
      const int wq = r0 / kPtPerRound + tid;
      const uint32_t qv = wq < nq ? q_word(wq) : 0u;
#pragma unroll
      for (int r = 0; r < kPtPerRound; r++) {
        const int j = r0 + r * T + tid;
        if (j < P) page_phys[j] = v[r];
      }
      if (wq < nq) ((uint32_t *)sh.qstage)[wq] = qv;
    }
  }
  __syncthreads();

  // ---- append of the token at position L-1, head g, by the last wave (its
  // key row, value column and the page summary: slot 0 starts it, later slots
  // widen it).  Its loads are issued with the wave's first summary loads and
  // its stores after the scoring, so their latency is hidden; the barrier
  // after the scoring orders them before any read of the page.
  const bool appending = k_new != nullptr && L > 0;  // block-uniform
  const bool my_append = appending && wave == W - 1;
  const int a_t = appending ? (L - 1) % PS : 0;
  // set and used only under my_append (no merge with other values where the
  // branches join, so nothing waits for these loads before the stores)
  size_t a_ph, a_sr;  // page-head of the K/V pools, summary record
  uint32_t a_k, a_lo, a_hi;
  uint16_t a_v0, a_v1;
  auto append_loads = [&]() {
    a_ph = (size_t)page_phys[(L - 1) / PS] * Hkv + g;
    a_sr = summ_record(page_phys[(L - 1) / PS], g, Hkv);
    const uint32_t *krow = (const uint32_t *)(k_new + ((size_t)b * Hkv + g) * D);  // D / 2 = 64 words
    a_k = krow[lane];
    const uint16_t *vn = v_new + ((size_t)b * Hkv + g) * DV;
    a_v0 = vn[lane];
    a_v1 = vn[lane + kWave];
    // the summary rows (without summaries, the key row again: read, unused)
    const uint32_t *sl = summ != nullptr ? (const uint32_t *)summ + a_sr * D : krow;
    a_lo = sl[lane];
    a_hi = sl[(summ != nullptr ? D / 2 : 0) + lane];
  };
  auto append_stores = [&]() {
    ((uint32_t *)k_pool)[(a_ph * PS + a_t) * (D / 2) + lane] = a_k;
    v_pool[(a_ph * DV + lane) * PS + a_t] = a_v0;
    v_pool[(a_ph * DV + lane + kWave) * PS + a_t] = a_v1;
    if (summ != nullptr) {
      uint32_t lo = a_k, hi = a_k;
      if (a_t != 0) {
        const int v0 = bf16_order_key(a_k & 0xffffu), v1 = bf16_order_key(a_k >> 16);
        lo = bf16_from_order_key(min(v0, bf16_order_key(a_lo & 0xffffu))) |
             (bf16_from_order_key(min(v1, bf16_order_key(a_lo >> 16))) << 16);
        hi = bf16_from_order_key(max(v0, bf16_order_key(a_hi & 0xffffu))) |
             (bf16_from_order_key(max(v1, bf16_order_key(a_hi >> 16))) << 16);
      }
      uint32_t *sp = (uint32_t *)summ + a_sr * D;
      sp[lane] = lo;
      sp[D / 2 + lane] = hi;
    }
    __threadfence_block();
  };
  // a last page that is itself a candidate is scored with the new token in
  // its summary, so then the append completes first
  const bool early_append = appending && ranked && cand_hi == P;  // block-uniform
  if (early_append) {
    if (my_append) {
      append_loads();
      append_stores();
    }
    __syncthreads();
  }

  // ---- scoring order: each wave's first 16-page group is in candidate
  // order and its summaries are loaded now; the other candidates follow by
  // physical page, bucketed into 256 equal ranges of the pool (a counting
  // sort while those loads are in flight; the order inside a bucket is
  // whatever the LDS atomics give, which changes no result).  Every block then
  // sweeps the summary pool from low to high addresses at about the pace of
  // the others, which the memory serves faster than records in random order.
  const int ngroups = (n + 15) / 16;
  const int my_groups = ngroups > wave ? (ngroups - wave + W - 1) / W : 0;
  const int s0 = min(n, W * 16);  // positions below s0 keep candidate order
  auto cand_of = [&](int gi) {    // candidate of this lane's column in the wave's gi-th group, -1 if none
    const int s = (wave + gi * W) * 16 + n_col;
    return gi < my_groups && s < n ? (s < s0 ? s : order[s]) : -1;
  };
  auto page_of = [&](int c) { return c >= 0 ? page_phys[cand_lo + c] : -1; };
  score::QOperands<D> op;
  uint4 bs[2][KSTEPS];
  int c_cur = -1, phys_cur = -1;
  if constexpr (CAUSAL) {
    if (defer_drafts && wave == W - 1) drafts.load_summary(summ, page_phys, L, n_draft, g, Hkv, lane);
  }
  if (ranked) {
    c_cur = cand_of(0);
    phys_cur = page_of(c_cur);
    score::load_group<D>(bs[0], summ, max(phys_cur, 0), Hkv, g, lane);
    // the q operands from the LDS copy of the q rows when there is one
    if (q_in_lds)
      score::load_q_operands<D>(op, sh.qstage, G, true, lane);
    else
      score::load_q_operands<D>(op, q + head0 * D, G, true, lane);
    if (my_append && !early_append) append_loads();
    // (sh.hist is zero here and zero again after the sort)
    score::bucket_order<T>(order, page_phys + cand_lo, s0, n, bucket_mul, &sh.hist[0][0]);
  } else if (my_append) {
    append_loads();
  }

  // ---- score the candidates in that order: wave w takes 16-page groups w,
  // w+W, ...; the summaries of the next group are in flight while the current
  // group is computed (past the last group the prefetch reads page 0, unused)
  float e_loc = 0.f;
  uint32_t k_min = ~0u, k_max = 0;
  if (ranked) {
    score::score_groups<D>(op, bs, summ, Hkv, g, G, my_groups, c_cur, phys_cur, lane, cand_of, page_of,
                           [&](int c, double best, float bound) {
                             const qasp_score sc = score::make_score(best, bound);
                             const uint32_t o = sel::f32_order(sc.value);
                             keys32[c] = o;
                             k_min = min(k_min, o);
                             k_max = max(k_max, o);
                             e_loc = fmaxf(e_loc, sc.err);
                           });
    // block-wide key range and largest error bound through LDS atomics (the
    // barrier before the selection orders them)
    k_min = ~(uint32_t)wave_max_dpp((int)(~k_min ^ 0x80000000u)) ^ 0x80000000u;
    k_max = (uint32_t)wave_max_dpp((int)(k_max ^ 0x80000000u)) ^ 0x80000000u;
    e_loc = wave_max_dpp(e_loc);
    if (lane == 0) {
      atomicMin(&sh_kmin, k_min);
      atomicMax(&sh_kmax, k_max);
      atomicMax(&sh_emax, __float_as_int(e_loc));  // non-negative floats order as integers
    }
  }
  if (!early_append && my_append) append_stores();
  if constexpr (CAUSAL) {
    if (defer_drafts && wave == W - 1) drafts.store(k_pool, v_pool, summ, page_phys, L, n_draft, g, Hkv, lane);
  }
  // the append is complete and the key range / error bound are final
  __syncthreads();

  // ---- attention order: the sink and local pages of a ranked unit are known
  // before its selection, so they come first and each wave loads its first
  // one now, under the selection; the top-k pages follow.  Attention position
  // p maps to position map_pos(p) of the ascending selection list.
  const int n_known = ranked ? cand_lo + (P - cand_hi) : 0;
  const int sink_end = is_static ? min(sink_tokens, L) : 0;
  const int win_begin = is_static ? max(0, L - window_tokens) : 0;
  uint4 bq[D / 32];
  attend::load_q_columns<D>(bq, CAUSAL ? (const uint16_t *)sh.qstage : q + head0 * D, G, lane);
  int Lq = L, winq = 0;
  if constexpr (CAUSAL) {
    const int per_query = G / n_draft;
    const int i = n_col < G ? n_col / per_query : n_draft - 1;
    Lq = L - (n_draft - 1 - i);
    winq = max(0, Lq - window_q);
  }
  const attend::PageWork<PS, D, DV, CAUSAL> pw{k_pool, v_pool, bq, Hkv, g, L, sink_end, win_begin,
                                               is_static, scale_log2, Lq, winq};
  const bool pre = !QUANT && wave < (is_static ? st_count : n_known);  // wave-uniform
  // issued by every wave (a valid page when there is nothing to preload:
  // physical page 0), so the registers are always defined and the load is
  // never waited on here
  attend::PageRegs<D, DV> first;
  if constexpr (!QUANT)
    first = pw.load(pre ? page_phys[is_static ? static_page(wave) : (wave < cand_lo ? wave : cand_hi + (wave - cand_lo))]
                        : 0,
                    lane);

  // ---- select (usually no page is in doubt: then the selection is the k
  // largest keys and the list is written straight from them)
  bool fast = false;
  uint32_t uk_fast = 0;
  int32_t *sel_row = sel_out ? sel_out + (size_t)unit * max_sel : nullptr;
  int count = st_count;
  if (is_static) {  // block-uniform: the list straight from the page ranges
    for (int i = tid; i < max_sel; i += T) {
      const int j = i < st_count ? static_page(i) : -1;
      if (i < st_count) list[i] = j;
      if (sel_row) sel_row[i] = j;
    }
  } else {
    if (ranked) {
      k_min = sh_kmin;
      k_max = sh_kmax;
      e_loc = __int_as_float(sh_emax);
      fast = sel::select_candidates<D, NW>(sh, keys32, keys64, sel_bits, band_bits, n, k, cand_lo, e_loc, k_min,
                                           k_max, q_in_lds ? sh.qstage : q + head0 * D, G, summ, pt_row, Hkv, g,
                                           nullptr, page_phys + cand_lo, &uk_fast);
    }
    if (!fast)
      for (int j = tid; j < P; j += T)
        if (j < cand_lo || j >= cand_hi || (!ranked && k > 0)) atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
    __syncthreads();
    count = fast ? sel::emit_by_threshold(sh, keys32, n, uk_fast, cand_lo, cand_hi, P, sel_row, list, max_sel)
                 : sel::emit_selection(sh, sel_bits, nwords, sel_row, list, max_sel);
  }
  if (tid == 0 && sel_count_out) sel_count_out[unit] = count;
  if constexpr (SEL_ONLY) return;  // block-uniform; the unused page preload above is not emitted
  __syncthreads();
  if constexpr (QUANT) {
    // the page leaving the residual region: quantised here (the merge area is
    // free until the end); the barriers inside order it before every read
    const int jl = quant::leaving_page(L, residual_pages);
    if (jl >= 0) quant::quantize_page_head(k_pool, v_pool, qpool, page_phys[jl], g, Hkv, merge_area);
    const int npg = count > wave ? (count - wave + W - 1) / W : 0;  // positions wave, wave + W, ... (<= 64)
    int my_j = 0, my_phys = 0;
    if (lane < npg) {
      my_j = list[wave + W * lane];
      my_phys = page_phys[my_j];
    }
    attend::WaveState st;
    attend::init_state(st);
    quant::attend_wave_quant(st, bq, npg, my_j, my_phys, P - residual_pages, qpool, k_pool, v_pool, Hkv, g, L,
                             is_static, sink_end, win_begin, scale_log2, lane);
    attend::merge_waves<W, DV>(merge_area, st, G, [&](int h, int dv, float a, float lsum, float M) {
      (void)M;
      out[(head0 + h) * DV + dv] = lsum > 0.f ? a / lsum : 0.f;
    });
    return;
  }

  // ---- attend: wave w takes attention positions w, w+W, ... (a fixed
  // assignment, so the result does not depend on timing)
  auto map_pos = [&](int p) {
    if (p >= n_known) return cand_lo + (p - n_known);           // top-k, ascending
    return p < cand_lo ? p : count - (P - cand_hi) + (p - cand_lo);  // sink, then local
  };
  const int npg = count > wave ? (count - wave + W - 1) / W : 0;
  attend::WaveState st;
  attend::init_state(st);
  attend::attend_list(
      st, pw, npg, lane,
      [&](int i) {
        const int j = list[n_known > 0 ? map_pos(wave + W * i) : wave + W * i];
        return make_int2(j, page_phys[j]);
      },
      pre && npg > 0, first);
  attend::merge_waves<W, DV>(merge_area, st, G, [&](int h, int dv, float a, float lsum, float M) {
    (void)M;
    size_t row = head0 + h;
    if constexpr (CAUSAL) {
      const int per_query = G / n_draft;
      row = ((size_t)b * n_draft + h / per_query) * (Hq / n_draft) + (size_t)g * per_query + h % per_query;
    }
    out[row * DV + dv] = lsum > 0.f ? a / lsum : 0.f;
  });
}

// A decode step of a layer that reuses the page selection of an earlier
// layer (cross-layer selection reuse, SparseEngine article, decode-hook
// paragraph: the OmniKV / DeltaKV family), in one kernel per (sequence, KV
// head) block: the step's token is appended (key row, value column, page
// summary when there are summaries), then softmax attention over the given
// selection (this layer's pools, the selection's logical page ids through
// this layer's page table).  No scoring, no selection.  The token's page is a
// local page, so the append completes (barrier) before the attention.
template <int D, int DV, int PS, int W>
__global__ __launch_bounds__(W * 64) void fused_reuse_gqa_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    uint16_t *__restrict__ k_pool, uint16_t *__restrict__ v_pool, uint16_t *__restrict__ summ,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel, const int32_t *__restrict__ sel_count, float *__restrict__ out,
    int pt_stride, int max_sel, int Hq, int Hkv, int G, int sink_tokens, int window_tokens, uint64_t static_mask,
    float scale_log2, int lpt) {
  static_assert(D == 128 && DV == 128, "append and staging assume 128 channels");
  constexpr int T = W * kWave;
  __shared__ int rank_sm[2 * T];
  extern __shared__ float merge_area[];  // attend::merge_lds_floats(W, G, DV)
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int2 bg = unit_for_block<T>(blockIdx.x, seq_lens, gridDim.x / Hkv, Hkv, static_mask, lpt != 0, rank_sm);
  const int b = bg.x, g = bg.y;
  const int unit = b * Hkv + g;
  const int L = seq_lens[b];
  const int32_t *pt_row = page_table + (size_t)b * pt_stride;
  const bool is_static = head_is_static(static_mask, g);
  const size_t head0 = (size_t)b * Hq + (size_t)g * G;
  const int count = min(sel_count[unit], max_sel);
  const int npg = count > wave ? (count - wave + W - 1) / W : 0;  // positions wave, wave + W, ...
  // the wave's first 64 pages, lane i holding its i-th (issued before the append)
  const int n0 = min(npg, kWave);
  int my_j = 0, my_phys = 0;
  if (lane < n0) my_j = sel[(size_t)unit * max_sel + wave + W * lane];
  if (lane < n0) my_phys = pt_row[my_j];

  // append of the token at position L-1 by the last wave
  if (k_new != nullptr && L > 0 && wave == W - 1) {
    const int a_t = (L - 1) % PS;
    const size_t a_ph = (size_t)pt_row[(L - 1) / PS] * Hkv + g;
    const size_t a_sr = summ_record(pt_row[(L - 1) / PS], g, Hkv);
    const uint32_t *krow = (const uint32_t *)(k_new + ((size_t)b * Hkv + g) * D);  // D / 2 = 64 words
    const uint32_t a_k = krow[lane];
    const uint16_t *vn = v_new + ((size_t)b * Hkv + g) * DV;
    const uint16_t a_v0 = vn[lane], a_v1 = vn[lane + kWave];
    uint32_t a_lo = 0, a_hi = 0;
    if (summ != nullptr) {
      const uint32_t *sl = (const uint32_t *)summ + a_sr * D;
      a_lo = sl[lane];
      a_hi = sl[D / 2 + lane];
    }
    ((uint32_t *)k_pool)[(a_ph * PS + a_t) * (D / 2) + lane] = a_k;
    v_pool[(a_ph * DV + lane) * PS + a_t] = a_v0;
    v_pool[(a_ph * DV + lane + kWave) * PS + a_t] = a_v1;
    if (summ != nullptr) {
      uint32_t lo = a_k, hi = a_k;
      if (a_t != 0) {
        const int v0 = bf16_order_key(a_k & 0xffffu), v1 = bf16_order_key(a_k >> 16);
        lo = bf16_from_order_key(min(v0, bf16_order_key(a_lo & 0xffffu))) |
             (bf16_from_order_key(min(v1, bf16_order_key(a_lo >> 16))) << 16);
        hi = bf16_from_order_key(max(v0, bf16_order_key(a_hi & 0xffffu))) |
             (bf16_from_order_key(max(v1, bf16_order_key(a_hi >> 16))) << 16);
      }
      uint32_t *sp = (uint32_t *)summ + a_sr * D;
      sp[lane] = lo;
      sp[D / 2 + lane] = hi;
    }
    __threadfence_block();
  }
  __syncthreads();  // the token is in the pools before any wave reads its page

  const int sink_end = is_static ? min(sink_tokens, L) : 0;
  const int win_begin = is_static ? max(0, L - window_tokens) : 0;
  uint4 bq[D / 32];
  attend::load_q_columns<D>(bq, q + head0 * D, G, lane);
  const attend::PageWork<PS, D, DV> pw{k_pool, v_pool, bq, Hkv, g, L, sink_end, win_begin, is_static, scale_log2};
  attend::WaveState st;
  attend::init_state(st);
  attend::attend_pages<PS, D, DV>(st, pw, n0, my_j, my_phys, lane);
  // pages past the 64th of this wave (selections of more than 64 W pages)
  const int32_t *sel_row = sel + (size_t)unit * max_sel;
  for (int c0 = kWave; c0 < npg; c0 += kWave) {
    const int nc = min(npg - c0, kWave);
    int j = 0, ph = 0;
    if (lane < nc) {
      j = sel_row[wave + W * (c0 + lane)];
      ph = pt_row[j];
    }
    attend::attend_pages<PS, D, DV>(st, pw, nc, j, ph, lane);
  }
  attend::merge_waves<W, DV>(merge_area, st, G, [&](int h, int dv, float a, float lsum, float M) {
    (void)M;
    out[(head0 + h) * DV + dv] = lsum > 0.f ? a / lsum : 0.f;
  });
}

hipError_t launch_fused_reuse_gqa(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                                  const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                                  uint16_t *k_pool, uint16_t *v_pool, uint16_t *summ, float scale, float *out,
                                  const int32_t *sel, const int32_t *sel_count, int max_sel, hipStream_t stream) {
  const int G = bat.num_q_heads / lay.num_kv_heads;
  if (G > 16) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.4426950408889634f;
  const int units = bat.batch * lay.num_kv_heads;
  const int lpt = units > device_cu_count() ? 1 : 0;
  const size_t lds = (size_t)attend::merge_lds_floats(kFusedWaves, G, 128) * 4;
  hipLaunchKernelGGL((fused_reuse_gqa_kernel<128, 128, 16, kFusedWaves>), dim3(units), dim3(kFusedWaves * 64), lds,
                     stream, q, k_new, v_new, k_pool, v_pool, summ, bat.page_table, bat.seq_lens, sel, sel_count,
                     out, bat.pt_stride, max_sel, bat.num_q_heads, lay.num_kv_heads, G, pol.sink_tokens,
                     pol.window_tokens, pol.static_head_mask, scale_log2, lpt);
  return hipGetLastError();
}

size_t fused_lds_bytes(const qasp_layout &lay, const qasp_batch &bat, int max_sel) {
  const int G = bat.num_q_heads / lay.num_kv_heads;
  return FusedLds(bat.max_pages > 0 ? bat.max_pages : 1, max_sel, G).total + sizeof(sel::SelShared<kFusedWaves>);
}

hipError_t launch_fused_step_gqa(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                                 const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                                 uint16_t *k_pool, uint16_t *v_pool, uint16_t *summ, float scale, float *out,
                                 int32_t *sel, int32_t *sel_count, int max_sel, hipStream_t stream, int n_draft,
                                 int window_q, bool sel_only, const uint16_t *draft_k, const uint16_t *draft_v,
                                 uint8_t *qpool, int residual_pages) {
  const int G = bat.num_q_heads / lay.num_kv_heads;
  const int mp = bat.max_pages > 0 ? bat.max_pages : 1;
  const size_t lds = FusedLds(mp, max_sel, G).total;
  const float scale_log2 = scale * 1.4426950408889634f;
  const uint32_t bucket_mul = score::bucket_multiplier(lay.num_pool_pages);
  // several rounds of blocks: longest processing time first (see unit_for_block)
  const int units = bat.batch * lay.num_kv_heads;
  const int lpt = units > device_cu_count() ? 1 : 0;
  dim3 grid(units);
  auto kernel = sel_only           ? fused_step_gqa_kernel<128, 128, 16, kFusedWaves, false, true>
                : n_draft > 1      ? fused_step_gqa_kernel<128, 128, 16, kFusedWaves, true>
                : qpool != nullptr ? fused_step_gqa_kernel<128, 128, 16, kFusedWaves, false, false, true>
                                   : fused_step_gqa_kernel<128, 128, 16, kFusedWaves, false>;
  hipLaunchKernelGGL(kernel, grid, dim3(kFusedWaves * 64), lds, stream, q, k_new, v_new, k_pool, v_pool, summ,
                     bat.page_table, bat.seq_lens, out, sel, sel_count, bat.pt_stride, mp, max_sel, bat.num_q_heads,
                     lay.num_kv_heads, G, pol.n_sink_pages, pol.n_local_pages, pol.top_k, pol.sink_tokens,
                     pol.window_tokens, pol.static_head_mask, scale_log2, bucket_mul, lpt, n_draft, window_q, draft_k,
                     draft_v, qpool, residual_pages);
  return hipGetLastError();
}

}  // namespace qasp
