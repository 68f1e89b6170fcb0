/*
 * Plain CPU oracle for query-aware sparse attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or helper with the GPU library: every definition here
 * is written out again from the method's description.
 *
 * What it computes (one decode step, per sequence b and KV head g):
 *   - per-page key summaries: elementwise min and max of the keys of the
 *     valid tokens of each page (SparseEngine article, blog.ontle.kr/blog/332,
 *     paragraph on the decode-time hook where Quest picks the pages to read
 *     for the current query);
 *   - an upper bound on q.k per page, sum_d max(q_d*lo_d, q_d*hi_d), and the
 *     group score = max over the query heads sharing the KV head;
 *   - selection: fixed sink pages + local-window pages + the top-k scored
 *     pages, ties to the lowest logical page id (Vortex explainer,
 *     gist.science paper 2606.06453, section 1 "the paged library": ask for
 *     the most relevant boxes and let a map find them);
 *   - static A-shape heads: sink tokens + a local window, no scoring
 *     (SCBench notes, notes.yuuk.io, "Tri-shape" paragraph);
 *   - exact softmax attention over the tokens of the selected pages only
 *     (SubQ/SSA article, news.neo-ai.one/ja/article/2719, section "How SSA
 *     works": attention computed exactly on the selected positions).
 *
 * All floating point is fp64.  Group scores are the exact real sums of the
 * exact products, rounded once to fp64 (round to nearest, ties to even).
 * bf16 values travel as their raw 16-bit patterns.
 */
#ifndef QASP_ORACLE_H
#define QASP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage layout of the pools (all arrays row-major):
 *   key pool      [num_pool_pages][num_kv_heads][page_size][head_dim_k]  bf16
 *   value pool    [num_pool_pages][num_kv_heads][head_dim_v][page_size]  bf16
 *                 (token index fastest), or absent when v_from_k = 1: the
 *                 value of a token is then the first head_dim_v channels of
 *                 its key (latent KV shared by keys and values)
 *   summary pool  [num_pool_pages][num_kv_heads][2][head_dim_k]          bf16
 *                 row 0 = elementwise min, row 1 = elementwise max          */
typedef struct {
    int32_t num_pool_pages;
    int32_t page_size;
    int32_t num_kv_heads;
    int32_t head_dim_k;
    int32_t head_dim_v;
    int32_t v_from_k;
} orc_layout;

/* A batch of sequences.  Logical page j of sequence b lives in physical page
 * page_table[b * pt_stride + j].  seq_lens[b] counts the tokens in the cache,
 * the current (query) token included. */
typedef struct {
    int32_t batch;
    int32_t num_q_heads;
    int32_t pt_stride;
    const int32_t *page_table;
    const int32_t *seq_lens;
} orc_batch;

/* Which pages each KV head reads.
 *   query-aware heads: pages [0, n_sink_pages) + the last n_local_pages pages
 *                      + the top_k best-scored of the remaining pages;
 *   static heads (static_heads[g] != 0): the tokens t < sink_tokens and
 *                      t >= L - window_tokens, no scoring. */
typedef struct {
    int32_t n_sink_pages;
    int32_t n_local_pages;
    int32_t top_k;
    int32_t sink_tokens;
    int32_t window_tokens;
    const uint8_t *static_heads; /* [num_kv_heads], NULL = none static */
} orc_policy;

/* Status codes. */
#define ORC_OK 0
#define ORC_ERR_ARG (-1)      /* null pointer, bad size or out-of-range id */
#define ORC_ERR_MAX_SEL (-2)  /* max_sel smaller than a selection          */
#define ORC_ERR_RANGE (-3)    /* value outside the exact-sum result range  */

/* Correctly rounded (nearest, ties to even) sum of n finite doubles. */
double orc_exact_sum(const double *x, int64_t n, int32_t *status);

/* Summaries of every page-head referenced by the batch (logical pages
 * 0..ceil(L/page_size)-1 of each sequence), written into summ_pool at the
 * physical page.  Only valid tokens (position < L) enter the min/max.
 * Signed zeros are ordered -0 < +0. */
int32_t orc_summaries(const orc_layout *lay, const orc_batch *bat,
                      const uint16_t *k_pool, uint16_t *summ_pool);

/* Writes the new token of every sequence at position seq_lens[b] (the length
 * before the append): key into the key pool, value into the value pool
 * (ignored when v_from_k).  k_new [B][Hkv][Dk], v_new [B][Hkv][Dv]. */
int32_t orc_append(const orc_layout *lay, const orc_batch *bat_before,
                   const uint16_t *k_new, const uint16_t *v_new,
                   uint16_t *k_pool, uint16_t *v_pool);

/* Group scores, fp64, [B][Hkv][max_pages]; -inf for pages that are not
 * candidates (sink, local, beyond the sequence, or static head). */
int32_t orc_scores(const orc_layout *lay, const orc_batch *bat,
                   const orc_policy *pol, const uint16_t *q,
                   const uint16_t *summ_pool, double *scores, int32_t max_pages);

/* Selected logical pages, ascending, [B][Hkv][max_sel], and their count
 * [B][Hkv].  Query-aware heads read `scores` (as produced by orc_scores);
 * static heads ignore it.  Unused entries of sel are set to -1. */
int32_t orc_select(const orc_layout *lay, const orc_batch *bat,
                   const orc_policy *pol, const double *scores, int32_t max_pages,
                   int32_t *sel, int32_t *sel_count, int32_t max_sel);

/* Softmax attention of every query head over the valid tokens of its group's
 * selected pages (static heads: only the sink and window tokens).
 * q [B][Hq][Dk] bf16; out [B][Hq][Dv] fp64.  A head with no token gets 0. */
int32_t orc_attend(const orc_layout *lay, const orc_batch *bat,
                   const orc_policy *pol, const uint16_t *q,
                   const uint16_t *k_pool, const uint16_t *v_pool,
                   const int32_t *sel, const int32_t *sel_count, int32_t max_sel,
                   double scale, double *out);

/* One decode step (scores, selection, attention) over precomputed summaries,
 * run over (sequence, KV head) units with num_threads OpenMP threads.
 * sel / sel_count may be NULL. */
int32_t orc_decode(const orc_layout *lay, const orc_batch *bat,
                   const orc_policy *pol, const uint16_t *q,
                   const uint16_t *k_pool, const uint16_t *v_pool,
                   const uint16_t *summ_pool, double scale, double *out,
                   int32_t *sel, int32_t *sel_count, int32_t max_sel,
                   int32_t num_threads);

/* Multi-query step (speculative decoding checks several draft tokens at
 * once: the llama.cpp SWA-only draft-head fix article on aikeizai.jp, the
 * section on why it matters, which describes multi-token prediction).  The batch's
 * seq_lens count the nq draft tokens, which sit at positions L - nq ... L - 1;
 * q and out hold nq rows per head: q [B][nq][Hq][Dk], out [B][nq][Hq][Dv].
 * Readings taken: the nq queries share one selection per (sequence, KV head);
 * a page's group score is the maximum of the bound over every draft query's
 * heads of the group; query i attends causally, as a one-token step of length
 * L - nq + 1 + i would over the shared pages; a static head's page set is the
 * union of the queries' sink + window sets (one window of window_tokens +
 * nq - 1 tokens ending at L when window_tokens >= 1).  A query with no position (L - nq + 1 + i <= 0)
 * gets 0.  nq = 1 gives orc_scores / orc_select / orc_attend exactly. */
int32_t orc_scores_multi(const orc_layout *lay, const orc_batch *bat,
                         const orc_policy *pol, int32_t nq, const uint16_t *q,
                         const uint16_t *summ_pool, double *scores, int32_t max_pages);
int32_t orc_select_multi(const orc_layout *lay, const orc_batch *bat,
                         const orc_policy *pol, int32_t nq, const double *scores, int32_t max_pages,
                         int32_t *sel, int32_t *sel_count, int32_t max_sel);
int32_t orc_attend_multi(const orc_layout *lay, const orc_batch *bat,
                         const orc_policy *pol, int32_t nq, const uint16_t *q,
                         const uint16_t *k_pool, const uint16_t *v_pool,
                         const int32_t *sel, const int32_t *sel_count, int32_t max_sel,
                         double scale, double *out);

/* 2-bit quantised pages (KIVI-style: 2 bits, groups of 32; a full-precision
 * residual region of the last residual_pages logical pages).  Readings, as
 * in oracle.c: a group is 32 consecutive channels of one token; zero point =
 * group min, step = (max - min) / 3, both stored as binary16; code =
 * round-half-even((x - m) / s) clamped to 0..3 in binary32 (s = 0: 0); read
 * back as m + code * s.  Layouts (logical, one byte per code):
 *   k_codes [num_pool_pages][num_kv_heads][page_size][head_dim_k]  uint8
 *   k_meta  [num_pool_pages][num_kv_heads][page_size][head_dim_k/32][2] binary16 (m, s)
 *   v_codes / v_meta likewise with head_dim_v (token-major, groups along dv).
 * orc_quantize fills the page-heads of logical pages j < P - residual_pages
 * of every sequence (complete pages; residual_pages >= 1). */
typedef struct {
    int32_t residual_pages;
    const uint8_t *k_codes;
    const uint16_t *k_meta;
    const uint8_t *v_codes;
    const uint16_t *v_meta;
} orc_quant;
int32_t orc_quantize(const orc_layout *lay, const orc_batch *bat, int32_t residual_pages,
                     const uint16_t *k_pool, const uint16_t *v_pool, uint8_t *k_codes, uint16_t *k_meta,
                     uint8_t *v_codes, uint16_t *v_meta);
/* orc_attend with the pages j < P - residual_pages read back from the
 * quantised pool (exact m + code * s in fp64), the others from the bf16 pools. */
int32_t orc_attend_quant(const orc_layout *lay, const orc_batch *bat, const orc_policy *pol,
                         int32_t residual_pages, const uint16_t *q, const uint16_t *k_pool,
                         const uint16_t *v_pool, const uint8_t *k_codes, const uint16_t *k_meta,
                         const uint8_t *v_codes, const uint16_t *v_meta, const int32_t *sel,
                         const int32_t *sel_count, int32_t max_sel, double scale, double *out);
/* binary16 pattern nearest to x (ties to even). */
uint16_t orc_half_bits(double x);

/* Largest selection any head can need under this policy. */
int32_t orc_max_sel(const orc_layout *lay, const orc_policy *pol, int32_t max_pages);

#ifdef __cplusplus
}
#endif
#endif
