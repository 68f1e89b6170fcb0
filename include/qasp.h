/*
 * qasp: one decode step of query-aware sparse attention over a paged KV cache,
 * as HIP kernels for AMD CDNA4 (gfx950), behind a C ABI.
 *
 * The method (as the pages describe it):
 *   - the KV cache lives in fixed-size pages scattered through a pool and
 *     reached through a page table (Vortex explainer, gist.science paper
 *     2606.06453, section 1: the "paged" library whose boxes are not
 *     contiguous, and the map that finds the boxes one asks for);
 *   - at decode time the pages to read are chosen from the current query
 *     (SparseEngine article, blog.ontle.kr/blog/332, the decode-hook paragraph
 *     naming Quest; the "dynamic sparse attention" family that keeps every
 *     token and reads only what the query needs);
 *   - choosing is logical: nothing is evicted, only the read set shrinks
 *     (same article, the paragraph separating "not looking" from "discarding");
 *   - static heads use the A-shape pattern, sink tokens plus a local window,
 *     with no scoring (SCBench notes, notes.yuuk.io, "Tri-shape" paragraph);
 *   - attention is computed exactly on the chosen positions (SubQ/SSA
 *     article, news.neo-ai.one/ja/article/2719, section "How SSA works").
 * Page summaries are the elementwise min and max of a page's keys; a page's
 * score is the group maximum of sum_d max(q_d lo_d, q_d hi_d), an upper bound
 * on q.k for every key in the page.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns and
 *     allocates every buffer; the library never allocates device memory.
 *     k_pool / v_pool may also be the device pointer of a host-tier
 *     allocation (qasp_host_alloc): the kernels then read the selected pages,
 *     and write the appended tokens, over the host link.
 *   - bf16 tensors are passed as their raw 16-bit patterns (uint16_t).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting for it.
 *   - Return value: QASP_OK (0) or a negative qasp_status.  Argument checks run
 *     on the host before anything is enqueued, so an error return means no
 *     work was queued.  QASP_ERR_LAUNCH reports hipGetLastError after a launch.
 *   - Device-side data (page-table entries, sequence lengths, a selection
 *     passed in) is read by the kernels as given.  Outside validate mode, page
 *     ids outside [0, num_pool_pages), lengths above max_pages * page_size and
 *     selected ids outside [0, ceil(seq_lens[b] / page_size)) are undefined
 *     behaviour.  Validate mode: with the environment variable QASP_VALIDATE
 *     set (and not "0"), every call that reads the pools through the page
 *     table first runs qasp_check_batch on its stream (a kernel that reads
 *     only seq_lens, the page-table rows and the selection, then a stream
 *     synchronisation) and returns QASP_ERR_BAD_PAGE_TABLE, with nothing
 *     else enqueued, when it finds an entry out of range.  Inputs must be
 *     finite.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef QASP_H
#define QASP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QASP_OK = 0,
    QASP_ERR_NULL_ARG = -1,        /* a required pointer is NULL              */
    QASP_ERR_BAD_SHAPE = -2,       /* negative size, inconsistent dimensions  */
    QASP_ERR_UNSUPPORTED = -3,     /* a shape the kernels are not built for   */
    QASP_ERR_WORKSPACE = -4,       /* workspace smaller than qasp_workspace_bytes */
    QASP_ERR_MAX_SEL = -5,         /* max_sel below qasp_max_sel             */
    QASP_ERR_LAUNCH = -6,          /* a HIP launch failed                     */
    QASP_ERR_ALLOC = -7,           /* a host-tier allocation failed           */
    QASP_ERR_BAD_PAGE_TABLE = -8,  /* validate mode / qasp_check_batch: a length,
                                      page-table entry or selected id is out
                                      of range                                */
    QASP_ERR_SCRATCH = -9          /* qasp_decode_step_noalloc: the call needs
                                      more than qasp_scratch_bytes()          */
} qasp_status;

/* Pool layout (row-major, bf16):
 *   k_pool   [num_pool_pages][num_kv_heads][page_size][head_dim_k]
 *   v_pool   [num_pool_pages][num_kv_heads][head_dim_v][page_size]
 *            (token index fastest inside a page-head), or NULL when
 *            v_from_k = 1: the value of a token is then the first head_dim_v
 *            channels of its key (one latent vector per token, as in MLA).
 *   summ     [num_pool_pages][num_kv_heads][2][head_dim_k] records,
 *            row 0 = elementwise minimum, row 1 = elementwise maximum of the
 *            keys of the page's valid tokens, with -0 ordered below +0; the
 *            record of KV head g of physical page p is in slot
 *            (g + p) mod num_kv_heads of row p (the library writes and reads
 *            it there; the rotation spreads every head's records over all
 *            the offsets of a row).
 * Supported shapes:
 *   grouped-query: page_size 16, head_dim_k = head_dim_v = 128,
 *                  1 <= num_q_heads / num_kv_heads <= 16, num_kv_heads <= 64;
 *   latent (MLA):  page_size 64, head_dim_k 576, head_dim_v 512, v_from_k = 1,
 *                  num_kv_heads = 1, num_q_heads = 128.                      */
typedef struct {
    int32_t num_pool_pages;
    int32_t page_size;
    int32_t num_kv_heads;
    int32_t head_dim_k;
    int32_t head_dim_v;
    int32_t v_from_k;
} qasp_layout;

/* A batch of decoding sequences.
 *   page_table [batch][pt_stride] int32: logical page j of sequence b is
 *              physical page page_table[b * pt_stride + j];
 *   seq_lens   [batch] int32: tokens in the cache, the current token included
 *              (an append with seq_lens = L writes position L);
 *   max_pages  host-side bound: every ceil(seq_lens[b] / page_size) is
 *              <= max_pages <= pt_stride.  It sizes scores and grids.
 * Query q is [batch][num_q_heads][head_dim_k] bf16; q head h reads KV head
 * h / (num_q_heads / num_kv_heads). */
typedef struct {
    int32_t batch;
    int32_t num_q_heads;
    int32_t pt_stride;
    int32_t max_pages;
    const int32_t *page_table;
    const int32_t *seq_lens;
} qasp_batch;

/* Which pages each KV head reads (logical page ids, per sequence):
 *   query-aware heads: sink pages [0, n_sink_pages), the local pages
 *       [P - n_local_pages, P) (the last one may be partial), and the top_k
 *       remaining pages by score; equal scores go to the lower page id.
 *   static heads (bit g of static_head_mask set): the tokens t < sink_tokens
 *       and t >= L - window_tokens; every page holding one is read, the other
 *       tokens of those pages are masked.  Static heads need no summaries. */
typedef struct {
    int32_t n_sink_pages;
    int32_t n_local_pages;
    int32_t top_k;
    int32_t sink_tokens;
    int32_t window_tokens;
    uint64_t static_head_mask;
} qasp_policy;

/* Scores as produced by qasp_score_pages: an fp32 approximation of the exact
 * group score and a bound on its error, |value - exact| <= err.  head is the
 * index, inside the KV head's group, of the query head that certainly
 * attains the group maximum (its approximate bound leads every other head's
 * by more than twice the error bound), or -1 when that is not certain; the
 * exact re-scoring in qasp_select_topk then evaluates only that head.
 * Pages that are not candidates hold value = -inf, err = 0, head = -1. */
typedef struct {
    float value;
    float err;
    int32_t head;
    int32_t reserved;  /* 0 */
} qasp_score;

/* Library version, "major.minor.patch". */
const char *qasp_version(void);

/* Human-readable text for a status code (static storage). */
const char *qasp_status_string(int32_t status);

/* Largest number of pages any KV head can select under `pol`
 * (n_sink + n_local + top_k for query-aware heads; for static heads the pages
 * that sink_tokens and window_tokens can touch), capped at max_pages.
 * Returns a negative status for invalid arguments. */
int32_t qasp_max_sel(const qasp_layout *lay, const qasp_policy *pol, int32_t max_pages);

/* Bytes of device workspace qasp_decode_step and qasp_sparse_paged_decode need
 * (scores, selections and the split partials of the attention).  Its content
 * needs no initialisation.  Returns 0 on invalid arguments. */
size_t qasp_workspace_bytes(const qasp_layout *lay, const qasp_batch *bat,
                            const qasp_policy *pol, int32_t max_sel);

/* Summaries of every page of every sequence (logical pages
 * [0, ceil(seq_lens[b] / page_size))), computed from k_pool and written into
 * summ at the physical pages.  Use after a prefill or to rebuild.  Only the
 * valid tokens of a partial last page enter its summary.
 * Defined by: the per-page key metadata a decode-time query-aware page
 * selector reads (SparseEngine article, blog.ontle.kr/blog/332, decode-hook
 * paragraph naming Quest); the summary as elementwise min / max of the keys is
 * the reading this library takes (the pages print no formula). */
int32_t qasp_build_summaries(const qasp_layout *lay, const qasp_batch *bat,
                             const uint16_t *k_pool, uint16_t *summ, void *stream);

/* Appends one token per sequence at position seq_lens[b] (the length BEFORE
 * the append; the caller increments it afterwards) and updates that page's
 * summary: a token in slot 0 starts the summary, later tokens widen it.
 *   k_new [batch][num_kv_heads][head_dim_k], v_new [batch][num_kv_heads]
 *   [head_dim_v] (ignored and may be NULL when v_from_k).
 * The caller has already mapped page_table[b][seq_lens[b] / page_size].
 * summ may be NULL only if every KV head is static (then no summary is kept).
 * A page being appended to must not be shared by two sequences.
 * Defined by: as qasp_build_summaries, kept current as tokens arrive
 * (SparseEngine article, decode-hook paragraph: selection happens at every
 * decode step, over a cache that grows by one token a step). */
int32_t qasp_append_kv(const qasp_layout *lay, const qasp_batch *bat_before,
                       const qasp_policy *pol, const uint16_t *k_new,
                       const uint16_t *v_new, uint16_t *k_pool, uint16_t *v_pool,
                       uint16_t *summ, void *stream);

/* Scores every candidate page of every query-aware head:
 * scores [batch][num_kv_heads][max_pages] qasp_score.
 * Defined by: Quest's query-aware page selection at decode (SparseEngine
 * article, decode-hook paragraph), page-granular (the same article's list of
 * compared systems: Vortex routes by page), the query deciding what is read
 * (its "dynamic sparse attention" paragraph: keep everything, read what the
 * query needs).  Score = the group maximum of sum_d max(q_d lo_d, q_d hi_d),
 * an upper bound on q.k over the page. */
int32_t qasp_score_pages(const qasp_layout *lay, const qasp_batch *bat,
                         const qasp_policy *pol, const uint16_t *q,
                         const uint16_t *summ, qasp_score *scores, void *stream);

/* Selects the pages to read, from the scores of qasp_score_pages.  Where the
 * fp32 scores cannot decide the top_k boundary within their error bounds, the
 * pages in doubt are re-scored exactly (the correctly rounded fp64 value of
 * the exact sum) from q and summ, so the selection equals the one the exact
 * scores give.  Output: sel [batch][num_kv_heads][max_sel] logical page ids in
 * ascending order, sel_count [batch][num_kv_heads]; entries past the count
 * are -1.  q and summ may be NULL only if every KV head is static.
 * Defined by: asking for "the top boxes" and finding them through the map
 * (Vortex explainer, gist.science paper 2606.06453, section 1); a logical
 * choice that evicts nothing (SparseEngine article, the paragraph separating
 * "not looking" from "discarding"); sink + local window as the static
 * pattern (SCBench notes, notes.yuuk.io, "Tri-shape" paragraph: A-shape). */
int32_t qasp_select_topk(const qasp_layout *lay, const qasp_batch *bat,
                         const qasp_policy *pol, const uint16_t *q,
                         const uint16_t *summ, const qasp_score *scores,
                         int32_t *sel, int32_t *sel_count, int32_t max_sel,
                         void *stream);

/* Softmax attention of every query head over the valid tokens of its KV
 * head's selected pages (static heads: only the sink and window tokens),
 * split across pages and merged: out [batch][num_q_heads][head_dim_v] fp32.
 * scale multiplies q.k before the softmax.  A head with no token gets 0.
 * workspace: >= qasp_workspace_bytes.
 * Defined by: attention computed exactly on the selected positions (SubQ/SSA
 * article, news.neo-ai.one/ja/article/2719, section "How SSA works"), the
 * pages reached through the page table (Vortex explainer, section 1); a
 * static head's tokens need nothing of the scored heads (llama.cpp
 * draft-head article, aikeizai.jp, "facts from primary sources"). */
int32_t qasp_sparse_paged_decode(const qasp_layout *lay, const qasp_batch *bat,
                                 const qasp_policy *pol, const uint16_t *q,
                                 const uint16_t *k_pool, const uint16_t *v_pool,
                                 const int32_t *sel, const int32_t *sel_count,
                                 int32_t max_sel, float scale, float *out,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);

/* One whole decode step on one stream: optional append (when k_new is not
 * NULL; bat->seq_lens is then the length AFTER the append, the token goes to
 * position seq_lens[b] - 1), scoring, selection, sparse attention and merge.
 * Scores and selections live in the workspace; sel / sel_count, when not
 * NULL, receive a copy of the selection ([batch][num_kv_heads][max_sel]).
 * Defined by: the decode hook as a whole (SparseEngine article, decode-hook
 * paragraph: the engine keeps the storage, the method decides per step which
 * pages are read; SCBench notes, complexity table: the loading class reads
 * only part of the KV per decode step). */
int32_t qasp_decode_step(const qasp_layout *lay, const qasp_batch *bat,
                         const qasp_policy *pol, const uint16_t *q,
                         const uint16_t *k_new, const uint16_t *v_new,
                         uint16_t *k_pool, uint16_t *v_pool, uint16_t *summ,
                         float scale, float *out, int32_t *sel, int32_t *sel_count,
                         int32_t max_sel, void *workspace, size_t workspace_bytes,
                         void *stream);

/* Which kernels qasp_decode_step (and the multi-query and quantised steps,
 * for their own batch shapes) launch for these arguments:
 * QASP_PATH_ONE_KERNEL, the whole step as one kernel with a block per
 * (sequence, KV head) (grouped-query layouts with at least 200 such units, or
 * with units of at most 640 KiB of summaries and selected pages each, whose
 * page list fits the kernel's on-chip arrays), or
 * QASP_PATH_CHAIN, the append / score / select / attend / merge kernels.
 * Negative status for invalid arguments.  (For timing tools: which kernel a
 * profile should show.) */
#define QASP_PATH_ONE_KERNEL 1
#define QASP_PATH_CHAIN 2
int32_t qasp_decode_step_path(const qasp_layout *lay, const qasp_batch *bat,
                              const qasp_policy *pol, int32_t max_sel);

/* qasp_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The workspace is a static array of
 * qasp_scratch_bytes() bytes (32 MiB) that the library holds on each GPU it
 * runs on until the process ends; the call allocates nothing.  Every call on
 * one GPU shares that GPU's array, so calls that overlap in time on one GPU
 * (other streams, other host threads) race and must not be issued; the array
 * keeps the last call's contents (nothing in it needs to start at zero).
 * Arguments, results and errors as qasp_decode_step, plus QASP_ERR_SCRATCH
 * (with nothing enqueued) when qasp_workspace_bytes for these arguments
 * exceeds qasp_scratch_bytes(). */
size_t qasp_scratch_bytes(void);
int32_t qasp_decode_step_noalloc(const qasp_layout *lay, const qasp_batch *bat,
                                 const qasp_policy *pol, const uint16_t *q,
                                 const uint16_t *k_new, const uint16_t *v_new,
                                 uint16_t *k_pool, uint16_t *v_pool, uint16_t *summ,
                                 float scale, float *out, int32_t *sel,
                                 int32_t *sel_count, int32_t max_sel, void *stream);

/* One decode step of a layer that reuses the page selection of an earlier
 * layer at the same step (cross-layer selection reuse: the OmniKV / DeltaKV
 * family named in the SparseEngine article's decode-hook paragraph): optional
 * append of the step's token (when k_new is not NULL; as in
 * qasp_decode_step, bat->seq_lens counts it), then softmax attention over
 * the given selection, as qasp_sparse_paged_decode.  No scoring and no
 * selection: sel / sel_count ([batch][num_kv_heads][max_sel], logical page
 * ids, read only) come from qasp_decode_step or qasp_select_topk of the
 * earlier layer and index this layer's page table and pools.  summ (may be
 * NULL) is this layer's summary pool: when given, the append keeps it
 * current.  workspace: >= qasp_workspace_bytes.  Errors as
 * qasp_decode_step. */
int32_t qasp_decode_step_reuse(const qasp_layout *lay, const qasp_batch *bat,
                               const qasp_policy *pol, const uint16_t *q,
                               const uint16_t *k_new, const uint16_t *v_new,
                               uint16_t *k_pool, uint16_t *v_pool, uint16_t *summ,
                               float scale, const int32_t *sel, const int32_t *sel_count,
                               int32_t max_sel, float *out, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Multi-query decode step: n_query draft tokens per sequence checked at once
 * (speculative decoding of multi-token-prediction drafts: the llama.cpp
 * draft-head fix article on aikeizai.jp, the section on why it matters).
 * Grouped-query layouts only (page 16, head_dim 128), with
 * (num_q_heads / num_kv_heads) * n_query <= 16 and 1 <= n_query <= 16
 * (otherwise QASP_ERR_UNSUPPORTED; n_query < 1: QASP_ERR_BAD_SHAPE).
 *   bat->seq_lens: lengths INCLUDING the drafts, which sit at positions
 *                  seq_lens[b] - n_query ... seq_lens[b] - 1.
 *   q     [batch][n_query][num_q_heads][head_dim_k] bf16.
 *   k_new [batch][n_query][num_kv_heads][head_dim_k], v_new
 *         [batch][n_query][num_kv_heads][head_dim_v] bf16, or both NULL when
 *         the drafts are already in the pools; when given they are written
 *         in order and folded into summ.
 *   out   [batch][n_query][num_q_heads][head_dim_v] fp32.
 * The drafts share one selection per (sequence, KV head), scored with the
 * maximum page bound over every draft query's heads of the group; draft i
 * attends causally (tokens at positions <= seq_lens[b] - n_query + i of the
 * selected pages); a static head's page set is the union of the drafts'
 * sink + window sets, and each draft attends its own window.  A draft with no
 * position (seq_lens[b] < n_query) is not written and gets 0.
 * max_sel >= qasp_max_sel_multi; workspace >= qasp_workspace_bytes_multi.
 * sel / sel_count: optional copy of the shared selection, as
 * qasp_decode_step.  Other errors as qasp_decode_step. */
int32_t qasp_max_sel_multi(const qasp_layout *lay, const qasp_policy *pol,
                           int32_t n_query, int32_t max_pages);
size_t qasp_workspace_bytes_multi(const qasp_layout *lay, const qasp_batch *bat,
                                  const qasp_policy *pol, int32_t n_query,
                                  int32_t max_sel);
int32_t qasp_decode_step_multi(const qasp_layout *lay, const qasp_batch *bat,
                               const qasp_policy *pol, int32_t n_query,
                               const uint16_t *q, const uint16_t *k_new,
                               const uint16_t *v_new, uint16_t *k_pool,
                               uint16_t *v_pool, uint16_t *summ, float scale,
                               float *out, int32_t *sel, int32_t *sel_count,
                               int32_t max_sel, void *workspace,
                               size_t workspace_bytes, void *stream);

/* 2-bit quantised KV pages (KIVI-style: 2 bits, groups of 32, SCBench notes'
 * method table; a quantised region kept with a full-precision residual region,
 * SparseEngine article, decode-hook paragraph).  Grouped-query layouts only
 * (page 16, head_dim 128; otherwise QASP_ERR_UNSUPPORTED).  The last
 * residual_pages (>= 1) logical pages of a sequence stay in the bf16 pools;
 * every earlier page is read from the quantised pool by the attention.
 * Scoring and selection are unchanged (summaries come from the bf16 keys).
 * Per token, each group of 32 consecutive channels of the key, and of the
 * value, has zero point m = its minimum and step s = (max - min) / 3, stored
 * as binary16; code = round-half-even((x - m) / s) clamped to 0..3 in binary32
 * (s = 0: 0); read back as m + code * s.  Keys and values must lie within the
 * binary16 range.
 *   qpool [num_pool_pages][num_kv_heads][1536] bytes, per page-head.  Codes
 *   come in 8-byte pairs of little-endian words (w0, w1) holding 16 code
 *   pairs: pair p is in word p / 8, rotated left by 2 (p % 8) bits from the
 *   position with its first code at bits 5-6 and its second at bits 21-22.
 *     [   0, 512) key codes: token t, kg < 4 at byte 32t + 8kg; pair 4i + k
 *                 (i, k < 4) = channels 32i + 8kg + 2k and 32i + 8kg + 2k + 1;
 *     [ 512, 768) key (m, s) binary16 pairs: token t, group i at 16t + 4i;
 *     [ 768,1280) value codes: n < 16, kg < 4 at byte 768 + 8(4n + kg); pair
 *                 2i + h (i < 8, h < 2) = tokens 4kg + 2h and 4kg + 2h + 1 of
 *                 channel 16i + n;
 *     [1280,1536) value pairs: token t, group g (channels 32g..) at 16t + 4g.
 * qasp_quant_pool_bytes: the size of qpool (0 for an unsupported layout).
 * qasp_quantize_pages: fills the page-heads of logical pages j < P -
 *   residual_pages of every sequence (P = pages of seq_lens[b]) from the bf16
 *   pools; run once to build the pool.
 * qasp_decode_step_quant: qasp_decode_step with quantised pages: the append
 *   (bf16, when k_new is given), then, for a sequence whose token opened a new
 *   page, page P - 1 - residual_pages (which has just left the residual
 *   region) is quantised; scoring, selection, attention.  Errors as
 *   qasp_decode_step, and QASP_ERR_BAD_SHAPE for residual_pages < 1. */
size_t qasp_quant_pool_bytes(const qasp_layout *lay);
int32_t qasp_quantize_pages(const qasp_layout *lay, const qasp_batch *bat,
                            int32_t residual_pages, const uint16_t *k_pool,
                            const uint16_t *v_pool, uint8_t *qpool, void *stream);
int32_t qasp_decode_step_quant(const qasp_layout *lay, const qasp_batch *bat,
                               const qasp_policy *pol, int32_t residual_pages,
                               const uint16_t *q, const uint16_t *k_new,
                               const uint16_t *v_new, uint16_t *k_pool,
                               uint16_t *v_pool, uint16_t *summ, uint8_t *qpool,
                               float scale, float *out, int32_t *sel,
                               int32_t *sel_count, int32_t max_sel, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Validation of the device-side batch description, on demand (validate mode
 * runs it inside every pool-reading call).  A kernel on `stream` reads only
 * seq_lens, the page-table rows and, when sel is given, sel / sel_count
 * ([batch][num_kv_heads][max_sel]); then the stream is synchronised.
 * Checks, per sequence b with L = seq_lens[b]:
 *   0 <= L <= max_pages * page_size and L + extra_tokens <= pt_stride *
 *   page_size (extra_tokens = 1 for an append at position L);
 *   0 <= page_table[b][j] < num_pool_pages for every j <
 *   ceil((L + extra_tokens) / page_size);
 *   with sel: 0 <= sel_count[b][g] <= max_sel and every listed id in
 *   [0, ceil(L / page_size)).
 * Returns QASP_OK, QASP_ERR_BAD_PAGE_TABLE, or a host-side argument error
 * (extra_tokens outside [0, 16]: QASP_ERR_BAD_SHAPE; sel without sel_count:
 * QASP_ERR_NULL_ARG).  Reads stay inside the stated array shapes, so a bad
 * table cannot make the check itself read out of bounds.
 * Defined by: the page table as the map from logical pages to scattered pool
 * pages (Vortex explainer, section 1); a guard per buffer at the interface
 * (llama.cpp draft-head article, "facts from primary sources"). */
int32_t qasp_check_batch(const qasp_layout *lay, const qasp_batch *bat, int32_t extra_tokens,
                         const int32_t *sel, const int32_t *sel_count, int32_t max_sel,
                         void *stream);

/* Host-tier KV pool (CPU-GPU cooperative loading: the full KV cache stays in
 * host RAM and each decode step loads only the pages it needs; SCBench notes,
 * the discussion of CPU-GPU cooperation for Quest / RetrievalAttention).
 * Allocates `bytes` of pinned host memory mapped into the current device's
 * address space, coherent (GPU accesses are not cached across kernels):
 * *host_ptr is its host address, *device_ptr the address kernels use (pass it
 * as k_pool / v_pool).  Summaries, page tables and workspaces stay in device
 * memory, so scoring and selection never cross the host link; the attention
 * reads only the selected pages.  Errors: QASP_ERR_NULL_ARG,
 * QASP_ERR_BAD_SHAPE (bytes == 0), QASP_ERR_ALLOC (both pointers set to
 * NULL).  Free with qasp_host_free (host_ptr); the memory must not be in use
 * by queued work. */
int32_t qasp_host_alloc(size_t bytes, void **host_ptr, void **device_ptr);
int32_t qasp_host_free(void *host_ptr);

#ifdef __cplusplus
}
#endif
#endif
