// Host-side launchers of the qasp kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qasp.h"
#include "common.h"

namespace qasp {

// Decode launch shape (tuning constants).
#ifndef QASP_GQA_WAVES
#define QASP_GQA_WAVES 8
#endif
#ifndef QASP_GQA_TARGET_BLOCKS
#define QASP_GQA_TARGET_BLOCKS 256
#endif
constexpr int kGqaDecodeWaves = QASP_GQA_WAVES;         // waves per decode block
constexpr int kGqaTargetBlocks = QASP_GQA_TARGET_BLOCKS; // split units until this many blocks
#ifndef QASP_MLA_PAGES_PER_SPLIT
#define QASP_MLA_PAGES_PER_SPLIT 8
#endif
constexpr int kMlaPagesPerSplit = QASP_MLA_PAGES_PER_SPLIT;  // selected pages per latent-head decode block
// Size of the static per-device workspace of qasp_decode_step_noalloc.
#ifndef QASP_SCRATCH_BYTES
#define QASP_SCRATCH_BYTES (32u << 20)
#endif

struct Workspace {
  qasp_score *scores;   // [B][Hkv][max_pages]
  int32_t *sel;         // [B][Hkv][max_sel]
  int32_t *sel_count;   // [B][Hkv]
  float *partial;       // [B][Hq][splits][Dv]
  float2 *partial_ml;   // [B][Hq][splits]  running max (log2 units) and sum
  int splits;
};

int decode_splits(const qasp_layout &lay, const qasp_batch &bat, int max_sel);
// Validate mode (the QASP_VALIDATE environment variable) and its check: a
// kernel reads the lengths, page-table rows and selection, then the stream is
// synchronised; QASP_OK or QASP_ERR_BAD_PAGE_TABLE.
bool validate_mode();
int32_t check_batch_on_device(const qasp_layout &lay, const qasp_batch &bat, int extra_tokens, const int32_t *sel,
                              const int32_t *sel_count, int max_sel, hipStream_t stream);
// Compute units of the current device (queried once per device).
int device_cu_count();
size_t workspace_bytes(const qasp_layout &lay, const qasp_batch &bat, int max_sel);
Workspace carve_workspace(const qasp_layout &lay, const qasp_batch &bat, int max_sel, void *base);

hipError_t launch_build_summaries(const qasp_layout &lay, const qasp_batch &bat,
                                  const uint16_t *k_pool, uint16_t *summ, hipStream_t stream);
hipError_t launch_append_kv(const qasp_layout &lay, const qasp_batch &bat, int pos_offset,
                            const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                            uint16_t *v_pool, uint16_t *summ, hipStream_t stream);
// The append of a decode step as kernel arguments (null k_new: no append).
TokenAppend token_append(const qasp_layout &lay, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                         uint16_t *v_pool, uint16_t *summ);
// Scoring; with ap.k_new set, the first block of every (sequence, KV head)
// row also appends the step's token at position L-1 (only valid when that
// page is not a candidate, i.e. n_local_pages >= 1).
// qpool (grouped-query layouts): also quantise the page-head that leaves the
// residual region of residual_pages at this step (from k_pool / v_pool)
hipError_t launch_score_pages(const qasp_layout &lay, const qasp_batch &bat,
                              const qasp_policy &pol, const uint16_t *q, const uint16_t *summ,
                              qasp_score *scores, hipStream_t stream, const TokenAppend &ap,
                              uint8_t *qpool = nullptr, int residual_pages = 0, const uint16_t *k_pool = nullptr,
                              const uint16_t *v_pool = nullptr);
hipError_t launch_score_mla(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                            const uint16_t *q, const uint16_t *summ, qasp_score *scores, hipStream_t stream,
                            const TokenAppend &ap);
hipError_t launch_select_topk(const qasp_layout &lay, const qasp_batch &bat,
                              const qasp_policy &pol, const uint16_t *q, const uint16_t *summ,
                              const qasp_score *scores, int32_t *sel, int32_t *sel_count,
                              int max_sel, hipStream_t stream);
hipError_t launch_sparse_decode(const qasp_layout &lay, const qasp_batch &bat,
                                const qasp_policy &pol, const uint16_t *q,
                                const uint16_t *k_pool, const uint16_t *v_pool,
                                const int32_t *sel, const int32_t *sel_count, int max_sel,
                                float scale, float *out, const Workspace &ws, hipStream_t stream);
// The kernel chain's selection and attention in one launch (grouped-query
// family) when its LDS fits: bytes of LDS it needs, and the launch (merge
// of the split partials included).
size_t select_decode_lds_bytes(const qasp_layout &lay, const qasp_batch &bat, int max_sel);
hipError_t launch_select_decode_gqa(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                                    const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                    const uint16_t *summ, const qasp_score *scores, int32_t *sel, int32_t *sel_count,
                                    int max_sel, float scale, float *out, const Workspace &ws, hipStream_t stream);
// The single-kernel decode step (grouped-query family), for many units.
constexpr int kFusedWaves = 8;  // waves per block of the one-kernel step
constexpr int kFusedMinUnits = 200;
constexpr int kFusedMaxPages = 4096;
// ... or fewer units, each with at most this much to read (summaries + K/V)
#ifndef QASP_FUSED_SMALL_UNIT_BYTES
#define QASP_FUSED_SMALL_UNIT_BYTES (640u << 10)
#endif
constexpr size_t kFusedSmallUnitBytes = QASP_FUSED_SMALL_UNIT_BYTES;
size_t fused_lds_bytes(const qasp_layout &lay, const qasp_batch &bat, int max_sel);
hipError_t launch_fused_step_gqa(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                                 const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                                 uint16_t *k_pool, uint16_t *v_pool, uint16_t *summ, float scale, float *out,
                                 int32_t *sel, int32_t *sel_count, int max_sel, hipStream_t stream, int n_draft = 1,
                                 int window_q = 0, bool sel_only = false, const uint16_t *draft_k = nullptr,
                                 const uint16_t *draft_v = nullptr, uint8_t *qpool = nullptr,
                                 int residual_pages = 0);
hipError_t launch_fused_reuse_gqa(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                                  const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                                  uint16_t *k_pool, uint16_t *v_pool, uint16_t *summ, float scale, float *out,
                                  const int32_t *sel, const int32_t *sel_count, int max_sel, hipStream_t stream);
// Multi-query step: the query into the grouped order ([B][Hkv][nq][G][Dk])
// and, when k_new is given, the nq draft tokens written with their summaries.
hipError_t launch_prepare_drafts(const qasp_layout &lay, const qasp_batch &bat, int nq, const uint16_t *q,
                                 uint16_t *q_grouped, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                                 uint16_t *v_pool, uint16_t *summ, hipStream_t stream);
// 2-bit quantised pages (grouped-query layouts): bytes per page-head, the
// quantiser (bulk: every page below P - residual_pages; step: the page that
// the step's token pushed out of the residual region) and the attention.
constexpr size_t kQuantPageHeadBytes = 1536;
hipError_t launch_quantize(const qasp_layout &lay, const qasp_batch &bat, int residual_pages, bool step_mode,
                           const uint16_t *k_pool, const uint16_t *v_pool, uint8_t *qpool, hipStream_t stream);
// (the attention also quantises the page that leaves the residual region at
// this step: inside its blocks when units are not split, else by a
// quantiser launch before it)
// scores != nullptr: the selection inside the same launch (sel / sel_count then receive it)
hipError_t launch_decode_quant_gqa(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                                   int residual_pages, const uint16_t *q, const uint16_t *k_pool,
                                   const uint16_t *v_pool, const uint8_t *qpool, const int32_t *sel,
                                   const int32_t *sel_count, int max_sel, float scale, float *out,
                                   const Workspace &ws, hipStream_t stream, const qasp_score *scores = nullptr,
                                   const uint16_t *summ = nullptr, bool quantised_before = false);
size_t select_quant_lds_bytes(const qasp_layout &lay, const qasp_batch &bat, int max_sel);
// Merge of the split partials; Gp (> 0) and nq map the partials' grouped
// heads to out [B][nq][Hq / nq][Dv] (nq = 1: out [B][Hq][Dv]).
hipError_t launch_merge_splits(const Workspace &ws, int batch, int Hq, int dv_dim, float *out,
                               hipStream_t stream, int nq = 1, int Gp = 0);

}  // namespace qasp
