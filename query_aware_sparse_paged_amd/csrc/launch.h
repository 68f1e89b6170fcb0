// Host-side launchers of the qasp kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qasp.h"

namespace qasp {

// Pages of one (sequence, KV head) unit handled by one decode block.
constexpr int kGqaPagesPerSplit = 32;
constexpr int kMlaPagesPerSplit = 2;

struct Workspace {
  qasp_score *scores;   // [B][Hkv][max_pages]
  int32_t *sel;         // [B][Hkv][max_sel]
  int32_t *sel_count;   // [B][Hkv]
  uint32_t *counters;   // [B][Hkv]  split-merge arrival counters, left at 0
  float *partial;       // [B][Hq][splits][Dv]
  float2 *partial_ml;   // [B][Hq][splits]  running max (log2 units) and sum
  int splits;
};

int decode_splits(const qasp_layout &lay, int max_sel);
size_t workspace_bytes(const qasp_layout &lay, const qasp_batch &bat, int max_sel);
Workspace carve_workspace(const qasp_layout &lay, const qasp_batch &bat, int max_sel, void *base);

hipError_t launch_build_summaries(const qasp_layout &lay, const qasp_batch &bat,
                                  const uint16_t *k_pool, uint16_t *summ, hipStream_t stream);
hipError_t launch_append_kv(const qasp_layout &lay, const qasp_batch &bat, int pos_offset,
                            const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                            uint16_t *v_pool, uint16_t *summ, hipStream_t stream);
hipError_t launch_score_pages(const qasp_layout &lay, const qasp_batch &bat,
                              const qasp_policy &pol, const uint16_t *q, const uint16_t *summ,
                              qasp_score *scores, hipStream_t stream);
hipError_t launch_select_topk(const qasp_layout &lay, const qasp_batch &bat,
                              const qasp_policy &pol, const uint16_t *q, const uint16_t *summ,
                              const qasp_score *scores, int32_t *sel, int32_t *sel_count,
                              int max_sel, uint32_t *counters_to_clear, hipStream_t stream);
hipError_t launch_sparse_decode(const qasp_layout &lay, const qasp_batch &bat,
                                const qasp_policy &pol, const uint16_t *q,
                                const uint16_t *k_pool, const uint16_t *v_pool,
                                const int32_t *sel, const int32_t *sel_count, int max_sel,
                                float scale, float *out, const Workspace &ws, hipStream_t stream);
hipError_t launch_fill_u32(uint32_t *p, size_t n, uint32_t value, hipStream_t stream);

}  // namespace qasp
