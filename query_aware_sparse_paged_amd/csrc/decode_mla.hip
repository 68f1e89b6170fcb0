// sparse_paged_decode for latent (MLA) heads: 128 query heads over one
// 576-channel latent KV head whose first 512 channels are the value.
#include "common.h"
#include "launch.h"

namespace qasp {

hipError_t launch_decode_mla(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                             const uint16_t *q, const uint16_t *k_pool, const int32_t *sel,
                             const int32_t *sel_count, int max_sel, float scale, float *out,
                             const Workspace &ws, hipStream_t stream) {
  (void)lay; (void)bat; (void)pol; (void)q; (void)k_pool; (void)sel; (void)sel_count;
  (void)max_sel; (void)scale; (void)out; (void)ws; (void)stream;
  return hipErrorNotSupported;
}

}  // namespace qasp
