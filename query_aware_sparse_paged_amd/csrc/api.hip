// The C ABI of include/qasp.h: host-side argument checks (before any HIP
// call), workspace layout and launch order.
#include <string.h>

#include <mutex>

#include "common.h"
#include "launch.h"

namespace qasp {

hipError_t launch_decode_gqa(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                             const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                             const int32_t *sel, const int32_t *sel_count, int max_sel, float scale,
                             float *out, const Workspace &ws, hipStream_t stream, int nq = 1,
                             int window_q = 0);
hipError_t launch_decode_mla(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                             const uint16_t *q, const uint16_t *k_pool, const int32_t *sel,
                             const int32_t *sel_count, int max_sel, float scale, float *out,
                             const Workspace &ws, hipStream_t stream, const qasp_score *scores = nullptr,
                             const uint16_t *summ = nullptr);
bool mla_select_fits(const qasp_batch &bat, int max_sel);

constexpr int kMaxPagesLimit = 16384;  // select keeps 8 bytes per page in LDS

enum Family { kFamilyNone, kFamilyGqa, kFamilyMla };

static Family family_of(const qasp_layout &lay) {
  if (lay.page_size == 16 && lay.head_dim_k == 128 && lay.head_dim_v == 128 && !lay.v_from_k)
    return kFamilyGqa;
  if (lay.page_size == 64 && lay.head_dim_k == 576 && lay.head_dim_v == 512 && lay.v_from_k)
    return kFamilyMla;
  return kFamilyNone;
}

static int32_t check_layout(const qasp_layout *lay) {
  if (!lay) return QASP_ERR_NULL_ARG;
  if (lay->num_pool_pages <= 0 || lay->page_size <= 0 || lay->num_kv_heads <= 0 ||
      lay->head_dim_k <= 0 || lay->head_dim_v <= 0)
    return QASP_ERR_BAD_SHAPE;
  if (lay->v_from_k && lay->head_dim_v > lay->head_dim_k) return QASP_ERR_BAD_SHAPE;
  if (lay->num_kv_heads > 64) return QASP_ERR_UNSUPPORTED;
  if (family_of(*lay) == kFamilyNone) return QASP_ERR_UNSUPPORTED;
  if (family_of(*lay) == kFamilyMla && lay->num_kv_heads != 1) return QASP_ERR_UNSUPPORTED;
  return QASP_OK;
}

static int32_t check_batch(const qasp_layout &lay, const qasp_batch *bat) {
  if (!bat) return QASP_ERR_NULL_ARG;
  if (bat->batch < 0 || bat->max_pages < 0 || bat->pt_stride < bat->max_pages || bat->num_q_heads <= 0)
    return QASP_ERR_BAD_SHAPE;
  if (bat->num_q_heads % lay.num_kv_heads != 0) return QASP_ERR_BAD_SHAPE;
  const int G = bat->num_q_heads / lay.num_kv_heads;
  const Family f = family_of(lay);
  if (f == kFamilyGqa && G > 16) return QASP_ERR_UNSUPPORTED;
  if (f == kFamilyMla && G != 128) return QASP_ERR_UNSUPPORTED;
  if (bat->max_pages > kMaxPagesLimit) return QASP_ERR_UNSUPPORTED;
  if (bat->batch > 65535) return QASP_ERR_UNSUPPORTED;
  if (bat->batch > 0 && (!bat->page_table || !bat->seq_lens)) return QASP_ERR_NULL_ARG;
  return QASP_OK;
}

static int32_t check_policy(const qasp_layout &lay, const qasp_policy *pol) {
  if (!pol) return QASP_ERR_NULL_ARG;
  if (pol->n_sink_pages < 0 || pol->n_local_pages < 0 || pol->top_k < 0 || pol->sink_tokens < 0 ||
      pol->window_tokens < 0)
    return QASP_ERR_BAD_SHAPE;
  if (lay.num_kv_heads < 64 && (pol->static_head_mask >> lay.num_kv_heads) != 0) return QASP_ERR_BAD_SHAPE;
  return QASP_OK;
}

static bool all_static(const qasp_layout &lay, const qasp_policy &pol) {
  const uint64_t all = lay.num_kv_heads == 64 ? ~0ull : ((1ull << lay.num_kv_heads) - 1);
  return (pol.static_head_mask & all) == all;
}

static int32_t max_sel_of(const qasp_layout &lay, const qasp_policy &pol, int32_t max_pages) {
  const int64_t ps = lay.page_size;
  const int64_t qa = (int64_t)pol.n_sink_pages + pol.n_local_pages + pol.top_k;
  const int64_t st = ((int64_t)pol.sink_tokens + ps - 1) / ps + ((int64_t)pol.window_tokens + ps - 1) / ps + 1;
  int64_t m = qa > st ? qa : st;
  if (m > max_pages) m = max_pages;
  return (int32_t)m;
}

// Splits per (sequence, KV head) unit: enough blocks to fill the chip, at
// most 64 pages per wave, at least one page per split.
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static int counts[kMaxDevices] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  if (counts[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    counts[dev] = n;
  }
  return counts[dev];
}

int decode_splits(const qasp_layout &lay, const qasp_batch &bat, int max_sel) {
  if (family_of(lay) == kFamilyMla) {
    const int s = (max_sel + kMlaPagesPerSplit - 1) / kMlaPagesPerSplit;
    return s < 1 ? 1 : s;
  }
  const long units = (long)bat.batch * lay.num_kv_heads;
  long s = units > 0 ? (kGqaTargetBlocks + units - 1) / units : 1;
  const long min_s = (max_sel + 64L * kGqaDecodeWaves - 1) / (64L * kGqaDecodeWaves);
  if (s < min_s) s = min_s;
  if (s > max_sel) s = max_sel;
  return s < 1 ? 1 : (int)s;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t workspace_bytes(const qasp_layout &lay, const qasp_batch &bat, int max_sel) {
  const size_t units = (size_t)bat.batch * lay.num_kv_heads;
  const size_t splits = (size_t)decode_splits(lay, bat, max_sel);
  size_t n = 0;
  n += align256(units * (size_t)bat.max_pages * sizeof(qasp_score));
  n += align256(units * (size_t)max_sel * sizeof(int32_t));
  n += align256(units * sizeof(int32_t));
  n += align256((size_t)bat.batch * bat.num_q_heads * splits * lay.head_dim_v * sizeof(float));
  n += align256((size_t)bat.batch * bat.num_q_heads * splits * sizeof(float2));
  return n;
}

Workspace carve_workspace(const qasp_layout &lay, const qasp_batch &bat, int max_sel, void *base) {
  Workspace w;
  const size_t units = (size_t)bat.batch * lay.num_kv_heads;
  w.splits = decode_splits(lay, bat, max_sel);
  char *p = (char *)base;
  w.scores = (qasp_score *)p;
  p += align256(units * (size_t)bat.max_pages * sizeof(qasp_score));
  w.sel = (int32_t *)p;
  p += align256(units * (size_t)max_sel * sizeof(int32_t));
  w.sel_count = (int32_t *)p;
  p += align256(units * sizeof(int32_t));
  w.partial = (float *)p;
  p += align256((size_t)bat.batch * bat.num_q_heads * w.splits * lay.head_dim_v * sizeof(float));
  w.partial_ml = (float2 *)p;
  return w;
}

hipError_t launch_sparse_decode(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                                const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                const int32_t *sel, const int32_t *sel_count, int max_sel, float scale,
                                float *out, const Workspace &ws, hipStream_t stream) {
  if (bat.batch == 0) return hipSuccess;
  if (family_of(lay) == kFamilyGqa)
    return launch_decode_gqa(lay, bat, pol, q, k_pool, v_pool, sel, sel_count, max_sel, scale, out, ws,
                             stream);
  return launch_decode_mla(lay, bat, pol, q, k_pool, sel, sel_count, max_sel, scale, out, ws, stream);
}

static int32_t status_of(hipError_t e) { return e == hipSuccess ? QASP_OK : QASP_ERR_LAUNCH; }

// Validate mode (QASP_VALIDATE set and not "0"): the device-side lengths,
// page-table entries and selection are checked before any kernel that reads
// the pools through them; the check synchronises the stream.
static int32_t maybe_validate(const qasp_layout &lay, const qasp_batch &bat, void *stream, int extra_tokens = 0,
                              const int32_t *sel = nullptr, const int32_t *sel_count = nullptr, int max_sel = 0) {
  if (!validate_mode()) return QASP_OK;
  return check_batch_on_device(lay, bat, extra_tokens, sel, sel_count, max_sel, (hipStream_t)stream);
}

// Whether a step runs as one kernel per (sequence, KV head) unit: grouped-query
// layouts whose page list fits the kernel's LDS arrays, with either enough
// units to give every CU a block or so little work per unit (summaries of
// every page plus the K/V tiles of a full selection) that one CU per unit
// beats a chain of kernels, each with its own launch and drain (bat: the
// batch as the kernel sees it, i.e. the multi-query step's widened group).
static bool one_kernel_step(const qasp_layout &lay, const qasp_batch &bat, int max_sel) {
  const long units = (long)bat.batch * lay.num_kv_heads;
  const size_t unit_bytes = (size_t)bat.max_pages * 2 * lay.head_dim_k * 2 +
                            (size_t)max_sel * lay.page_size * (lay.head_dim_k + lay.head_dim_v) * 2;
  return family_of(lay) == kFamilyGqa && (units >= kFusedMinUnits || unit_bytes <= kFusedSmallUnitBytes) &&
         bat.max_pages <= kFusedMaxPages && fused_lds_bytes(lay, bat, max_sel) <= 160 * 1024;
}

// Multi-query step: nq draft queries regrouped so that KV head g's group holds
// G heads per draft query (num_q_heads * nq columns in all); a static head's
// selection covers the union of the queries' windows (window + nq - 1 tokens
// ending at L, when the window is not empty).
constexpr int kMaxDrafts = 16;
static qasp_batch multi_batch(const qasp_batch &bat, int nq) {
  qasp_batch b = bat;
  b.num_q_heads = bat.num_q_heads * nq;
  return b;
}
static qasp_policy multi_policy(const qasp_policy &pol, int nq) {
  qasp_policy p = pol;
  if (p.window_tokens > 0) p.window_tokens += nq - 1;
  return p;
}
static int32_t check_multi(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol, int32_t nq) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_batch(*lay, bat)) != QASP_OK) return rc;
  if ((rc = check_policy(*lay, pol)) != QASP_OK) return rc;
  if (nq < 1) return QASP_ERR_BAD_SHAPE;
  if (nq > kMaxDrafts || nq > lay->page_size || family_of(*lay) != kFamilyGqa) return QASP_ERR_UNSUPPORTED;
  if ((long)(bat->num_q_heads / lay->num_kv_heads) * nq > 16) return QASP_ERR_UNSUPPORTED;
  if (pol->window_tokens > INT32_MAX - kMaxDrafts) return QASP_ERR_BAD_SHAPE;
  return QASP_OK;
}
static size_t multi_workspace_bytes(const qasp_layout &lay, const qasp_batch &bat, int nq, int max_sel) {
  const size_t rows = (size_t)bat.batch * nq * bat.num_q_heads;
  return workspace_bytes(lay, multi_batch(bat, nq), max_sel) + align256(rows * lay.head_dim_k * sizeof(uint16_t));
}

}  // namespace qasp

using namespace qasp;

extern "C" {

const char *qasp_version(void) { return "0.1.0"; }

const char *qasp_status_string(int32_t status) {
  switch (status) {
    case QASP_OK: return "ok";
    case QASP_ERR_NULL_ARG: return "a required pointer is NULL";
    case QASP_ERR_BAD_SHAPE: return "invalid or inconsistent sizes";
    case QASP_ERR_UNSUPPORTED: return "shape not supported by the kernels";
    case QASP_ERR_WORKSPACE: return "workspace too small";
    case QASP_ERR_MAX_SEL: return "max_sel smaller than the largest possible selection";
    case QASP_ERR_LAUNCH: return "HIP kernel launch failed";
    case QASP_ERR_ALLOC: return "host-tier allocation failed";
    case QASP_ERR_BAD_PAGE_TABLE: return "a sequence length, page-table entry or selected page is out of range";
    case QASP_ERR_SCRATCH: return "the call needs more workspace than the library's static scratch buffer holds";
    default: return "unknown status";
  }
}

int32_t qasp_max_sel(const qasp_layout *lay, const qasp_policy *pol, int32_t max_pages) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_policy(*lay, pol)) != QASP_OK) return rc;
  if (max_pages < 0) return QASP_ERR_BAD_SHAPE;
  return max_sel_of(*lay, *pol, max_pages);
}

size_t qasp_workspace_bytes(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol,
                            int32_t max_sel) {
  if (check_layout(lay) != QASP_OK || check_batch(*lay, bat) != QASP_OK || check_policy(*lay, pol) != QASP_OK)
    return 0;
  if (max_sel < 0) return 0;
  return workspace_bytes(*lay, *bat, max_sel);
}

int32_t qasp_build_summaries(const qasp_layout *lay, const qasp_batch *bat, const uint16_t *k_pool,
                             uint16_t *summ, void *stream) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_batch(*lay, bat)) != QASP_OK) return rc;
  if (bat->batch == 0) return QASP_OK;
  if (!k_pool || !summ) return QASP_ERR_NULL_ARG;
  if ((rc = maybe_validate(*lay, *bat, stream)) != QASP_OK) return rc;
  return status_of(launch_build_summaries(*lay, *bat, k_pool, summ, (hipStream_t)stream));
}

int32_t qasp_append_kv(const qasp_layout *lay, const qasp_batch *bat_before, const qasp_policy *pol,
                       const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool, uint16_t *v_pool,
                       uint16_t *summ, void *stream) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_batch(*lay, bat_before)) != QASP_OK) return rc;
  if ((rc = check_policy(*lay, pol)) != QASP_OK) return rc;
  if (bat_before->batch == 0) return QASP_OK;
  if (!k_new || !k_pool) return QASP_ERR_NULL_ARG;
  if (!lay->v_from_k && (!v_new || !v_pool)) return QASP_ERR_NULL_ARG;
  if (!summ && !all_static(*lay, *pol)) return QASP_ERR_NULL_ARG;
  if ((rc = maybe_validate(*lay, *bat_before, stream, 1)) != QASP_OK) return rc;
  return status_of(launch_append_kv(*lay, *bat_before, 0, k_new, v_new, k_pool, v_pool, summ,
                                    (hipStream_t)stream));
}

int32_t qasp_score_pages(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol,
                         const uint16_t *q, const uint16_t *summ, qasp_score *scores, void *stream) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_batch(*lay, bat)) != QASP_OK) return rc;
  if ((rc = check_policy(*lay, pol)) != QASP_OK) return rc;
  if (bat->batch == 0 || bat->max_pages == 0) return QASP_OK;
  if (!scores) return QASP_ERR_NULL_ARG;
  if (!all_static(*lay, *pol) && (!q || !summ)) return QASP_ERR_NULL_ARG;
  if ((rc = maybe_validate(*lay, *bat, stream)) != QASP_OK) return rc;
  return status_of(launch_score_pages(*lay, *bat, *pol, q, summ, scores, (hipStream_t)stream,
                                      token_append(*lay, nullptr, nullptr, nullptr, nullptr, nullptr)));
}

int32_t qasp_select_topk(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol,
                         const uint16_t *q, const uint16_t *summ, const qasp_score *scores, int32_t *sel,
                         int32_t *sel_count, int32_t max_sel, void *stream) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_batch(*lay, bat)) != QASP_OK) return rc;
  if ((rc = check_policy(*lay, pol)) != QASP_OK) return rc;
  if (max_sel < 0) return QASP_ERR_BAD_SHAPE;
  if (max_sel < max_sel_of(*lay, *pol, bat->max_pages)) return QASP_ERR_MAX_SEL;
  if (bat->batch == 0) return QASP_OK;
  if (!sel || !sel_count) return QASP_ERR_NULL_ARG;
  if (!all_static(*lay, *pol) && (!q || !summ || !scores)) return QASP_ERR_NULL_ARG;
  if ((rc = maybe_validate(*lay, *bat, stream)) != QASP_OK) return rc;
  return status_of(launch_select_topk(*lay, *bat, *pol, q, summ, scores, sel, sel_count, max_sel,
                                      (hipStream_t)stream));
}

int32_t qasp_sparse_paged_decode(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol,
                                 const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                 const int32_t *sel, const int32_t *sel_count, int32_t max_sel, float scale,
                                 float *out, void *workspace, size_t workspace_bytes_given, void *stream) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_batch(*lay, bat)) != QASP_OK) return rc;
  if ((rc = check_policy(*lay, pol)) != QASP_OK) return rc;
  if (max_sel < 0) return QASP_ERR_BAD_SHAPE;
  if (bat->batch == 0) return QASP_OK;
  if (!q || !k_pool || !sel || !sel_count || !out || !workspace) return QASP_ERR_NULL_ARG;
  if (!lay->v_from_k && !v_pool) return QASP_ERR_NULL_ARG;
  if (workspace_bytes_given < workspace_bytes(*lay, *bat, max_sel)) return QASP_ERR_WORKSPACE;
  if ((rc = maybe_validate(*lay, *bat, stream, 0, sel, sel_count, max_sel)) != QASP_OK) return rc;
  const Workspace ws = carve_workspace(*lay, *bat, max_sel, workspace);
  return status_of(launch_sparse_decode(*lay, *bat, *pol, q, k_pool, v_pool, sel, sel_count, max_sel, scale,
                                        out, ws, (hipStream_t)stream));
}

}  // extern "C"

namespace qasp {

// Checks of qasp_decode_step's arguments other than the workspace (shared
// with its no-allocation form).
static int32_t check_step_args(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol,
                               const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                               const uint16_t *k_pool, const uint16_t *v_pool, const uint16_t *summ, const float *out,
                               const int32_t *sel, const int32_t *sel_count, int32_t max_sel) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_batch(*lay, bat)) != QASP_OK) return rc;
  if ((rc = check_policy(*lay, pol)) != QASP_OK) return rc;
  if (max_sel < 0) return QASP_ERR_BAD_SHAPE;
  if (max_sel < max_sel_of(*lay, *pol, bat->max_pages)) return QASP_ERR_MAX_SEL;
  if (bat->batch == 0) return QASP_OK;
  if (!q || !k_pool || !out) return QASP_ERR_NULL_ARG;
  if (!lay->v_from_k && !v_pool) return QASP_ERR_NULL_ARG;
  if (!all_static(*lay, *pol) && !summ) return QASP_ERR_NULL_ARG;
  if (k_new && !lay->v_from_k && !v_new) return QASP_ERR_NULL_ARG;
  if ((sel == nullptr) != (sel_count == nullptr)) return QASP_ERR_NULL_ARG;
  return QASP_OK;
}

// The step's launches once every argument has been checked; workspace holds
// workspace_bytes(lay, bat, max_sel) bytes.
static int32_t run_step(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol, const uint16_t *q,
                        const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool, uint16_t *v_pool,
                        uint16_t *summ, float scale, float *out, int32_t *sel, int32_t *sel_count, int32_t max_sel,
                        void *workspace, hipStream_t s) {
  const bool scored = !all_static(lay, pol);
  // many units: the whole step as one kernel per (sequence, KV head) block
  if (one_kernel_step(lay, bat, max_sel))
    return status_of(launch_fused_step_gqa(lay, bat, pol, q, k_new, v_new, k_pool, v_pool, summ, scale, out, sel,
                                           sel_count, max_sel, s));
  const Workspace ws = carve_workspace(lay, bat, max_sel, workspace);
  int32_t *sel_out = sel ? sel : ws.sel;
  int32_t *cnt_out = sel_count ? sel_count : ws.sel_count;
  hipError_t e = hipSuccess;
  // the scoring kernel appends the token when its page is no candidate (a local
  // page); otherwise the append runs first, so the page is scored with it
  const bool fold_append = k_new && scored && pol.n_local_pages >= 1;
  if (k_new && !fold_append) e = launch_append_kv(lay, bat, -1, k_new, v_new, k_pool, v_pool, summ, s);
  if (e == hipSuccess && scored)
    e = launch_score_pages(lay, bat, pol, q, summ, ws.scores, s,
                           token_append(lay, fold_append ? k_new : nullptr, v_new, k_pool, v_pool, summ));
  // selection and attention in one launch when its LDS fits
  if (e == hipSuccess && family_of(lay) == kFamilyGqa && select_decode_lds_bytes(lay, bat, max_sel) <= 160 * 1024)
    return status_of(launch_select_decode_gqa(lay, bat, pol, q, k_pool, v_pool, summ, ws.scores, sel_out, cnt_out,
                                              max_sel, scale, out, ws, s));
  if (e == hipSuccess && family_of(lay) == kFamilyMla && mla_select_fits(bat, max_sel))
    return status_of(launch_decode_mla(lay, bat, pol, q, k_pool, sel_out, cnt_out, max_sel, scale, out, ws, s,
                                       ws.scores, summ));
  if (e == hipSuccess) e = launch_select_topk(lay, bat, pol, q, summ, ws.scores, sel_out, cnt_out, max_sel, s);
  if (e == hipSuccess)
    e = launch_sparse_decode(lay, bat, pol, q, k_pool, v_pool, sel_out, cnt_out, max_sel, scale, out, ws, s);
  return status_of(e);
}

// The no-allocation form's workspace: one static array per device (each GPU
// the library runs on holds its own copy until the process ends).  Host code
// never uses the array's name as an address: the device address of each
// GPU's copy is looked up once, with that device current, and kept.
constexpr size_t kScratchBytes = (size_t)QASP_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static void *scratch_on_current_device() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *ptrs[kMaxDevices] = {nullptr};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace qasp

extern "C" {

int32_t qasp_decode_step(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol,
                         const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                         uint16_t *v_pool, uint16_t *summ, float scale, float *out, int32_t *sel,
                         int32_t *sel_count, int32_t max_sel, void *workspace, size_t workspace_bytes_given,
                         void *stream) {
  int32_t rc = check_step_args(lay, bat, pol, q, k_new, v_new, k_pool, v_pool, summ, out, sel, sel_count, max_sel);
  if (rc != QASP_OK || bat->batch == 0) return rc;
  if (!workspace) return QASP_ERR_NULL_ARG;
  if (workspace_bytes_given < workspace_bytes(*lay, *bat, max_sel)) return QASP_ERR_WORKSPACE;
  if ((rc = maybe_validate(*lay, *bat, stream)) != QASP_OK) return rc;
  return run_step(*lay, *bat, *pol, q, k_new, v_new, k_pool, v_pool, summ, scale, out, sel, sel_count, max_sel,
                  workspace, (hipStream_t)stream);
}

size_t qasp_scratch_bytes(void) { return kScratchBytes; }

int32_t qasp_decode_step_path(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol,
                              int32_t max_sel) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_batch(*lay, bat)) != QASP_OK) return rc;
  if ((rc = check_policy(*lay, pol)) != QASP_OK) return rc;
  if (max_sel < 0) return QASP_ERR_BAD_SHAPE;
  return one_kernel_step(*lay, *bat, max_sel) ? QASP_PATH_ONE_KERNEL : QASP_PATH_CHAIN;
}

int32_t qasp_decode_step_noalloc(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol,
                                 const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                                 uint16_t *v_pool, uint16_t *summ, float scale, float *out, int32_t *sel,
                                 int32_t *sel_count, int32_t max_sel, void *stream) {
  int32_t rc = check_step_args(lay, bat, pol, q, k_new, v_new, k_pool, v_pool, summ, out, sel, sel_count, max_sel);
  if (rc != QASP_OK || bat->batch == 0) return rc;
  if (workspace_bytes(*lay, *bat, max_sel) > kScratchBytes) return QASP_ERR_SCRATCH;
  void *ws = scratch_on_current_device();
  if (ws == nullptr) return QASP_ERR_LAUNCH;
  if ((rc = maybe_validate(*lay, *bat, stream)) != QASP_OK) return rc;
  return run_step(*lay, *bat, *pol, q, k_new, v_new, k_pool, v_pool, summ, scale, out, sel, sel_count, max_sel, ws,
                  (hipStream_t)stream);
}

int32_t qasp_check_batch(const qasp_layout *lay, const qasp_batch *bat, int32_t extra_tokens, const int32_t *sel,
                         const int32_t *sel_count, int32_t max_sel, void *stream) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_batch(*lay, bat)) != QASP_OK) return rc;
  if (extra_tokens < 0 || extra_tokens > kMaxDrafts || max_sel < 0) return QASP_ERR_BAD_SHAPE;
  if ((sel == nullptr) != (sel_count == nullptr)) return QASP_ERR_NULL_ARG;
  return check_batch_on_device(*lay, *bat, extra_tokens, sel, sel_count, max_sel, (hipStream_t)stream);
}

int32_t qasp_host_alloc(size_t bytes, void **host_ptr, void **device_ptr) {
  if (!host_ptr || !device_ptr) return QASP_ERR_NULL_ARG;
  *host_ptr = nullptr;
  *device_ptr = nullptr;
  if (bytes == 0) return QASP_ERR_BAD_SHAPE;
  void *h = nullptr, *d = nullptr;
  if (hipHostMalloc(&h, bytes, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess || !h)
    return QASP_ERR_ALLOC;
  if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess || !d) {
    (void)hipHostFree(h);
    return QASP_ERR_ALLOC;
  }
  *host_ptr = h;
  *device_ptr = d;
  return QASP_OK;
}

int32_t qasp_host_free(void *host_ptr) {
  if (!host_ptr) return QASP_ERR_NULL_ARG;
  return hipHostFree(host_ptr) == hipSuccess ? QASP_OK : QASP_ERR_ALLOC;
}

size_t qasp_quant_pool_bytes(const qasp_layout *lay) {
  if (check_layout(lay) != QASP_OK || family_of(*lay) != kFamilyGqa) return 0;
  return (size_t)lay->num_pool_pages * lay->num_kv_heads * kQuantPageHeadBytes;
}

int32_t qasp_quantize_pages(const qasp_layout *lay, const qasp_batch *bat, int32_t residual_pages,
                            const uint16_t *k_pool, const uint16_t *v_pool, uint8_t *qpool, void *stream) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_batch(*lay, bat)) != QASP_OK) return rc;
  if (family_of(*lay) != kFamilyGqa) return QASP_ERR_UNSUPPORTED;
  if (residual_pages < 1) return QASP_ERR_BAD_SHAPE;
  if (bat->batch == 0) return QASP_OK;
  if (!k_pool || !v_pool || !qpool) return QASP_ERR_NULL_ARG;
  if ((rc = maybe_validate(*lay, *bat, stream)) != QASP_OK) return rc;
  return status_of(launch_quantize(*lay, *bat, residual_pages, false, k_pool, v_pool, qpool, (hipStream_t)stream));
}

int32_t qasp_decode_step_quant(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol,
                               int32_t residual_pages, const uint16_t *q, const uint16_t *k_new,
                               const uint16_t *v_new, uint16_t *k_pool, uint16_t *v_pool, uint16_t *summ,
                               uint8_t *qpool, float scale, float *out, int32_t *sel, int32_t *sel_count,
                               int32_t max_sel, void *workspace, size_t workspace_bytes_given, void *stream) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_batch(*lay, bat)) != QASP_OK) return rc;
  if ((rc = check_policy(*lay, pol)) != QASP_OK) return rc;
  if (family_of(*lay) != kFamilyGqa) return QASP_ERR_UNSUPPORTED;
  if (residual_pages < 1 || max_sel < 0) return QASP_ERR_BAD_SHAPE;
  if (max_sel < max_sel_of(*lay, *pol, bat->max_pages)) return QASP_ERR_MAX_SEL;
  if (bat->batch == 0) return QASP_OK;
  if (!q || !k_pool || !v_pool || !qpool || !out || !workspace) return QASP_ERR_NULL_ARG;
  const bool scored = !all_static(*lay, *pol);
  if (scored && !summ) return QASP_ERR_NULL_ARG;
  if (k_new && !v_new) return QASP_ERR_NULL_ARG;
  if ((sel == nullptr) != (sel_count == nullptr)) return QASP_ERR_NULL_ARG;
  if (workspace_bytes_given < workspace_bytes(*lay, *bat, max_sel)) return QASP_ERR_WORKSPACE;
  if ((rc = maybe_validate(*lay, *bat, stream)) != QASP_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  const Workspace ws = carve_workspace(*lay, *bat, max_sel, workspace);
  int32_t *sel_out = sel ? sel : ws.sel;
  int32_t *cnt_out = sel_count ? sel_count : ws.sel_count;
  hipError_t e = hipSuccess;
  if (one_kernel_step(*lay, *bat, max_sel)) {
    // the whole step in one kernel (at most 64 selected pages per wave of it)
    if (max_sel <= 64 * kFusedWaves)
      return status_of(launch_fused_step_gqa(*lay, *bat, *pol, q, k_new, v_new, k_pool, v_pool, summ, scale, out,
                                             sel, sel_count, max_sel, s, 1, 0, false, nullptr, nullptr, qpool,
                                             residual_pages));
    // else: append, score and select in the one-kernel step's selection-only form
    e = launch_fused_step_gqa(*lay, *bat, *pol, q, k_new, v_new, k_pool, v_pool, summ, scale, out, sel_out, cnt_out,
                              max_sel, s, 1, 0, true);
    if (e == hipSuccess)  // (quantises the page leaving the residual region too)
      e = launch_decode_quant_gqa(*lay, *bat, *pol, residual_pages, q, k_pool, v_pool, qpool, sel_out, cnt_out,
                                  max_sel, scale, out, ws, s);
    return status_of(e);
  }
  // as in the bf16 chain: the scoring kernel appends the token when its page
  // is no candidate, and the selection runs inside the attention launch when
  // its LDS fits (a token that opened a new page pushed page P - 1 - R out of
  // the residual region: the attention launch quantises it first)
  // (the scoring kernel, when there is one, also quantises the page-head that
  // leaves the residual region)
  const bool fold_append = k_new && scored && pol->n_local_pages >= 1;
  if (k_new && !fold_append) e = launch_append_kv(*lay, *bat, -1, k_new, v_new, k_pool, v_pool, summ, s);
  if (e == hipSuccess && scored)
    e = launch_score_pages(*lay, *bat, *pol, q, summ, ws.scores, s,
                           token_append(*lay, fold_append ? k_new : nullptr, v_new, k_pool, v_pool, summ), qpool,
                           residual_pages, k_pool, v_pool);
  if (e == hipSuccess && select_quant_lds_bytes(*lay, *bat, max_sel) <= 160 * 1024)
    return status_of(launch_decode_quant_gqa(*lay, *bat, *pol, residual_pages, q, k_pool, v_pool, qpool, sel_out,
                                             cnt_out, max_sel, scale, out, ws, s, ws.scores, summ, scored));
  if (e == hipSuccess)
    e = launch_select_topk(*lay, *bat, *pol, q, summ, ws.scores, sel_out, cnt_out, max_sel, s);
  if (e == hipSuccess)
    e = launch_decode_quant_gqa(*lay, *bat, *pol, residual_pages, q, k_pool, v_pool, qpool, sel_out, cnt_out,
                                max_sel, scale, out, ws, s, nullptr, nullptr, scored);
  return status_of(e);
}

int32_t qasp_max_sel_multi(const qasp_layout *lay, const qasp_policy *pol, int32_t n_query, int32_t max_pages) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_policy(*lay, pol)) != QASP_OK) return rc;
  if (max_pages < 0 || n_query < 1 || pol->window_tokens > INT32_MAX - kMaxDrafts) return QASP_ERR_BAD_SHAPE;
  if (n_query > kMaxDrafts) return QASP_ERR_UNSUPPORTED;
  return max_sel_of(*lay, multi_policy(*pol, n_query), max_pages);
}

size_t qasp_workspace_bytes_multi(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol,
                                  int32_t n_query, int32_t max_sel) {
  if (check_multi(lay, bat, pol, n_query) != QASP_OK || max_sel < 0) return 0;
  return multi_workspace_bytes(*lay, *bat, n_query, max_sel);
}

int32_t qasp_decode_step_multi(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol,
                               int32_t n_query, const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                               uint16_t *k_pool, uint16_t *v_pool, uint16_t *summ, float scale, float *out,
                               int32_t *sel, int32_t *sel_count, int32_t max_sel, void *workspace,
                               size_t workspace_bytes_given, void *stream) {
  int32_t rc = check_multi(lay, bat, pol, n_query);
  if (rc != QASP_OK) return rc;
  const int nq = n_query;
  const qasp_policy wpol = multi_policy(*pol, nq);
  if (max_sel < 0) return QASP_ERR_BAD_SHAPE;
  if (max_sel < max_sel_of(*lay, wpol, bat->max_pages)) return QASP_ERR_MAX_SEL;
  if (bat->batch == 0) return QASP_OK;
  if (!q || !k_pool || !v_pool || !out || !workspace) return QASP_ERR_NULL_ARG;
  const bool scored = !all_static(*lay, *pol);
  if (scored && !summ) return QASP_ERR_NULL_ARG;
  if (k_new && !v_new) return QASP_ERR_NULL_ARG;
  if ((sel == nullptr) != (sel_count == nullptr)) return QASP_ERR_NULL_ARG;
  if (workspace_bytes_given < multi_workspace_bytes(*lay, *bat, nq, max_sel)) return QASP_ERR_WORKSPACE;
  if ((rc = maybe_validate(*lay, *bat, stream)) != QASP_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  const qasp_batch wbat = multi_batch(*bat, nq);
  const Workspace ws = carve_workspace(*lay, wbat, max_sel, workspace);
  uint16_t *q_grouped = (uint16_t *)((char *)workspace + workspace_bytes(*lay, wbat, max_sel));
  int32_t *sel_out = sel ? sel : ws.sel;
  int32_t *cnt_out = sel_count ? sel_count : ws.sel_count;
  // many units: one kernel per (sequence, KV head) appends the drafts, stages
  // the query rows in the grouped order, scores, selects and attends
  if (one_kernel_step(*lay, wbat, max_sel)) {
    if (nq == 1)  // one draft: the one-token step, its token appended at L - 1
      return status_of(launch_fused_step_gqa(*lay, wbat, wpol, q, k_new, v_new, k_pool, v_pool, summ, scale, out, sel,
                                             sel_count, max_sel, s));
    return status_of(launch_fused_step_gqa(*lay, wbat, wpol, q, nullptr, nullptr, k_pool, v_pool, summ, scale, out,
                                           sel, sel_count, max_sel, s, nq, pol->window_tokens, false, k_new, v_new));
  }
  // q [B][nq][Hkv][G][Dk] -> [B][Hkv][nq][G][Dk], and the drafts appended
  hipError_t e = launch_prepare_drafts(*lay, *bat, nq, q, q_grouped, k_new, v_new, k_pool, v_pool, summ, s);
  if (e == hipSuccess && scored)
    e = launch_score_pages(*lay, wbat, wpol, q_grouped, summ, ws.scores, s,
                           token_append(*lay, nullptr, nullptr, nullptr, nullptr, nullptr));
  if (e == hipSuccess)
    e = launch_select_topk(*lay, wbat, wpol, q_grouped, summ, ws.scores, sel_out, cnt_out, max_sel, s);
  if (e == hipSuccess)  // writes out in the caller's [B][nq][Hq][Dv] order
    e = launch_decode_gqa(*lay, wbat, wpol, q_grouped, k_pool, v_pool, sel_out, cnt_out, max_sel, scale, out, ws, s,
                          nq, pol->window_tokens);
  return status_of(e);
}

int32_t qasp_decode_step_reuse(const qasp_layout *lay, const qasp_batch *bat, const qasp_policy *pol,
                               const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                               uint16_t *v_pool, uint16_t *summ, float scale, const int32_t *sel,
                               const int32_t *sel_count, int32_t max_sel, float *out, void *workspace,
                               size_t workspace_bytes_given, void *stream) {
  int32_t rc = check_layout(lay);
  if (rc != QASP_OK) return rc;
  if ((rc = check_batch(*lay, bat)) != QASP_OK) return rc;
  if ((rc = check_policy(*lay, pol)) != QASP_OK) return rc;
  if (max_sel < 0) return QASP_ERR_BAD_SHAPE;
  if (bat->batch == 0) return QASP_OK;
  if (!q || !k_pool || !sel || !sel_count || !out || !workspace) return QASP_ERR_NULL_ARG;
  if (!lay->v_from_k && !v_pool) return QASP_ERR_NULL_ARG;
  if (k_new && !lay->v_from_k && !v_new) return QASP_ERR_NULL_ARG;
  if (workspace_bytes_given < workspace_bytes(*lay, *bat, max_sel)) return QASP_ERR_WORKSPACE;
  if ((rc = maybe_validate(*lay, *bat, stream, 0, sel, sel_count, max_sel)) != QASP_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  const long units = (long)bat->batch * lay->num_kv_heads;
  if (family_of(*lay) == kFamilyGqa && units >= kFusedMinUnits)
    return status_of(launch_fused_reuse_gqa(*lay, *bat, *pol, q, k_new, v_new, k_pool, v_pool, summ, scale, out, sel,
                                            sel_count, max_sel, s));
  const Workspace ws = carve_workspace(*lay, *bat, max_sel, workspace);
  hipError_t e = hipSuccess;
  if (k_new) e = launch_append_kv(*lay, *bat, -1, k_new, v_new, k_pool, v_pool, summ, s);
  if (e == hipSuccess)
    e = launch_sparse_decode(*lay, *bat, *pol, q, k_pool, v_pool, sel, sel_count, max_sel, scale, out, ws, s);
  return status_of(e);
}

}  // extern "C"
