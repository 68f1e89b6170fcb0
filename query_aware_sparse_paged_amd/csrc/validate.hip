// Opt-in validation of the device-side description of a batch: sequence
// lengths, page-table entries and, for the calls that take one, a selection.
// The page table is the map from a sequence's logical pages to pool pages
// (Vortex explainer, gist.science paper 2606.06453, section 1: the map that
// finds the scattered boxes); a bad entry would send every kernel after it to
// the wrong place, so in validate mode a check kernel that reads only those
// arrays runs first and the call returns QASP_ERR_BAD_PAGE_TABLE before any
// kernel indexes the pools (the per-buffer guard at an interface of the
// llama.cpp draft-head article, aikeizai.jp, "facts from primary sources").
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "common.h"
#include "launch.h"

namespace qasp {

// One result word per check in flight (a check waits for its own word before
// returning, so slots are reused only by calls that overlap more than this).
constexpr int kCheckSlots = 64;
__device__ unsigned int check_result[kCheckSlots];

// One block.  Every read stays inside the arrays' stated shapes: a page-table
// row is read only below pt_stride and only when the length fits; a selection
// row only below max_sel and only when its count fits.
__global__ __launch_bounds__(1024) void check_batch_kernel(const int32_t *__restrict__ page_table,
                                                           const int32_t *__restrict__ seq_lens, int batch,
                                                           int pt_stride, int max_pages, int ps, int num_pool_pages,
                                                           int extra_tokens, const int32_t *__restrict__ sel,
                                                           const int32_t *__restrict__ sel_count, int max_sel,
                                                           int Hkv, unsigned int *__restrict__ result) {
  bool bad = false;
  for (int b = 0; b < batch; b++) {
    const int L = seq_lens[b];
    const long need = (long)L + extra_tokens;  // tokens the call touches
    const bool len_ok = L >= 0 && (long)L <= (long)max_pages * ps && need <= (long)pt_stride * ps;
    bad |= !len_ok;
    const int P = len_ok ? (int)((need + ps - 1) / ps) : 0;
    const int32_t *row = page_table + (size_t)b * pt_stride;
    for (int j = threadIdx.x; j < P; j += blockDim.x) {
      const int p = row[j];
      bad |= p < 0 || p >= num_pool_pages;
    }
    if (sel != nullptr) {
      const int P_len = len_ok ? num_pages_of(L, ps) : 0;  // a selection names pages of the length
      for (int g = 0; g < Hkv; g++) {
        const int c = sel_count[(size_t)b * Hkv + g];
        const bool c_ok = c >= 0 && c <= max_sel;
        bad |= !c_ok;
        const int32_t *srow = sel + ((size_t)b * Hkv + g) * max_sel;
        for (int i = threadIdx.x; i < (c_ok ? c : 0); i += blockDim.x) {
          const int j = srow[i];
          bad |= j < 0 || j >= P_len;
        }
      }
    }
  }
  const int any = __syncthreads_or(bad ? 1 : 0);
  if (threadIdx.x == 0) result[0] = any ? 1u : 0u;
}

bool validate_mode() {
  const char *v = getenv("QASP_VALIDATE");
  return v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0;
}

int32_t check_batch_on_device(const qasp_layout &lay, const qasp_batch &bat, int extra_tokens, const int32_t *sel,
                              const int32_t *sel_count, int max_sel, hipStream_t stream) {
  if (bat.batch == 0) return QASP_OK;
  static std::atomic<unsigned int> next_slot{0};
  unsigned int *res = nullptr;
  if (hipGetSymbolAddress((void **)&res, HIP_SYMBOL(check_result)) != hipSuccess || res == nullptr)
    return QASP_ERR_LAUNCH;
  res += next_slot.fetch_add(1) % kCheckSlots;
  hipLaunchKernelGGL(check_batch_kernel, dim3(1), dim3(1024), 0, stream, bat.page_table, bat.seq_lens, bat.batch,
                     bat.pt_stride, bat.max_pages, lay.page_size, lay.num_pool_pages, extra_tokens, sel, sel_count,
                     max_sel, lay.num_kv_heads, res);
  if (hipGetLastError() != hipSuccess) return QASP_ERR_LAUNCH;
  unsigned int h = 1;
  if (hipMemcpyAsync(&h, res, sizeof h, hipMemcpyDeviceToHost, stream) != hipSuccess) return QASP_ERR_LAUNCH;
  if (hipStreamSynchronize(stream) != hipSuccess) return QASP_ERR_LAUNCH;
  return h == 0 ? QASP_OK : QASP_ERR_BAD_PAGE_TABLE;
}

}  // namespace qasp
