// sparse_paged_decode for grouped-query heads (page 16, head_dim 128).
//
// Softmax attention of each query head over the tokens of its group's
// selected pages only, computed exactly on those positions (SubQ/SSA article,
// news.neo-ai.one/ja/article/2719, section "How SSA works"), reached through
// the page table (Vortex explainer, gist.science paper 2606.06453, section 1).
// The per-wave page loop is in attend_core.h.
//
// Work split: block (split, g, b) takes selected pages
// [pps*split, pps*split + pps) of unit (b, g); its WAVES waves take every
// WAVES-th page and merge through LDS.  With one split per unit the block
// writes the output; otherwise it writes a partial (m, l, acc) and
// merge_splits_kernel combines the partials (a kernel boundary orders the
// two; no device-wide fences inside a kernel).
//
// Multi-query form (CAUSAL): the group's head columns are nq draft queries
// x G/nq heads (query i's heads are columns i*G/nq ...); query i sits at
// position L - nq + i and scores only the tokens up to it and, for a static
// head, its own window of window_q tokens (the selection holds the union).
#include "attend_core.h"
#include "launch.h"
#include "select_core.h"

namespace qasp {

template <int PS, int D, int DV, int WAVES, bool CAUSAL>
__global__ __launch_bounds__(WAVES * 64) void decode_gqa_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_pool,
    const uint16_t *__restrict__ v_pool, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ sel_count, float *__restrict__ partial,
    float2 *__restrict__ partial_ml, float *__restrict__ out, int pt_stride, int max_sel, int Hq,
    int Hkv, int G, int splits, int pps, float scale_log2, int sink_tokens, int window_tokens,
    uint64_t static_mask, int nq, int window_q) {
  extern __shared__ float lds[];
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int unit = b * Hkv + g;
  const int L = seq_lens[b];
  const bool is_static = head_is_static(static_mask, g);
  const int sink_end = is_static ? min(sink_tokens, L) : 0;
  const int win_begin = is_static ? max(0, L - window_tokens) : 0;
  const int count = sel_count[unit];
  const int first = split * pps, last = min(first + pps, count);
  const int npg = max(0, (last - first - wave + WAVES - 1) / WAVES);

  // lane i holds the logical id and physical page of this wave's i-th page
  int my_j = 0, my_phys = 0;
  if (lane < npg) {
    my_j = sel[(size_t)unit * max_sel + first + wave + WAVES * lane];
    my_phys = page_table[(size_t)b * pt_stride + my_j];
  }
  const size_t head0 = (size_t)b * Hq + (size_t)g * G;
  uint4 bq[D / 32];
  attend::load_q_columns<D>(bq, q + head0 * D, G, lane);
  attend::WaveState st;
  attend::init_state(st);
  int Lq = L, winq = 0;
  if constexpr (CAUSAL) {
    const int n = lane & 15, per_query = G / nq;
    const int i = n < G ? n / per_query : nq - 1;
    Lq = L - (nq - 1 - i);
    winq = max(0, Lq - window_q);
  }
  const attend::PageWork<PS, D, DV, CAUSAL> pw{k_pool, v_pool, bq, Hkv, g, L, sink_end, win_begin,
                                               is_static, scale_log2, Lq, winq};
  attend::attend_pages<PS, D, DV>(st, pw, npg, my_j, my_phys, lane);
  attend::merge_waves<WAVES, DV>(lds, st, G, [&](int h, int dv, float a, float lsum, float M) {
    if (splits == 1) {
      size_t row = head0 + h;
      if constexpr (CAUSAL) {  // the caller's [B][nq][Hq / nq] order
        const int per_query = G / nq;
        row = ((size_t)b * nq + h / per_query) * (Hq / nq) + (size_t)g * per_query + h % per_query;
      }
      out[row * DV + dv] = lsum > 0.f ? a / lsum : 0.f;
    } else {
      const size_t ps_idx = (head0 + h) * splits + split;
      partial[ps_idx * DV + dv] = a;
      if (dv == 0) partial_ml[ps_idx] = make_float2(M, lsum);
    }
  });
}

// LDS of select_decode_gqa_kernel (bytes): the selection's keys (8 bytes per
// page), which the wave merge reuses at the end, two bit maps, the list.
struct SelectDecodeLds {
  size_t bits, list, total;
  __host__ __device__ SelectDecodeLds(int max_pages, int max_sel, int W, int G) {
    const size_t keys = (size_t)max_pages * 8, merge = (size_t)attend::merge_lds_floats(W, G, 128) * 4;
    bits = ((keys > merge ? keys : merge) + 15) & ~(size_t)15;
    list = bits + 2 * (size_t)((max_pages + 31) / 32) * 4;
    total = list + (size_t)max_sel * 4;
  }
};

// The selection and the attention of the kernel chain in one launch (one
// kernel boundary fewer): block (unit, split) selects its unit's pages from
// the stored scores exactly as select_topk_kernel does (every split of a
// unit computes the same list; the first split also writes it out), then
// attends its split of the list as decode_gqa_kernel does.  The splits of a
// unit are consecutive items of the XCD-contiguous order, so their score
// reads come through one L2.
template <int W>
__global__ __launch_bounds__(W * 64) void select_decode_gqa_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_pool, const uint16_t *__restrict__ v_pool,
    const uint16_t *__restrict__ summ, const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    const qasp_score *__restrict__ scores, int32_t *__restrict__ sel_out, int32_t *__restrict__ sel_count_out,
    float *__restrict__ partial, float2 *__restrict__ partial_ml, float *__restrict__ out, int pt_stride,
    int max_pages, int max_sel, int Hq, int Hkv, int G, int splits, int pps, float scale_log2, int n_sink,
    int n_local, int top_k, int sink_tokens, int window_tokens, uint64_t static_mask) {
  constexpr int PS = 16, D = 128, DV = 128;
  extern __shared__ __attribute__((aligned(16))) uint64_t dyn[];  // 16-byte aligned: the list is written from 16-byte key loads
  __shared__ sel::SelShared<W> sh;
  const SelectDecodeLds lay(max_pages, max_sel, W, G);
  uint32_t *bits = (uint32_t *)((char *)dyn + lay.bits);
  int32_t *list = (int32_t *)((char *)dyn + lay.list);
  const int item = xcd_contiguous_item(blockIdx.x, gridDim.x);
  const int unit = item / splits, split = item % splits;
  const int b = unit / Hkv, g = unit % Hkv;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int L = seq_lens[b];
  const bool is_static = head_is_static(static_mask, g);
  const size_t head0 = (size_t)b * Hq + (size_t)g * G;
  const int32_t *pt_row = page_table + (size_t)b * pt_stride;
  const int count = sel::select_unit<D, W>(sh, dyn, bits, (max_pages + 31) / 32, scores + (size_t)unit * max_pages,
                                           L, PS, is_static, n_sink, n_local, top_k, sink_tokens, window_tokens,
                                           q + head0 * D, G, summ, pt_row, Hkv, g,
                                           split == 0 ? sel_out + (size_t)unit * max_sel : nullptr, list, max_sel);
  if (split == 0 && threadIdx.x == 0) sel_count_out[unit] = count;
  __syncthreads();  // the list is complete; the keys are dead

  const int sink_end = is_static ? min(sink_tokens, L) : 0;
  const int win_begin = is_static ? max(0, L - window_tokens) : 0;
  const int first = split * pps, last = min(first + pps, count);
  const int npg = max(0, (last - first - wave + W - 1) / W);
  int my_j = 0, my_phys = 0;
  if (lane < npg) {
    my_j = list[first + wave + W * lane];
    my_phys = pt_row[my_j];
  }
  uint4 bq[D / 32];
  attend::load_q_columns<D>(bq, q + head0 * D, G, lane);
  attend::WaveState st;
  attend::init_state(st);
  const attend::PageWork<PS, D, DV> pw{k_pool, v_pool, bq, Hkv, g, L, sink_end, win_begin, is_static, scale_log2};
  attend::attend_pages<PS, D, DV>(st, pw, npg, my_j, my_phys, lane);
  attend::merge_waves<W, DV>((float *)dyn, st, G, [&](int h, int dv, float a, float lsum, float M) {
    if (splits == 1) {
      out[(head0 + h) * DV + dv] = lsum > 0.f ? a / lsum : 0.f;
    } else {
      const size_t ps_idx = (head0 + h) * splits + split;
      partial[ps_idx * DV + dv] = a;
      if (dv == 0) partial_ml[ps_idx] = make_float2(M, lsum);
    }
  });
}

size_t select_decode_lds_bytes(const qasp_layout &lay, const qasp_batch &bat, int max_sel) {
  const int G = bat.num_q_heads / lay.num_kv_heads;
  return SelectDecodeLds(bat.max_pages > 0 ? bat.max_pages : 1, max_sel, kGqaDecodeWaves, G).total +
         sizeof(sel::SelShared<kGqaDecodeWaves>);
}

hipError_t launch_select_decode_gqa(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                                    const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                    const uint16_t *summ, const qasp_score *scores, int32_t *sel, int32_t *sel_count,
                                    int max_sel, float scale, float *out, const Workspace &ws, hipStream_t stream) {
  constexpr int W = kGqaDecodeWaves;
  const int G = bat.num_q_heads / lay.num_kv_heads;
  const int mp = bat.max_pages > 0 ? bat.max_pages : 1;
  const float scale_log2 = scale * 1.4426950408889634f;
  const int pps = (max_sel + ws.splits - 1) / ws.splits;
  const size_t lds = SelectDecodeLds(mp, max_sel, W, G).total;
  dim3 grid((unsigned)ws.splits * lay.num_kv_heads * bat.batch);
  hipLaunchKernelGGL(select_decode_gqa_kernel<W>, grid, dim3(W * 64), lds, stream, q, k_pool, v_pool, summ,
                     bat.page_table, bat.seq_lens, scores, sel, sel_count, ws.partial, ws.partial_ml, out,
                     bat.pt_stride, mp, max_sel, bat.num_q_heads, lay.num_kv_heads, G, ws.splits, pps, scale_log2,
                     pol.n_sink_pages, pol.n_local_pages, pol.top_k, pol.sink_tokens, pol.window_tokens,
                     pol.static_head_mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ws.splits == 1) return e;
  return launch_merge_splits(ws, bat.batch, bat.num_q_heads, lay.head_dim_v, out, stream, 1, G);
}

constexpr int kMergeFew = 4;  // up to this many splits: all of a thread's loads in one round

// Combines the split partials of every (sequence, query head):
// out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.  One block per
// (sequence, head); a thread owns 4 consecutive channels and reads four
// splits' partials per step (16-byte loads, several in flight).  Head h of
// the partials is column h % Gp of KV head h / Gp's group; with nq draft
// queries that column is head (h % Gp) % (Gp / nq) of draft (h % Gp) / (Gp / nq),
// written to out [B][nq][Hq / nq][Dv] (nq = 1: out [B][Hq][Dv]).
__global__ __launch_bounds__(128) void merge_splits_kernel(const float *__restrict__ partial,
                                                           const float2 *__restrict__ partial_ml,
                                                           float *__restrict__ out, int Hq, int splits,
                                                           int dv_dim, int nq, int Gp) {
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t base = ((size_t)b * Hq + h) * splits;
  const int per_query = Gp / nq, col = h % Gp;
  const size_t out_row = ((size_t)b * nq + col / per_query) * (Hq / nq) + (size_t)(h / Gp) * per_query +
                         col % per_query;
  if (splits <= kMergeFew) {  // block-uniform: every load of the thread in one round
    float2 ml[kMergeFew];
#pragma unroll
    for (int s = 0; s < kMergeFew; s++) ml[s] = s < splits ? partial_ml[base + s] : make_float2(-INFINITY, 0.f);
    for (int c = 4 * threadIdx.x; c < dv_dim; c += 4 * blockDim.x) {
      float4 v[kMergeFew];
#pragma unroll
      for (int s = 0; s < kMergeFew; s++)
        v[s] = s < splits ? *(const float4 *)(partial + (base + s) * dv_dim + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      float M = -INFINITY;
#pragma unroll
      for (int s = 0; s < kMergeFew; s++) M = fmaxf(M, ml[s].x);
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
      float lsum = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int s = 0; s < kMergeFew; s++) {
          if (ml[s].x == -INFINITY) continue;  // empty split (or none): no weight
          const float f = __builtin_amdgcn_exp2f(ml[s].x - M);
          lsum += f * ml[s].y;
          a.x += f * v[s].x;
          a.y += f * v[s].y;
          a.z += f * v[s].z;
          a.w += f * v[s].w;
        }
      }
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      *(float4 *)(out + out_row * dv_dim + c) = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    }
    return;
  }
  float M = -INFINITY;
  for (int s = 0; s < splits; s++) M = fmaxf(M, partial_ml[base + s].x);
  for (int c = 4 * threadIdx.x; c < dv_dim; c += 4 * blockDim.x) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float lsum = 0.f;
    if (M != -INFINITY) {
      int s = 0;
      for (; s + 4 <= splits; s += 4) {
        float4 v[4];
        float f[4];
#pragma unroll
        for (int u = 0; u < 4; u++) v[u] = *(const float4 *)(partial + (base + s + u) * dv_dim + c);
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const float2 ml = partial_ml[base + s + u];
          f[u] = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);  // empty split: no weight
          lsum += ml.x == -INFINITY ? 0.f : f[u] * ml.y;
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
          if (f[u] == 0.f) continue;
          a.x += f[u] * v[u].x;
          a.y += f[u] * v[u].y;
          a.z += f[u] * v[u].z;
          a.w += f[u] * v[u].w;
        }
      }
      for (; s < splits; s++) {
        const float2 ml = partial_ml[base + s];
        if (ml.x == -INFINITY) continue;
        const float f = __builtin_amdgcn_exp2f(ml.x - M);
        const float4 v = *(const float4 *)(partial + (base + s) * dv_dim + c);
        a.x += f * v.x;
        a.y += f * v.y;
        a.z += f * v.z;
        a.w += f * v.w;
        lsum += f * ml.y;
      }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    *(float4 *)(out + out_row * dv_dim + c) = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
  }
}

hipError_t launch_merge_splits(const Workspace &ws, int batch, int Hq, int dv_dim, float *out,
                               hipStream_t stream, int nq, int Gp) {
  hipLaunchKernelGGL(merge_splits_kernel, dim3(Hq, batch), dim3(dv_dim >= 512 ? 128 : dv_dim / 4), 0, stream,
                     ws.partial, ws.partial_ml, out, Hq, ws.splits, dv_dim, nq, Gp > 0 ? Gp : Hq);
  return hipGetLastError();
}

hipError_t launch_decode_gqa(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                             const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                             const int32_t *sel, const int32_t *sel_count, int max_sel, float scale,
                             float *out, const Workspace &ws, hipStream_t stream, int nq, int window_q) {
  constexpr int W = kGqaDecodeWaves;
  const int G = bat.num_q_heads / lay.num_kv_heads;
  const float scale_log2 = scale * 1.4426950408889634f;
  const int pps = (max_sel + ws.splits - 1) / ws.splits;
  const size_t lds = (size_t)attend::merge_lds_floats(W, G, 128) * sizeof(float);
  dim3 grid(ws.splits, lay.num_kv_heads, bat.batch);
  auto kernel = nq > 1 ? decode_gqa_kernel<16, 128, 128, W, true> : decode_gqa_kernel<16, 128, 128, W, false>;
  hipLaunchKernelGGL(kernel, grid, dim3(W * 64), lds, stream, q, k_pool, v_pool, bat.page_table, bat.seq_lens,
                     sel, sel_count, ws.partial, ws.partial_ml, out, bat.pt_stride, max_sel, bat.num_q_heads,
                     lay.num_kv_heads, G, ws.splits, pps, scale_log2, pol.sink_tokens, pol.window_tokens,
                     pol.static_head_mask, nq, window_q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ws.splits == 1) return e;
  return launch_merge_splits(ws, bat.batch, bat.num_q_heads, lay.head_dim_v, out, stream, nq, G);
}

}  // namespace qasp
