// sparse_paged_decode for grouped-query heads (page 16, head_dim 128).
//
// Softmax attention of each query head over the tokens of its group's
// selected pages only, computed exactly on those positions (SubQ/SSA article,
// news.neo-ai.one/ja/article/2719, section "How SSA works"), reached through
// the page table (Vortex explainer, gist.science paper 2606.06453, section 1).
//
// Work split: block (split, g, b) takes selected pages
// [pps*split, pps*split + pps) of unit (b, g); its WAVES waves take every
// WAVES-th page.  Per page-head a wave
//   - loads the 16x128 key tile straight into the A operand of 4 MFMAs
//     (16x16x32): lane (token m = l%16, k block l/16) reads 16 contiguous
//     bytes of key row m, so the 64 lanes read the page-head's 4 KiB once;
//   - S^T = K q^T puts token 4*(l/16)+r of head l%16 in lane l, register r;
//   - online softmax in the exp2 domain per head (running max m, sum l);
//   - O^T += V^T P with 16x16x16 MFMAs: the value tile is stored transposed
//     ([dv][token], tokens fastest), so lane (dv = l%16, l/16) reads 4
//     consecutive tokens as 8 contiguous bytes, and P^T comes straight from
//     the S^T registers.  P is split into bf16 hi + lo parts (two MFMAs) so
//     the weights keep ~16 significant bits.
// The waves merge through LDS.  With one split per unit the block writes the
// output; otherwise it writes a partial (m, l, acc) and merge_splits_kernel
// combines the partials (a kernel boundary orders the two, no device-wide
// fences inside a kernel).
#include "common.h"
#include "launch.h"

namespace qasp {

namespace {

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16),
                    f32_to_bf16_rne(c) | (f32_to_bf16_rne(d) << 16));
}
__device__ __forceinline__ float bf16_round_f32(float a) { return __uint_as_float(f32_to_bf16_rne(a) << 16); }

}  // namespace

template <int PS, int D, int DV, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void decode_gqa_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_pool,
    const uint16_t *__restrict__ v_pool, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ sel_count, float *__restrict__ partial,
    float2 *__restrict__ partial_ml, float *__restrict__ out, int pt_stride, int max_sel, int Hq,
    int Hkv, int G, int splits, int pps, float scale_log2, int sink_tokens, int window_tokens,
    uint64_t static_mask) {
  static_assert(PS == 16 && D == 128 && DV == 128, "tile shapes");
  constexpr int ROW = DV + 4;  // padded LDS row of one head's accumulator
  extern __shared__ float lds[];
  float *sm_m = lds;                      // [WAVES][G]
  float *sm_l = sm_m + WAVES * G;         // [WAVES][G]
  float *sm_acc = sm_l + WAVES * G;       // [WAVES][G][ROW]
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane & 15, kg = lane >> 4;
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

  // q^T as the B operand: column n = head g*G + n, k block kg
  uint4 bq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; i++)
    bq[i] = n < G ? *(const uint4 *)(q + ((size_t)b * Hq + (size_t)g * G + n) * D + 32 * i + 8 * kg)
                  : make_uint4(0, 0, 0, 0);

  float m_run = -INFINITY, l_run = 0.f;
  floatx4 acc[DV / 16];
#pragma unroll
  for (int i = 0; i < DV / 16; i++) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};

  // three register stages: while page i is computed, pages i+1 and i+2 load
  uint4 kA[D / 32], kB[D / 32], kC[D / 32];
  uint2 vA[DV / 16], vB[DV / 16], vC[DV / 16];
  auto load_page = [&](int it, uint4 *kk, uint2 *vv) {
    const int phys = __shfl(my_phys, it, kWave);
    const size_t ph = (size_t)phys * Hkv + g;
    const uint16_t *kp = k_pool + (ph * PS + n) * D + 8 * kg;
    const uint16_t *vp = v_pool + ph * DV * PS + (size_t)n * PS + 4 * kg;
#pragma unroll
    for (int i = 0; i < D / 32; i++) kk[i] = *(const uint4 *)(kp + 32 * i);
#pragma unroll
    for (int i = 0; i < DV / 16; i++) vv[i] = *(const uint2 *)(vp + 16 * i * PS);
  };
  auto compute_page = [&](int it, const uint4 *kt, const uint2 *vt) {
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D / 32; i++) s = mfma16x16x32(kt[i], bq[i], s);
    const int j = __shfl(my_j, it, kWave);
    float sv[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int pos = j * PS + 4 * kg + r;
      const bool ok = pos < L && (!is_static || pos < sink_end || pos >= win_begin);
      sv[r] = ok ? s[r] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, sv[r]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);
    float alpha = 1.f;
    float p[4];
    if (m_new == -INFINITY) {
#pragma unroll
      for (int r = 0; r < 4; r++) p[r] = 0.f;
    } else {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int r = 0; r < 4; r++) p[r] = sv[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[r] - m_new);
    }
    float psum = (p[0] + p[1]) + (p[2] + p[3]);
    psum += __shfl_xor(psum, 16, kWave);
    psum += __shfl_xor(psum, 32, kWave);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const uint2 ph = pack_bf16x4(p[0], p[1], p[2], p[3]);
    const uint2 pl = pack_bf16x4(p[0] - bf16_round_f32(p[0]), p[1] - bf16_round_f32(p[1]),
                                 p[2] - bf16_round_f32(p[2]), p[3] - bf16_round_f32(p[3]));
#pragma unroll
    for (int i = 0; i < DV / 16; i++) {
      acc[i] *= alpha;
      acc[i] = mfma16x16x16(vt[i], ph, acc[i]);
      acc[i] = mfma16x16x16(vt[i], pl, acc[i]);
    }
  };
  // page it computes from (kc, vc) after prefetching page it+2 into (kn, vn);
  // the buffer roles rotate through the unrolled body, so no register copies
  // wait on loads in flight
  auto page_step = [&](int it, const uint4 *kc, const uint2 *vc, uint4 *kn, uint2 *vn) {
    if (it + 2 < npg) load_page(it + 2, kn, vn);
    compute_page(it, kc, vc);
  };
  if (npg > 0) load_page(0, kA, vA);
  if (npg > 1) load_page(1, kB, vB);
  for (int it = 0; it < npg; it += 3) {
    page_step(it, kA, vA, kC, vC);
    if (it + 1 < npg) page_step(it + 1, kB, vB, kA, vA);
    if (it + 2 < npg) page_step(it + 2, kC, vC, kB, vB);
  }

  // merge the waves: lanes of head column n < G publish their state
  if (n < G) {
    if (kg == 0) {
      sm_m[wave * G + n] = m_run;
      sm_l[wave * G + n] = l_run;
    }
    float *row = sm_acc + ((size_t)wave * G + n) * ROW;
#pragma unroll
    for (int i = 0; i < DV / 16; i++)
#pragma unroll
      for (int r = 0; r < 4; r++) row[16 * i + 4 * kg + r] = acc[i][r];
  }
  __syncthreads();
  const size_t head0 = (size_t)b * Hq + (size_t)g * G;
  for (int item = tid; item < G * DV; item += WAVES * 64) {
    const int h = item / DV, dv = item % DV;
    float M = sm_m[h];
#pragma unroll
    for (int w = 1; w < WAVES; w++) M = fmaxf(M, sm_m[w * G + h]);
    float a = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; w++) {
        const float f = __builtin_amdgcn_exp2f(sm_m[w * G + h] - M);  // exp2(-inf) = 0
        a += f * sm_acc[((size_t)w * G + h) * ROW + dv];
        lsum += f * sm_l[w * G + h];
      }
    }
    if (splits == 1) {
      out[(head0 + h) * DV + dv] = lsum > 0.f ? a / lsum : 0.f;
    } else {
      const size_t ps_idx = (head0 + h) * splits + split;
      partial[ps_idx * DV + dv] = a;
      if (dv == 0) partial_ml[ps_idx] = make_float2(M, lsum);
    }
  }
}

// Combines the split partials of every (sequence, query head):
// out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
__global__ __launch_bounds__(256) void merge_splits_kernel(const float *__restrict__ partial,
                                                           const float2 *__restrict__ partial_ml,
                                                           float *__restrict__ out, int Hq, int splits,
                                                           int dv_dim) {
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t base = ((size_t)b * Hq + h) * splits;
  float M = -INFINITY;
  for (int s = 0; s < splits; s++) M = fmaxf(M, partial_ml[base + s].x);
  for (int dv = threadIdx.x; dv < dv_dim; dv += blockDim.x) {
    float a = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < splits; s++) {
        const float2 ml = partial_ml[base + s];
        const float f = __builtin_amdgcn_exp2f(ml.x - M);
        a += f * partial[(base + s) * dv_dim + dv];
        lsum += f * ml.y;
      }
    }
    out[((size_t)b * Hq + h) * dv_dim + dv] = lsum > 0.f ? a / lsum : 0.f;
  }
}

hipError_t launch_merge_splits(const Workspace &ws, int batch, int Hq, int dv_dim, float *out,
                               hipStream_t stream) {
  hipLaunchKernelGGL(merge_splits_kernel, dim3(Hq, batch), dim3(dv_dim <= 128 ? 128 : 256), 0, stream,
                     ws.partial, ws.partial_ml, out, Hq, ws.splits, dv_dim);
  return hipGetLastError();
}

hipError_t launch_decode_gqa(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                             const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                             const int32_t *sel, const int32_t *sel_count, int max_sel, float scale,
                             float *out, const Workspace &ws, hipStream_t stream) {
  constexpr int W = kGqaDecodeWaves;
  const int G = bat.num_q_heads / lay.num_kv_heads;
  const float scale_log2 = scale * 1.4426950408889634f;
  const int pps = (max_sel + ws.splits - 1) / ws.splits;
  const size_t lds = (size_t)(2 * W * G + W * G * (128 + 4)) * sizeof(float);
  dim3 grid(ws.splits, lay.num_kv_heads, bat.batch);
  hipLaunchKernelGGL((decode_gqa_kernel<16, 128, 128, W>), grid, dim3(W * 64), lds, stream, q, k_pool,
                     v_pool, bat.page_table, bat.seq_lens, sel, sel_count, ws.partial, ws.partial_ml, out,
                     bat.pt_stride, max_sel, bat.num_q_heads, lay.num_kv_heads, G, ws.splits, pps,
                     scale_log2, pol.sink_tokens, pol.window_tokens, pol.static_head_mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ws.splits == 1) return e;
  return launch_merge_splits(ws, bat.batch, bat.num_q_heads, lay.head_dim_v, out, stream);
}

}  // namespace qasp
