// sparse_paged_decode for grouped-query heads (page 16, head_dim 128).
//
// Softmax attention of each query head over the tokens of its group's
// selected pages only, computed exactly on those positions (SubQ/SSA article,
// news.neo-ai.one/ja/article/2719, section "How SSA works"), reached through
// the page table (Vortex explainer, gist.science paper 2606.06453, section 1).
//
// Work split: block (split, g, b) takes selected pages [32*split, 32*split+32)
// of unit (b, g); its 4 waves take every 4th page.  Per page-head a wave
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
// The 4 waves merge through LDS; with several splits the last block to
// arrive (arrival counter per unit) merges the split partials.
#include "common.h"
#include "launch.h"

namespace qasp {

namespace {

constexpr int kDecWaves = 4;

struct DecShared {
  float m[kDecWaves][16];
  float l[kDecWaves][16];
  float acc[kDecWaves][16][128 + 4];
  int last;
};

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16),
                    f32_to_bf16_rne(c) | (f32_to_bf16_rne(d) << 16));
}
__device__ __forceinline__ float bf16_round_f32(float a) { return __uint_as_float(f32_to_bf16_rne(a) << 16); }

}  // namespace

template <int PS, int D, int DV>
__global__ __launch_bounds__(256) void decode_gqa_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_pool,
    const uint16_t *__restrict__ v_pool, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ sel_count, float *__restrict__ partial,
    float2 *__restrict__ partial_ml, uint32_t *__restrict__ counters, float *__restrict__ out,
    int pt_stride, int max_sel, int Hq, int Hkv, int G, int splits, float scale_log2,
    int sink_tokens, int window_tokens, uint64_t static_mask) {
  static_assert(PS == 16 && D == 128 && DV == 128, "tile shapes");
  constexpr int PPS = kGqaPagesPerSplit;
  constexpr int PPW = PPS / kDecWaves;  // pages per wave
  __shared__ DecShared sh;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane & 15, kg = lane >> 4;
  const int unit = b * Hkv + g;
  const int L = seq_lens[b];
  const bool is_static = head_is_static(static_mask, g);
  const int sink_end = is_static ? min(sink_tokens, L) : 0;
  const int win_begin = is_static ? max(0, L - window_tokens) : 0;
  const int count = sel_count[unit];
  const int first = split * PPS, last = min(first + PPS, count);
  const int npg = max(0, (last - first - wave + kDecWaves - 1) / kDecWaves);

  // lane i < PPW holds the logical id and physical page of this wave's i-th page
  int my_j = 0, my_phys = 0;
  if (lane < PPW) {
    const int idx = first + wave + kDecWaves * lane;
    if (idx < last) {
      my_j = sel[(size_t)unit * max_sel + idx];
      my_phys = page_table[(size_t)b * pt_stride + my_j];
    }
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

  uint4 kt[D / 32], kt_next[D / 32];
  uint2 vt[DV / 16], vt_next[DV / 16];
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
  if (npg > 0) load_page(0, kt, vt);

  for (int it = 0; it < npg; it++) {
    if (it + 1 < npg) load_page(it + 1, kt_next, vt_next);
    // scores of the page's 16 tokens for the 16 head columns
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
    if (it + 1 < npg) {
#pragma unroll
      for (int i = 0; i < D / 32; i++) kt[i] = kt_next[i];
#pragma unroll
      for (int i = 0; i < DV / 16; i++) vt[i] = vt_next[i];
    }
  }

  // merge the 4 waves
  if (kg == 0) {
    sh.m[wave][n] = m_run;
    sh.l[wave][n] = l_run;
  }
#pragma unroll
  for (int i = 0; i < DV / 16; i++)
#pragma unroll
    for (int r = 0; r < 4; r++) sh.acc[wave][n][16 * i + 4 * kg + r] = acc[i][r];
  __syncthreads();
  const size_t head0 = (size_t)b * Hq + (size_t)g * G;
  for (int item = tid; item < G * DV; item += blockDim.x) {
    const int h = item / DV, dv = item % DV;
    float M = sh.m[0][h];
#pragma unroll
    for (int w = 1; w < kDecWaves; w++) M = fmaxf(M, sh.m[w][h]);
    float a = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecWaves; w++) {
        const float f = __builtin_amdgcn_exp2f(sh.m[w][h] - M);  // exp2(-inf) = 0
        a += f * sh.acc[w][h][dv];
        lsum += f * sh.l[w][h];
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
  if (splits == 1) return;

  // the last block of the unit to arrive merges the splits
  __threadfence();
  __syncthreads();
  if (tid == 0) sh.last = atomicAdd(&counters[unit], 1u) == (uint32_t)(splits - 1);
  __syncthreads();
  if (!sh.last) return;
  __threadfence();
  for (int item = tid; item < G * DV; item += blockDim.x) {
    const int h = item / DV, dv = item % DV;
    const size_t base = (head0 + h) * splits;
    float M = -INFINITY;
    for (int s2 = 0; s2 < splits; s2++) M = fmaxf(M, __builtin_nontemporal_load(&partial_ml[base + s2].x));
    float a = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
      for (int s2 = 0; s2 < splits; s2++) {
        const float mx = __builtin_nontemporal_load(&partial_ml[base + s2].x);
        const float ly = __builtin_nontemporal_load(&partial_ml[base + s2].y);
        const float f = __builtin_amdgcn_exp2f(mx - M);
        a += f * __builtin_nontemporal_load(&partial[(base + s2) * DV + dv]);
        lsum += f * ly;
      }
    }
    out[(head0 + h) * DV + dv] = lsum > 0.f ? a / lsum : 0.f;
  }
  if (tid == 0) counters[unit] = 0;
}

hipError_t launch_decode_gqa(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                             const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                             const int32_t *sel, const int32_t *sel_count, int max_sel, float scale,
                             float *out, const Workspace &ws, hipStream_t stream) {
  const int G = bat.num_q_heads / lay.num_kv_heads;
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid(ws.splits, lay.num_kv_heads, bat.batch);
  hipLaunchKernelGGL((decode_gqa_kernel<16, 128, 128>), grid, dim3(256), 0, stream, q, k_pool, v_pool,
                     bat.page_table, bat.seq_lens, sel, sel_count, ws.partial, ws.partial_ml,
                     ws.counters, out, bat.pt_stride, max_sel, bat.num_q_heads, lay.num_kv_heads, G,
                     ws.splits, scale_log2, pol.sink_tokens, pol.window_tokens, pol.static_head_mask);
  return hipGetLastError();
}

}  // namespace qasp
