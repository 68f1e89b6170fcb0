// sparse_paged_decode for latent (MLA) heads: 128 query heads share one
// 576-channel latent KV head whose first 512 channels are the value.
//
// Softmax attention of every query head over the tokens of the selected
// pages only (SubQ/SSA article, section "How SSA works"), reached through the
// page table (Vortex explainer, section 1).  With 128 heads per KV head the
// two products are real matrix products, so they run on MFMA:
//   S^T = K q^T   16x16x32, A = 16 key rows (tokens), B = q^T (16 heads);
//   O^T += V^T P^T  16x16x32, A = V^T (16 value channels x 32 tokens), B = P^T.
//
// Block (split, head group, unit) takes the selected pages [8 split, 8 split
// + 8) of unit (b, g) for 32 of the 128 heads; the four head groups of a
// (unit, split) run on one XCD, so its L2 serves the pages to all four.  A
// page (64 tokens x 1152 bytes) is read from HBM into registers (9 pieces of
// 16 bytes per thread) and stored to LDS token-major (rows padded so the 16
// rows of an A fragment fall on different banks), one page ahead of the
// computation; two page buffers.  Per page, wave w:
//   - S^T of tokens 16 (w % 4) .. +16 and heads 16 (w / 4) .. +16 (18 MFMAs,
//     q^T of its 16 heads kept in registers), softmax weights, which go to an
//     LDS P^T tile (bf16 hi and lo parts);
//   - after a barrier, O^T of value channels 64 w .. 64 w + 63 for all 32
//     heads (2 head tiles x 2 token halves x hi/lo = 32 MFMAs; 32
//     accumulator registers).
// The V^T fragments come straight from the token-major rows through the
// transposing LDS read of gfx950 (ds_read_b64_tr_b16): within a group of 16
// lanes, lane i receives element i % 4 of the 8-byte pieces that lanes 4j +
// i / 4 address (j = 0..3), so pointing lane l' at token 4G + l' / 4,
// channels dv0 + 4 (l' % 4) gives lane i the 4 tokens 4G .. 4G+3 of channel
// dv0 + i, the layout of the MFMA A operand.  The k order of the PV product
// follows: k slot (kg, r) of a lane is token 4kg + r for r < 4 and 16 + 4kg +
// r - 4 for r >= 4 of each 32-token half, and the P^T tile stores its tokens
// in that order, so a B fragment is 16 contiguous bytes.
// Tokens that are not attended (past the length, outside a static head's
// sink and window) are zeroed while staging, so stale pool contents never
// reach the products, and get weight 0.
// P is split into bf16 hi + lo parts (two MFMAs) to keep ~16 significant bits.
// Softmax in the exp2 domain against a fixed reference max per head (the max
// over the first page), so the accumulators are never rescaled: weights stay
// below 2^64 unless a later page's max lies further above the reference, and
// then the block runs its pages again with the largest max seen as reference
// (almost never in practice).  The splits of a unit are combined by
// merge_splits_kernel (four splits of 8 pages for 32 selected pages: 16 MB of
// partials at 16 sequences, against 67 MB with 128 heads x 2 pages per block).
#include "launch.h"
#include "common.h"

namespace qasp {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

constexpr int kD = 576, kDV = 512, kPS = 64, kG = 128;
constexpr int kHeads = 32;                       // heads per block
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;         // 512
constexpr int kKRow = kD * 2 + 16;               // bytes per LDS row (padded): 1168
constexpr int kBufBytes = kPS * kKRow;           // 74752 per page buffer
constexpr int kRowU4 = kD / 8;                   // 72 pieces of 16 bytes per row
constexpr int kStage = kPS * kRowU4 / kThreads;  // 9 loads per thread per page
constexpr int kPRow = kPS * 2 + 16;              // bytes per P^T row (one head, padded): 144
constexpr int kPBytes = kHeads * kPRow;          // 4608 per part (hi, lo)
constexpr float kHeadroom = 64.f;                // weights stay below 2^64 (log2 units)
static_assert(kStage * kThreads == kPS * kRowU4, "whole pages per staging round");
static_assert(kBufBytes % 16 == 0 && kKRow % 16 == 0 && kPRow % 16 == 0, "LDS alignment");
static_assert(kMlaPagesPerSplit <= 16, "page list");

struct MlaDecodeShared {
  int2 pages[kMlaPagesPerSplit];  // (physical page, first position) of the block's pages
  float red[4][kHeads];           // per token quarter and head: max, later sum
  int npages, overflow;
};

__device__ __forceinline__ uint2 pack_bf16x4(const float *a) {
  return make_uint2(f32_to_bf16_rne(a[0]) | (f32_to_bf16_rne(a[1]) << 16),
                    f32_to_bf16_rne(a[2]) | (f32_to_bf16_rne(a[3]) << 16));
}

__device__ __forceinline__ float bf16_round(float a) { return __uint_as_float(f32_to_bf16_rne(a) << 16); }

// Transposing 8-byte LDS read (see the file comment for its lane layout).
__device__ __forceinline__ uint2 lds_read_tr16(const char *p) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)p);
  return __builtin_bit_cast(uint2, v);
}

}  // namespace

__global__ __launch_bounds__(kThreads) void decode_mla_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_pool, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel, const int32_t *__restrict__ sel_count,
    float *__restrict__ partial, float2 *__restrict__ partial_ml, float *__restrict__ out, int pt_stride,
    int max_sel, int Hq, int Hkv, int splits, float scale_log2, int sink_tokens, int window_tokens,
    uint64_t static_mask) {
  extern __shared__ uint4 lds_u4[];
  char *kvbuf = (char *)lds_u4;                 // 2 page buffers
  char *pbuf = kvbuf + 2 * (size_t)kBufBytes;  // P^T hi, then lo
  __shared__ MlaDecodeShared sh;
  constexpr int kGroups = kG / kHeads;  // 4 head groups
  // the head groups and splits of a unit run on one XCD
  const int item = xcd_contiguous_item(blockIdx.x, gridDim.x);
  const int hg = item % kGroups, split = (item / kGroups) % splits, g = (item / (kGroups * splits)) % Hkv,
            b = item / (kGroups * splits * Hkv);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane & 15, kg = lane >> 4;
  const int tq = wave % 4, ht = wave / 4;  // S^T: token quarter, head tile
  const int unit = b * Hkv + g;
  const int L = seq_lens[b];
  const bool is_static = head_is_static(static_mask, g);
  const int sink_end = is_static ? min(sink_tokens, L) : 0;
  const int win_begin = is_static ? max(0, L - window_tokens) : 0;
  auto attended = [&](int pos) {  // branch-free: evaluated per element in the hot loop
    return (pos < L) & (!is_static | (pos < sink_end) | (pos >= win_begin));
  };

  // the block's pages that hold an attended position
  if (tid == 0) {
    const int count = sel_count[unit];
    const int first = split * kMlaPagesPerSplit, last = min(first + kMlaPagesPerSplit, count);
    int np = 0;
    for (int p = first; p < last; p++) {
      const int j = sel[(size_t)unit * max_sel + p];
      const int pos0 = j * kPS, pos1 = min(pos0 + kPS, L);
      if (pos0 < pos1 && (!is_static || pos0 < sink_end || pos1 > win_begin))
        sh.pages[np++] = make_int2(page_table[(size_t)b * pt_stride + j], pos0);
    }
    sh.npages = np;
    sh.overflow = 0;
  }

  // q^T of the wave's S heads: column n = head 32 hg + 16 ht + n, channels 32i + 8kg ..
  const size_t head_base = (size_t)b * Hq + (size_t)g * kG + kHeads * hg;
  uint4 qB[kD / 32];
#pragma unroll
  for (int i = 0; i < kD / 32; i++)
    qB[i] = *(const uint4 *)(q + (head_base + 16 * ht + n) * kD + 32 * i + 8 * kg);
  __syncthreads();
  const int npages = sh.npages;

  // staging: thread loads the 16-byte pieces e = tid + 512 u of a page
  // (token e / 72, channels 8 (e % 72) ..), consecutive lanes along a row
  uint4 stg[kStage];
  auto load_page = [&](int c) {
    const int2 pg = sh.pages[c];
    const uint4 *base = (const uint4 *)(k_pool + ((size_t)pg.x * Hkv + g) * kPS * kD);
#pragma unroll
    for (int u = 0; u < kStage; u++) stg[u] = base[tid + u * kThreads];
  };
  auto store_page = [&](int c, int buf) {
    const int pos0 = sh.pages[c].y;
    char *kb = kvbuf + (size_t)buf * kBufBytes;
#pragma unroll
    for (int u = 0; u < kStage; u++) {
      const int e = tid + u * kThreads, t = e / kRowU4, cb = e % kRowU4;
      const uint32_t k = attended(pos0 + t) ? ~0u : 0u;
      *(uint4 *)(kb + t * kKRow + 16 * cb) = make_uint4(stg[u].x & k, stg[u].y & k, stg[u].z & k, stg[u].w & k);
    }
  };
  // lane's transposing-read address inside a page buffer: token 4kg + n/4, channels 4 (n % 4) ..
  const int tr_off = (4 * kg + n / 4) * kKRow + 8 * (n % 4);
  // where this lane's 4 weights go in the P^T tile: head row 16 ht + n, token
  // slot 32 (tq / 2) + 8 kg + 4 (tq % 2) (the PV k order of the file comment)
  const int p_off = (16 * ht + n) * kPRow + 2 * (32 * (tq / 2) + 8 * kg + 4 * (tq % 2));

  floatx4 acc[4][2];  // O^T: value channel tile 4 wave + d, head tile t
  float m = -INFINITY, l = 0.f, seen = -INFINITY;  // head column n of tile ht (log2 units)
  // one pass over the block's pages with reference m (fixed once set)
  auto run_pass = [&]() {
    l = 0.f;
#pragma unroll
    for (int d = 0; d < 4; d++)
#pragma unroll
      for (int t = 0; t < 2; t++) acc[d][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (npages > 0) {
      load_page(0);
      store_page(0, 0);
    }
    if (npages > 1) load_page(1);
    for (int c = 0; c < npages; c++) {
      const int buf = c & 1;
      const char *kb = kvbuf + (size_t)buf * kBufBytes;
      const int pos0 = sh.pages[c].y;
      __syncthreads();  // page c is in buf; the previous page's products are done (P^T is free)

      // S^T: token 16 tq + 4 kg + r of head column n
      floatx4 s = floatx4{0.f, 0.f, 0.f, 0.f};
      {
        const char *kr = kb + (16 * tq + n) * kKRow + 16 * kg;
#pragma unroll
        for (int i = 0; i < kD / 32; i++) s = mfma16x16x32(*(const uint4 *)(kr + 64 * i), qB[i], s);
      }
      float sv[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const bool ok = attended(pos0 + 16 * tq + 4 * kg + r);
        sv[r] = ok ? s[r] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[r]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));  // this quarter's max of head column n
      if (m == -INFINITY) {  // first page (block-uniform): the reference is its max over all 64 tokens
        if (kg == 0) sh.red[tq][16 * ht + n] = tmax;
        __syncthreads();
        m = fmaxf(fmaxf(sh.red[0][16 * ht + n], sh.red[1][16 * ht + n]),
                  fmaxf(sh.red[2][16 * ht + n], sh.red[3][16 * ht + n]));
      }
      seen = fmaxf(seen, tmax);
      if (__any(tmax > m + kHeadroom) && lane == 0) sh.overflow = 1;
      float p[4], pl[4];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        p[r] = sv[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[r] - m);
        psum += p[r];
        pl[r] = p[r] - bf16_round(p[r]);
      }
      psum += __shfl_xor(psum, 16, kWave);
      psum += __shfl_xor(psum, 32, kWave);
      l += psum;
      *(uint2 *)(pbuf + p_off) = pack_bf16x4(p);
      *(uint2 *)(pbuf + kPBytes + p_off) = pack_bf16x4(pl);
      __syncthreads();  // P^T is complete; every wave is done with the other buffer
      if (c + 1 < npages) {
        store_page(c + 1, buf ^ 1);  // loaded while page c was computed
        if (c + 2 < npages) load_page(c + 2);
      }

      // O^T += V^T P^T over value channels 16 (4 wave + d) + n, both head tiles
      const char *vb = kb + tr_off;
#pragma unroll
      for (int h2 = 0; h2 < 2; h2++) {  // 32-token halves of the page
        uint4 ph[2], plo[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
          const int o = (16 * t + n) * kPRow + 2 * (32 * h2 + 8 * kg);
          ph[t] = *(const uint4 *)(pbuf + o);
          plo[t] = *(const uint4 *)(pbuf + kPBytes + o);
        }
#pragma unroll
        for (int d = 0; d < 4; d++) {
          const int dv0 = 16 * (4 * wave + d);
          const uint2 x0 = lds_read_tr16(vb + (32 * h2) * kKRow + 2 * dv0),
                      x1 = lds_read_tr16(vb + (32 * h2 + 16) * kKRow + 2 * dv0);
          const uint4 a = make_uint4(x0.x, x0.y, x1.x, x1.y);
#pragma unroll
          for (int t = 0; t < 2; t++) {
            acc[d][t] = mfma16x16x32(a, ph[t], acc[d][t]);
            acc[d][t] = mfma16x16x32(a, plo[t], acc[d][t]);
          }
        }
      }
    }
  };
  run_pass();
  __syncthreads();
  if (sh.overflow) {  // some weight could exceed 2^kHeadroom: again, from the largest score seen
    if (kg == 0) sh.red[tq][16 * ht + n] = seen;
    __syncthreads();
    m = fmaxf(fmaxf(sh.red[0][16 * ht + n], sh.red[1][16 * ht + n]),
              fmaxf(sh.red[2][16 * ht + n], sh.red[3][16 * ht + n]));
    __syncthreads();
    run_pass();
    __syncthreads();
  }
  // the heads' sums over the four token quarters
  if (kg == 0) sh.red[tq][16 * ht + n] = l;
  __syncthreads();

  // lane (n, kg) holds O^T rows 16 (4 wave + d) + 4 kg + r of head column n of tile t
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int hc = 16 * t + n;  // head within the block
    const float lsum = sh.red[0][hc] + sh.red[1][hc] + sh.red[2][hc] + sh.red[3][hc];
    const size_t row = head_base + hc;
    if (splits == 1) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
      for (int d = 0; d < 4; d++)
        *(float4 *)(out + row * kDV + 16 * (4 * wave + d) + 4 * kg) =
            make_float4(acc[d][t][0] * inv, acc[d][t][1] * inv, acc[d][t][2] * inv, acc[d][t][3] * inv);
    } else {
      const size_t ps_idx = row * splits + split;
#pragma unroll
      for (int d = 0; d < 4; d++)
        *(float4 *)(partial + ps_idx * kDV + 16 * (4 * wave + d) + 4 * kg) =
            make_float4(acc[d][t][0], acc[d][t][1], acc[d][t][2], acc[d][t][3]);
    }
  }
  // (m, l) of each head, by the wave that holds its reference
  if (splits > 1 && tq == 0 && kg == 0) {
    const int hc = 16 * ht + n;
    const float lsum = sh.red[0][hc] + sh.red[1][hc] + sh.red[2][hc] + sh.red[3][hc];
    partial_ml[(head_base + hc) * splits + split] = make_float2(m, lsum);
  }
}

hipError_t launch_decode_mla(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                             const uint16_t *q, const uint16_t *k_pool, const int32_t *sel,
                             const int32_t *sel_count, int max_sel, float scale, float *out,
                             const Workspace &ws, hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  if (bat.num_q_heads != kG * lay.num_kv_heads) return hipErrorInvalidValue;
  const size_t lds = 2 * (size_t)kBufBytes + 2 * (size_t)kPBytes;
  dim3 grid((unsigned)(kG / kHeads) * ws.splits * lay.num_kv_heads * bat.batch);
  hipLaunchKernelGGL(decode_mla_kernel, grid, dim3(kThreads), lds, stream, q, k_pool, bat.page_table,
                     bat.seq_lens, sel, sel_count, ws.partial, ws.partial_ml, out, bat.pt_stride, max_sel,
                     bat.num_q_heads, lay.num_kv_heads, ws.splits, scale_log2, pol.sink_tokens,
                     pol.window_tokens, pol.static_head_mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ws.splits == 1) return e;
  return launch_merge_splits(ws, bat.batch, bat.num_q_heads, kDV, out, stream);
}

}  // namespace qasp
