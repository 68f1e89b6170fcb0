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
// Block (split, g, b) takes the selected pages [P split, P split + P) of
// unit (b, g) and all 128 heads; wave w (of 8) owns heads 16w .. 16w+15,
// keeps their q^T (the B operand, 72 registers) and their O^T (16 heads x
// 512 channels, 128 accumulators per lane).  Two waves share each SIMD, so
// one wave's LDS reads overlap the other's MFMAs.  Tokens go through in
// chunks of 32, read from HBM once per block into registers and stored to
// LDS token-major (rows padded so the 16 rows of an A fragment fall on
// different banks); the next chunk is loaded while the current one is
// computed.  The V^T fragments come straight from the token-major rows
// through the transposing LDS read of gfx950 (ds_read_b64_tr_b16): within a
// group of 16 lanes, lane i receives element i % 4 of the 8-byte pieces that
// lanes 4j + i / 4 address (j = 0..3), so pointing lane l' at token
// 4G + l' / 4, channels dv0 + 4 (l' % 4) gives lane i the 4 tokens
// 4G .. 4G+3 of channel dv0 + i, the layout of the MFMA A operand.
// Tokens that are not attended (past the length, outside a static head's
// sink and window) are zeroed while staging, so stale pool contents never
// reach the products.
// The k order of the PV product: k slot (kg, r) of a lane is token 4kg + r
// for r < 4 and 16 + 4kg + r - 4 for r >= 4, the order in which the two
// 16-token S^T blocks come out of the QK product, so P^T needs no shuffle.
// P is split into bf16 hi + lo parts (two MFMAs) to keep ~16 significant bits.
// Softmax in the exp2 domain against a fixed reference max per head (the max
// of the first attended chunk), so the accumulators are never rescaled:
// weights stay below 2^64 unless a later chunk's max lies further above the
// reference, and then the block starts its pages again with the largest max
// seen as reference (almost never in practice).
// Several splits per unit are combined by merge_splits_kernel.
#include "launch.h"
#include "common.h"

namespace qasp {

hipError_t launch_merge_splits(const Workspace &ws, int batch, int Hq, int dv_dim, float *out,
                               hipStream_t stream);

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

constexpr int kD = 576, kDV = 512, kPS = 64, kG = 128;
constexpr int kChunk = 32;                       // tokens per staged chunk
constexpr int kWaves = kG / 16;                  // 8, one 16-head block each
constexpr int kThreads = kWaves * kWave;         // 512
constexpr int kKRow = kD * 2 + 16;               // bytes per LDS row (padded): 1168
constexpr int kBufBytes = kChunk * kKRow;        // 37376 per buffer
constexpr int kRowU4 = kD / 8;                   // 72 uint4 per row
constexpr int kStage = (kChunk * kRowU4 + kThreads - 1) / kThreads;  // 5 loads per thread per chunk
constexpr int kMaxChunks = kMlaPagesPerSplit * (kPS / kChunk);
constexpr float kHeadroom = 64.f;                // weights stay below 2^64 (log2 units)
static_assert(kBufBytes % 16 == 0 && kKRow % 16 == 0, "LDS alignment");

__device__ __forceinline__ uint4 pack_bf16x8(const float *a, const float *b) {
  return make_uint4(f32_to_bf16_rne(a[0]) | (f32_to_bf16_rne(a[1]) << 16),
                    f32_to_bf16_rne(a[2]) | (f32_to_bf16_rne(a[3]) << 16),
                    f32_to_bf16_rne(b[0]) | (f32_to_bf16_rne(b[1]) << 16),
                    f32_to_bf16_rne(b[2]) | (f32_to_bf16_rne(b[3]) << 16));
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
  char *lds = (char *)lds_u4;
  __shared__ int2 chunks[kMaxChunks];  // (physical page, position of the chunk's first token)
  __shared__ int nchunks_sh, overflow;
  // the splits of a unit run on one XCD, which then reads its q once into L2
  const int item = xcd_contiguous_item(blockIdx.x, gridDim.x);
  const int split = item % splits, g = (item / splits) % Hkv, b = item / (splits * Hkv);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane & 15, kg = lane >> 4;
  const int unit = b * Hkv + g;
  const int L = seq_lens[b];
  const bool is_static = head_is_static(static_mask, g);
  const int sink_end = is_static ? min(sink_tokens, L) : 0;
  const int win_begin = is_static ? max(0, L - window_tokens) : 0;
  auto attended = [&](int pos) {  // branch-free: evaluated per element in the hot loop
    return (pos < L) & (!is_static | (pos < sink_end) | (pos >= win_begin));
  };

  // the block's chunks: halves of its pages that hold an attended position
  if (tid == 0) {
    const int count = sel_count[unit];
    const int first = split * kMlaPagesPerSplit, last = min(first + kMlaPagesPerSplit, count);
    int nc = 0;
    for (int p = first; p < last; p++) {
      const int j = sel[(size_t)unit * max_sel + p];
      const int phys = page_table[(size_t)b * pt_stride + j];
      for (int h = 0; h < kPS / kChunk; h++) {
        const int pos0 = j * kPS + h * kChunk, pos1 = min(pos0 + kChunk, L);  // [pos0, pos1) below L
        const bool any = pos0 < pos1 && (!is_static || pos0 < sink_end || pos1 > win_begin);
        if (any) chunks[nc++] = make_int2(phys, pos0);
      }
    }
    nchunks_sh = nc;
    overflow = 0;
  }

  // q^T of the wave's heads: column n = head 16 wave + n, channels 32i + 8kg ..
  const size_t head0 = (size_t)b * Hq + (size_t)g * kG + 16 * wave;
  uint4 qB[kD / 32];
#pragma unroll
  for (int i = 0; i < kD / 32; i++) qB[i] = *(const uint4 *)(q + (head0 + n) * kD + 32 * i + 8 * kg);
  __syncthreads();
  const int nchunks = nchunks_sh;

  // staging: thread loads the 16-byte pieces e = tid + 512 u of the chunk
  // (token e / 72, channels 8 (e % 72) ..), consecutive lanes along a row
  uint4 stg[kStage];
  auto load_chunk = [&](int c) {
    const int2 ch = chunks[c];
    const uint4 *base = (const uint4 *)(k_pool + (((size_t)ch.x * Hkv + g) * kPS + (ch.y % kPS)) * kD);
#pragma unroll
    for (int u = 0; u < kStage; u++) stg[u] = base[min(tid + u * kThreads, kChunk * kRowU4 - 1)];
  };
  auto store_chunk = [&](int c, int buf) {
    const int pos0 = chunks[c].y;
    char *kb = lds + (size_t)buf * kBufBytes;
#pragma unroll
    for (int u = 0; u < kStage; u++) {
      const int e = tid + u * kThreads;
      if (e < kChunk * kRowU4) {
        const int t = e / kRowU4, cb = e % kRowU4;
        const uint32_t k = attended(pos0 + t) ? ~0u : 0u;
        *(uint4 *)(kb + t * kKRow + 16 * cb) = make_uint4(stg[u].x & k, stg[u].y & k, stg[u].z & k, stg[u].w & k);
      }
    }
  };
  // lane's transposing-read address inside a buffer: token 4kg + n/4, channels 4 (n % 4) ..
  const int tr_off = (4 * kg + n / 4) * kKRow + 8 * (n % 4);

  floatx4 acc[kDV / 16];
  float m = -INFINITY, l = 0.f, seen = -INFINITY;  // per head column n (log2 units)
  // one pass over the block's chunks with reference m (fixed once set)
  auto run_pass = [&]() {
    l = 0.f;
#pragma unroll
    for (int d = 0; d < kDV / 16; d++) acc[d] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (nchunks > 0) {
      load_chunk(0);
      store_chunk(0, 0);
    }
    if (nchunks > 1) load_chunk(1);
    __syncthreads();
    for (int c = 0; c < nchunks; c++) {
      const int buf = c & 1;
      const char *kb = lds + (size_t)buf * kBufBytes;
      const int pos0 = chunks[c].y;

      // S^T: token 16 tb + 4 kg + r of head column n
      floatx4 s[2];
#pragma unroll
      for (int tb = 0; tb < 2; tb++) {
        s[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
        const char *kr = kb + (16 * tb + n) * kKRow + 16 * kg;
#pragma unroll
        for (int i = 0; i < kD / 32; i++) s[tb] = mfma16x16x32(*(const uint4 *)(kr + 64 * i), qB[i], s[tb]);
      }

      // softmax weights against the reference max; P^T hi / lo as the B operand
      float sv[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; tb++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const bool ok = attended(pos0 + 16 * tb + 4 * kg + r);
          sv[tb][r] = ok ? s[tb][r] * scale_log2 : -INFINITY;
          tmax = fmaxf(tmax, sv[tb][r]);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
      seen = fmaxf(seen, tmax);
      if (m == -INFINITY) m = tmax;  // first attended chunk: nothing accumulated yet
      if (__any(tmax > m + kHeadroom) && lane == 0) overflow = 1;
      float p[2][4], pl[2][4];
      float psum = 0.f;
#pragma unroll
      for (int tb = 0; tb < 2; tb++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          p[tb][r] = sv[tb][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[tb][r] - m);
          psum += p[tb][r];
          pl[tb][r] = p[tb][r] - bf16_round(p[tb][r]);
        }
      psum += __shfl_xor(psum, 16, kWave);
      psum += __shfl_xor(psum, 32, kWave);
      l += psum;
      const uint4 phi = pack_bf16x8(p[0], p[1]);
      const uint4 plo = pack_bf16x8(pl[0], pl[1]);

      // O^T += V^T P^T over value channels 16 d + n
      const char *vb = kb + tr_off;
#pragma unroll
      for (int d = 0; d < kDV / 16; d++) {
        const uint2 x0 = lds_read_tr16(vb + 32 * d), x1 = lds_read_tr16(vb + 16 * kKRow + 32 * d);
        const uint4 a = make_uint4(x0.x, x0.y, x1.x, x1.y);
        acc[d] = mfma16x16x32(a, phi, acc[d]);
        acc[d] = mfma16x16x32(a, plo, acc[d]);
      }

      __syncthreads();  // every wave is done with buffer buf
      if (c + 1 < nchunks) {
        store_chunk(c + 1, buf ^ 1);  // loaded while chunk c was computed
        if (c + 2 < nchunks) load_chunk(c + 2);
        __syncthreads();
      }
    }
  };
  run_pass();
  if (overflow) {  // some weight could exceed 2^kHeadroom: again, from the largest score seen
    m = seen;
    run_pass();
  }

  // lane (n, kg) holds O^T rows 16 d + 4 kg + r of head column n
  const size_t row = head0 + n;
  if (splits == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int d = 0; d < kDV / 16; d++)
      *(float4 *)(out + row * kDV + 16 * d + 4 * kg) =
          make_float4(acc[d][0] * inv, acc[d][1] * inv, acc[d][2] * inv, acc[d][3] * inv);
  } else {
    const size_t ps_idx = row * splits + split;
#pragma unroll
    for (int d = 0; d < kDV / 16; d++)
      *(float4 *)(partial + ps_idx * kDV + 16 * d + 4 * kg) = make_float4(acc[d][0], acc[d][1], acc[d][2], acc[d][3]);
    if (kg == 0) partial_ml[ps_idx] = make_float2(m, l);
  }
}

hipError_t launch_decode_mla(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                             const uint16_t *q, const uint16_t *k_pool, const int32_t *sel,
                             const int32_t *sel_count, int max_sel, float scale, float *out,
                             const Workspace &ws, hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const size_t lds = 2 * (size_t)kBufBytes;
  dim3 grid((unsigned)ws.splits * lay.num_kv_heads * bat.batch);
  hipLaunchKernelGGL(decode_mla_kernel, grid, dim3(kThreads), lds, stream, q, k_pool, bat.page_table,
                     bat.seq_lens, sel, sel_count, ws.partial, ws.partial_ml, out, bat.pt_stride, max_sel,
                     bat.num_q_heads, lay.num_kv_heads, ws.splits, scale_log2, pol.sink_tokens,
                     pol.window_tokens, pol.static_head_mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ws.splits == 1) return e;
  return launch_merge_splits(ws, bat.batch, bat.num_q_heads, kDV, out, stream);
}

}  // namespace qasp
