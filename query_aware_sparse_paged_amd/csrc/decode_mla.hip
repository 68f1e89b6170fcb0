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
// Block (split, g, b) takes the selected pages [2 split, 2 split + 2) of unit
// (b, g) and all 128 heads; wave w owns heads 32w .. 32w+31 (two 16-head
// column blocks), keeps their q^T (B operand) in registers and their O^T
// (32 heads x 512 channels, 256 floats per lane) in the accumulation
// registers.  Tokens go through in chunks of 32, each read from HBM once per
// block and staged twice in LDS (double-buffered, the next chunk's loads in
// flight while the current one is computed):
//   Ktok  token-major rows, row stride padded to spread the 16 rows of an
//         A fragment over the banks;
//   Vt    the 512 value channels channel-major (32 tokens per row), made by
//         a 4x8 transpose in registers, so a V^T fragment is two 8-byte reads.
// Tokens that are not attended (past the length, outside a static head's
// sink and window) are zeroed while staging, so stale pool contents never
// reach the products.
// The k order of the PV product: k slot (kg, r) of a lane is token 4kg + r
// for r < 4 and 16 + 4kg + r - 4 for r >= 4, the order in which the two
// 16-token S^T blocks come out of the QK product, so P^T needs no shuffle.
// P is split into bf16 hi + lo parts (two MFMAs) to keep ~16 significant bits.
// Softmax in the exp2 domain against a fixed reference max per head (the max
// of the first attended chunk), so the 256 accumulators are never rescaled:
// weights stay below 2^64 unless a later chunk's max lies further above the
// reference, and then the block starts its pages again with the largest max
// seen as reference (at most once per chunk, almost never in practice).
// Several splits per unit are combined by merge_splits_kernel.
#include "launch.h"
#include "common.h"

namespace qasp {

hipError_t launch_merge_splits(const Workspace &ws, int batch, int Hq, int dv_dim, float *out,
                               hipStream_t stream);

namespace {

constexpr int kD = 576, kDV = 512, kPS = 64, kG = 128;
constexpr int kChunk = 32;                       // tokens per staged chunk
constexpr int kHB = 2;                           // 16-head column blocks per wave
constexpr int kWaves = kG / (16 * kHB);          // 4
constexpr int kThreads = kWaves * kWave;         // 256
constexpr int kKRow = kD * 2 + 16;               // bytes per Ktok row (padded)
constexpr int kVRow = kChunk * 2 + 8;            // bytes per Vt row (padded)
constexpr int kKBytes = kChunk * kKRow;          // 37376
constexpr int kVBytes = kDV * kVRow;             // 36864
constexpr int kBufBytes = kKBytes + kVBytes;     // 74240 per buffer
constexpr int kMaxChunks = kMlaPagesPerSplit * (kPS / kChunk);
constexpr float kHeadroom = 64.f;                // weights stay below 2^64 (log2 units)
static_assert((kChunk / 4) * (kDV / 8) == 2 * kThreads, "two V items (4 tokens x 8 channels) per thread");
static_assert(kChunk * (kD - kDV) / 8 == kThreads, "one 16-byte rope load per thread");
static_assert(kBufBytes % 16 == 0 && kKBytes % 16 == 0, "LDS alignment");

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

__device__ __forceinline__ uint4 pack_bf16x8(const float *a, const float *b) {
  return make_uint4(f32_to_bf16_rne(a[0]) | (f32_to_bf16_rne(a[1]) << 16),
                    f32_to_bf16_rne(a[2]) | (f32_to_bf16_rne(a[3]) << 16),
                    f32_to_bf16_rne(b[0]) | (f32_to_bf16_rne(b[1]) << 16),
                    f32_to_bf16_rne(b[2]) | (f32_to_bf16_rne(b[3]) << 16));
}

__device__ __forceinline__ float bf16_round(float a) { return __uint_as_float(f32_to_bf16_rne(a) << 16); }

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
  __shared__ int nchunks_sh;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
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
  auto keep_if = [](uint4 v, bool keep) {
    const uint32_t k = keep ? ~0u : 0u;
    return make_uint4(v.x & k, v.y & k, v.z & k, v.w & k);
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
  }

  // q^T of the wave's heads: column n of block hb = head 32 wave + 16 hb + n
  const size_t head0 = (size_t)b * Hq + (size_t)g * kG + 32 * wave;
  uint4 qB[kHB][kD / 32];
#pragma unroll
  for (int hb = 0; hb < kHB; hb++)
#pragma unroll
    for (int i = 0; i < kD / 32; i++)
      qB[hb][i] = *(const uint4 *)(q + (head0 + 16 * hb + n) * kD + 32 * i + 8 * kg);
  __syncthreads();
  const int nchunks = nchunks_sh;

  // staging in two parts, each a set of loads held in registers until stored:
  // part 0 = V item 0, part 1 = V item 1 and the rope channels.  A V item is
  // (token quad a, channel block cb): four 16-byte loads, one per token.
  uint4 rv[4], rr;
  auto load_part = [&](int c, int part) {
    const int2 ch = chunks[c];
    const uint16_t *base = k_pool + (((size_t)ch.x * Hkv + g) * kPS + (ch.y % kPS)) * kD;
    const int e = tid + part * kThreads, a = e & 7, cb = e >> 3;
#pragma unroll
    for (int y = 0; y < 4; y++) rv[y] = *(const uint4 *)(base + (size_t)(4 * a + y) * kD + 8 * cb);
    if (part == 1) {
      const int t = tid >> 3, rb = kDV / 8 + (tid & 7);
      rr = *(const uint4 *)(base + (size_t)t * kD + 8 * rb);
    }
  };
  auto store_part = [&](int c, int buf, int part) {
    const int pos0 = chunks[c].y;
    char *kb = lds + (size_t)buf * kBufBytes;
    char *vb = kb + kKBytes;
    const int e = tid + part * kThreads, a = e & 7, cb = e >> 3;
    uint4 r[4];
#pragma unroll
    for (int y = 0; y < 4; y++) {
      r[y] = keep_if(rv[y], attended(pos0 + 4 * a + y));
      *(uint4 *)(kb + (4 * a + y) * kKRow + 16 * cb) = r[y];
    }
    // channel 8 cb + 2w (+1), tokens 4a .. 4a+3
#pragma unroll
    for (int w = 0; w < 4; w++) {
      const uint32_t d0 = word_of(r[0], w), d1 = word_of(r[1], w), d2 = word_of(r[2], w), d3 = word_of(r[3], w);
      const uint2 lo = make_uint2((d0 & 0xffffu) | (d1 << 16), (d2 & 0xffffu) | (d3 << 16));
      const uint2 hi = make_uint2((d0 >> 16) | (d1 & 0xffff0000u), (d2 >> 16) | (d3 & 0xffff0000u));
      *(uint2 *)(vb + (8 * cb + 2 * w) * kVRow + 8 * a) = lo;
      *(uint2 *)(vb + (8 * cb + 2 * w + 1) * kVRow + 8 * a) = hi;
    }
    if (part == 1) {
      const int t = tid >> 3, rb = kDV / 8 + (tid & 7);
      *(uint4 *)(kb + t * kKRow + 16 * rb) = keep_if(rr, attended(pos0 + t));
    }
  };

  floatx4 acc[kHB][kDV / 16];
  float m[kHB], l[kHB], seen[kHB];  // reference max, sum, largest score seen (log2 units)
#pragma unroll
  for (int hb = 0; hb < kHB; hb++) {
    m[hb] = -INFINITY;
    seen[hb] = -INFINITY;
  }
  __shared__ int overflow;
  if (tid == 0) overflow = 0;
  // one pass over the block's chunks with reference m (fixed per head once set)
  auto run_pass = [&]() {
#pragma unroll
    for (int hb = 0; hb < kHB; hb++) {
      l[hb] = 0.f;
#pragma unroll
      for (int d = 0; d < kDV / 16; d++) acc[hb][d] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    if (nchunks > 0) {
      load_part(0, 0);
      store_part(0, 0, 0);
      load_part(0, 1);
      store_part(0, 0, 1);
    }
    __syncthreads();
    for (int c = 0; c < nchunks; c++) {
      const int buf = c & 1;
      const bool more = c + 1 < nchunks;
      if (more) load_part(c + 1, 0);
      const char *kb = lds + (size_t)buf * kBufBytes;
      const char *vb = kb + kKBytes;
      const int pos0 = chunks[c].y;

      // S^T: token 16 tb + 4 kg + r of column n, head block hb
      floatx4 s[2][kHB];
#pragma unroll
      for (int tb = 0; tb < 2; tb++) {
#pragma unroll
        for (int hb = 0; hb < kHB; hb++) s[tb][hb] = floatx4{0.f, 0.f, 0.f, 0.f};
        const char *kr = kb + (16 * tb + n) * kKRow + 16 * kg;
#pragma unroll
        for (int i = 0; i < kD / 32; i++) {
          const uint4 a = *(const uint4 *)(kr + 64 * i);
#pragma unroll
          for (int hb = 0; hb < kHB; hb++) s[tb][hb] = mfma16x16x32(a, qB[hb][i], s[tb][hb]);
        }
      }

      if (more) {
        store_part(c + 1, buf ^ 1, 0);
        load_part(c + 1, 1);
      }

      // softmax weights against the reference max; P^T hi / lo as the B operand
      uint4 phi[kHB], plo[kHB];
      bool over = false;
#pragma unroll
      for (int hb = 0; hb < kHB; hb++) {
        float sv[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; tb++)
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const bool ok = attended(pos0 + 16 * tb + 4 * kg + r);
            sv[tb][r] = ok ? s[tb][hb][r] * scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, sv[tb][r]);
          }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
        seen[hb] = fmaxf(seen[hb], tmax);
        if (m[hb] == -INFINITY) m[hb] = tmax;  // first attended chunk: nothing accumulated yet
        over |= tmax > m[hb] + kHeadroom;
        float p[2][4], pl[2][4];
        float psum = 0.f;
#pragma unroll
        for (int tb = 0; tb < 2; tb++)
#pragma unroll
          for (int r = 0; r < 4; r++) {
            p[tb][r] = sv[tb][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[tb][r] - m[hb]);
            psum += p[tb][r];
            pl[tb][r] = p[tb][r] - bf16_round(p[tb][r]);
          }
        psum += __shfl_xor(psum, 16, kWave);
        psum += __shfl_xor(psum, 32, kWave);
        l[hb] += psum;
        phi[hb] = pack_bf16x8(p[0], p[1]);
        plo[hb] = pack_bf16x8(pl[0], pl[1]);
      }
      if (__any(over) && lane == 0) overflow = 1;

      // O^T += V^T P^T: A = channels 16 d + n, tokens 4kg..4kg+3 and 16+4kg..16+4kg+3
#pragma unroll
      for (int d = 0; d < kDV / 16; d++) {
        const char *vr = vb + (16 * d + n) * kVRow + 8 * kg;
        const uint2 x0 = *(const uint2 *)vr, x1 = *(const uint2 *)(vr + 32);
        const uint4 a = make_uint4(x0.x, x0.y, x1.x, x1.y);
#pragma unroll
        for (int hb = 0; hb < kHB; hb++) {
          acc[hb][d] = mfma16x16x32(a, phi[hb], acc[hb][d]);
          acc[hb][d] = mfma16x16x32(a, plo[hb], acc[hb][d]);
        }
      }

      if (more) store_part(c + 1, buf ^ 1, 1);
      __syncthreads();
    }
  };
  run_pass();
  if (overflow) {  // some weight could exceed 2^kHeadroom: again, from the largest score seen
#pragma unroll
    for (int hb = 0; hb < kHB; hb++) m[hb] = seen[hb];
    run_pass();
  }

  // lane (n, kg) holds O^T rows 16 d + 4 kg + r of head column n
#pragma unroll
  for (int hb = 0; hb < kHB; hb++) {
    const size_t row = head0 + 16 * hb + n;
    if (splits == 1) {
      const float inv = l[hb] > 0.f ? 1.f / l[hb] : 0.f;
#pragma unroll
      for (int d = 0; d < kDV / 16; d++)
        *(float4 *)(out + row * kDV + 16 * d + 4 * kg) =
            make_float4(acc[hb][d][0] * inv, acc[hb][d][1] * inv, acc[hb][d][2] * inv, acc[hb][d][3] * inv);
    } else {
      const size_t ps_idx = row * splits + split;
#pragma unroll
      for (int d = 0; d < kDV / 16; d++)
        *(float4 *)(partial + ps_idx * kDV + 16 * d + 4 * kg) =
            make_float4(acc[hb][d][0], acc[hb][d][1], acc[hb][d][2], acc[hb][d][3]);
      if (kg == 0) partial_ml[ps_idx] = make_float2(m[hb], l[hb]);
    }
  }
}

hipError_t launch_decode_mla(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                             const uint16_t *q, const uint16_t *k_pool, const int32_t *sel,
                             const int32_t *sel_count, int max_sel, float scale, float *out,
                             const Workspace &ws, hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const size_t lds = 2 * (size_t)kBufBytes;
  hipError_t e = hipFuncSetAttribute((const void *)decode_mla_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid(ws.splits, lay.num_kv_heads, bat.batch);
  hipLaunchKernelGGL(decode_mla_kernel, grid, dim3(kThreads), lds, stream, q, k_pool, bat.page_table,
                     bat.seq_lens, sel, sel_count, ws.partial, ws.partial_ml, out, bat.pt_stride, max_sel,
                     bat.num_q_heads, lay.num_kv_heads, ws.splits, scale_log2, pol.sink_tokens,
                     pol.window_tokens, pol.static_head_mask);
  e = hipGetLastError();
  if (e != hipSuccess || ws.splits == 1) return e;
  return launch_merge_splits(ws, bat.batch, bat.num_q_heads, kDV, out, stream);
}

}  // namespace qasp
