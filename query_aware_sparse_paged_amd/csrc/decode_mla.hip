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
// page (64 tokens x 1152 bytes) goes from HBM straight into LDS
// (global_load_lds, 16 bytes per lane, 73 wave-wide transfers of 1 KiB),
// token-major with rows padded to 73 pieces of 16 bytes so the 16 rows of an
// A fragment fall on different banks (the pad piece of a row receives a copy
// of its last piece, never read).  Two page buffers, each an LDS object of
// its own so the compiler sees which transfers a read depends on: page c + 1
// loads into the buffer page c - 1 used while page c is computed.  Per page,
// wave w:
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
// The rows of tokens that are not attended (past the length, outside a
// static head's sink and window) are written as zeros instead of loaded, so
// stale pool or LDS contents never reach the products, and get weight 0.
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
#include "select_core.h"

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
constexpr int kRowSlots = kKRow / 16;            // 73 slots per LDS row (the last one padding)
constexpr int kXfer = kBufBytes / 1024;          // 73 wave-wide transfers per page
constexpr int kXferPerWave = (kXfer + kWaves - 1) / kWaves;  // 10 for wave 0, 9 for the others
static_assert(kXfer == kWaves * (kXferPerWave - 1) + 1, "one more transfer for wave 0 than for the others");
constexpr int kPRow = kPS * 2 + 16;              // bytes per P^T row (one head, padded): 144
constexpr int kPBytes = kHeads * kPRow;          // 4608 per part (hi, lo)
constexpr float kHeadroom = 64.f;                // weights stay below 2^64 (log2 units)
static_assert(kXfer * 1024 == kBufBytes && kRowSlots == kRowU4 + 1, "whole transfers per page buffer");
static_assert(kBufBytes % 16 == 0 && kKRow % 16 == 0 && kPRow % 16 == 0, "LDS alignment");
static_assert(kMlaPagesPerSplit <= 16, "page list");
constexpr int kQChunks = kHeads * kD / 8;        // 16-byte chunks of the block's q rows: 2304
constexpr int kQLoads = (kQChunks + kThreads - 1) / kThreads;  // 5 per lane (the last for half the lanes)
constexpr int kQRow = kD * 2 + 16;               // LDS row of one head's q (padded: conflict-free reads)
static_assert(kHeads * kQRow <= kBufBytes && kRowU4 == kD / 8, "q staging fits the second page buffer");

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

typedef __attribute__((address_space(3))) void lds_void;

// Waits until at most N (< 16) of this wave's vector memory operations are
// outstanding.  The empty asm statements keep the compiler from moving
// memory accesses across it.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(N | (7 << 4) | (15 << 8));  // vmcnt N, expcnt and lgkmcnt at their maximum
  asm volatile("" ::: "memory");
}

// Workgroup barrier after this wave's LDS operations (not its transfers into
// LDS still in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // vmcnt and expcnt at their maximum, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Transposing 8-byte LDS read (see the file comment for its lane layout).
__device__ __forceinline__ uint2 lds_read_tr16(const char *p) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)p);
  return __builtin_bit_cast(uint2, v);
}

}  // namespace

// SELECT: the block first selects its unit's pages from the stored scores
// (select_unit, as select_topk_kernel does: every block of a unit computes
// the same list, the first one also writes it to sel / sel_count), with the
// selection's LDS laid over the first page buffer, which is not in use yet.
// Otherwise sel / sel_count are read.
template <bool SELECT>
__global__ __launch_bounds__(kThreads) void decode_mla_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_pool, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, int32_t *__restrict__ sel, int32_t *__restrict__ sel_count,
    float *__restrict__ partial, float2 *__restrict__ partial_ml, float *__restrict__ out, int pt_stride,
    int max_sel, int Hq, int Hkv, int splits, float scale_log2, int sink_tokens, int window_tokens,
    uint64_t static_mask, const qasp_score *__restrict__ scores, const uint16_t *__restrict__ summ, int max_pages,
    int n_sink, int n_local, int top_k) {
  // the two page buffers are LDS objects of their own (see the file comment)
  __shared__ uint4 kbuf0[kBufBytes / 16], kbuf1[kBufBytes / 16];
  __shared__ uint4 pbuf_u4[2 * kPBytes / 16];
  __shared__ MlaDecodeShared sh;
  char *kvbuf = (char *)kbuf0;     // the selection's LDS, before the pages
  char *pbuf = (char *)pbuf_u4;    // P^T hi, then lo
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

  const size_t head_base = (size_t)b * Hq + (size_t)g * kG + kHeads * hg;
  // q of the block's 32 heads (36 KB) is loaded coalesced, 16 bytes per lane
  // and load (chunk c = tid + 512 k of the heads' contiguous rows), then goes
  // through LDS (rows padded to kQRow bytes) into the MFMA layout: q^T of the
  // wave's S heads, column n = head 32 hg + 16 ht + n, channels 32i + 8kg ..
  // (Loading that layout straight from memory touches 16 rows per load and
  // took ~3 us longer.)  With the selection, the loads are issued right after
  // its score loads (loads complete in order: q first would hold them up).
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // (a plain vector: the array stays in registers)
  u32x4 qs[kQLoads];
  auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kQLoads; k++) {
      const int c = tid + kThreads * k;
      qs[k] = *(const u32x4 *)(q + head_base * kD + 8 * min(c, kQChunks - 1));
    }
  };
  if constexpr (!SELECT) load_q();

  // the block's pages that hold an attended position
  const int32_t *list = sel + (size_t)unit * max_sel;
  int count = 0;
  if constexpr (SELECT) {
    // the selection's LDS over the first page buffer: shared state, keys, bit maps, list
    using Shared = sel::SelShared<kWaves>;
    Shared &ssh = *(Shared *)kvbuf;
    uint64_t *keys = (uint64_t *)(kvbuf + ((sizeof(Shared) + 15) & ~(size_t)15));
    uint32_t *bits = (uint32_t *)(keys + max_pages);
    int32_t *lds_list = (int32_t *)(bits + 2 * ((max_pages + 31) / 32));
    const bool first_block = hg == 0 && split == 0;
    count = sel::select_unit<kD, kWaves>(ssh, keys, bits, (max_pages + 31) / 32, scores + (size_t)unit * max_pages, L,
                                         kPS, is_static, n_sink, n_local, top_k, sink_tokens, window_tokens,
                                         q + ((size_t)b * Hq + (size_t)g * kG) * kD, kG, summ,
                                         page_table + (size_t)b * pt_stride, Hkv, g,
                                         first_block ? sel + (size_t)unit * max_sel : nullptr, lds_list, max_sel,
                                         load_q);
    if (first_block && tid == 0) sel_count[unit] = count;
    __syncthreads();  // the list is complete
    list = lds_list;
  }
  // wave 0: lane i takes the block's i-th page of the list
  if (wave == 0) {
    if constexpr (!SELECT) count = sel_count[unit];
    const int first = split * kMlaPagesPerSplit, last = min(first + kMlaPagesPerSplit, count);
    const int p = first + lane;
    bool keep = false;
    int2 pg = make_int2(0, 0);
    if (lane < kMlaPagesPerSplit && p < last) {
      const int j = list[p];
      const int pos0 = j * kPS, pos1 = min(pos0 + kPS, L);
      keep = pos0 < pos1 && (!is_static || pos0 < sink_end || pos1 > win_begin);
      if (keep) pg = make_int2(page_table[(size_t)b * pt_stride + j], pos0);
    }
    const uint64_t kept = __ballot(keep);
    if (keep) sh.pages[__popcll(kept & ((1ull << lane) - 1))] = pg;
    if (lane == 0) {
      sh.npages = __popcll(kept);
      sh.overflow = 0;
    }
  }

  // q into the MFMA layout through the second page buffer (free until the
  // page loop starts; the selection's LDS lies in the first)
  {
    char *qstage = (char *)kbuf1;
#pragma unroll
    for (int k = 0; k < kQLoads; k++) {
      const int c = tid + kThreads * k;
      if (c < kQChunks) *(u32x4 *)(qstage + (c / kRowU4) * kQRow + 16 * (c % kRowU4)) = qs[k];
    }
  }
  __syncthreads();
  uint4 qB[kD / 32];
#pragma unroll
  for (int i = 0; i < kD / 32; i++)
    qB[i] = *(const uint4 *)((const char *)kbuf1 + (16 * ht + n) * kQRow + 64 * i + 16 * kg);
  // q is in registers before the page loop (which then reuses kbuf1), and
  // every load has landed: otherwise the loop's first products carry waits
  // that the in-order load counter turns into waits for page loads
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int npages = sh.npages;

  // transfer k of this wave (t = wave + 8 k < kXfer) fills slots 64 t .. 64 t
  // + 63 of a page buffer; lane l's slot e = 64 t + l is piece e % 73 of LDS
  // row e / 73, which receives the same piece of token row e / 73 (the pad
  // piece a copy of piece 71)
  int xrow[kXferPerWave], xsrc[kXferPerWave];
#pragma unroll
  for (int k = 0; k < kXferPerWave; k++) {
    const int e = 64 * (wave + kWaves * k) + lane, r = e / kRowSlots, cb = e % kRowSlots;
    xrow[k] = r;
    xsrc[k] = r * kD + 8 * min(cb, kRowU4 - 1);
  }
  // page c into buffer kb: every transfer is issued, so the wave's count of
  // outstanding transfers per page is fixed
  auto issue_page = [&](int c, char *kb) __attribute__((always_inline)) {
    const uint16_t *base = k_pool + ((size_t)sh.pages[c].x * Hkv + g) * kPS * kD;
#pragma unroll
    for (int k = 0; k < kXferPerWave; k++) {
      const int t = wave + kWaves * k;  // wave-uniform
      if (t < kXfer)
        __builtin_amdgcn_global_load_lds((const void *)(base + xsrc[k]), (lds_void *)(kb + 1024 * t), 16, 0, 0);
    }
  };
  // once this wave's transfers of page c have landed: zeros over the rows of
  // the tokens it does not attend (slots this lane's transfers wrote)
  auto zero_rows = [&](int c, char *kb) __attribute__((always_inline)) {
    const int pos0 = sh.pages[c].y;
    const bool whole = pos0 + kPS <= L && (!is_static || pos0 + kPS <= sink_end || pos0 >= win_begin);
    if (!whole) {  // block-uniform
#pragma unroll
      for (int k = 0; k < kXferPerWave; k++) {
        const int t = wave + kWaves * k;
        if (t < kXfer && !attended(pos0 + xrow[k])) *(uint4 *)(kb + 1024 * t + 16 * lane) = make_uint4(0, 0, 0, 0);
      }
    }
  };
  // lane's transposing-read address inside a page buffer: token 4kg + n/4, channels 4 (n % 4) ..
  const int tr_off = (4 * kg + n / 4) * kKRow + 8 * (n % 4);
  // where this lane's 4 weights go in the P^T tile: head row 16 ht + n, token
  // slot 32 (tq / 2) + 8 kg + 4 (tq % 2) (the PV k order of the file comment)
  const int p_off = (16 * ht + n) * kPRow + 2 * (32 * (tq / 2) + 8 * kg + 4 * (tq % 2));

  floatx4 acc[4][2];  // O^T: value channel tile 4 wave + d, head tile t
  float m = -INFINITY, l = 0.f, seen = -INFINITY;  // head column n of tile ht (log2 units)
  // page c, in buffer kb (the other buffer: ob); on entry this wave has page
  // c's transfers and, for c = 0, page 1's outstanding.  (Page 0 is peeled off
  // the loop below, so the compiler's count of the transfers in flight at
  // each read is exact.)
  auto page_step = [&](int c, char *kb, char *ob) __attribute__((always_inline)) {
    const int pos0 = sh.pages[c].y;
    // this wave's transfers of page c have landed (for c = 0 page 1's may
    // still be in flight)
    if (c == 0 && npages > 1) {
      if (wave == 0) vm_wait<kXferPerWave>();
      else vm_wait<kXferPerWave - 1>();
    } else {
      vm_wait<0>();
    }
    zero_rows(c, kb);
    // page c is complete; the previous page's products are done, so ob and
    // P^T are free
    lds_barrier();
    if (c >= 1 && c + 1 < npages) issue_page(c + 1, ob);

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
    if (m == -INFINITY) {  // first page (block-uniform): the reference is its max over all 64 tokens
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));  // this quarter's max of head column n
      if (kg == 0) sh.red[tq][16 * ht + n] = tmax;
      lds_barrier();
      m = fmaxf(fmaxf(sh.red[0][16 * ht + n], sh.red[1][16 * ht + n]),
                fmaxf(sh.red[2][16 * ht + n], sh.red[3][16 * ht + n]));
    }
    // the largest score seen and the weight sum stay per lane (this lane's
    // tokens) until the loop ends
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
    l += psum;
    *(uint2 *)(pbuf + p_off) = pack_bf16x4(p);
    *(uint2 *)(pbuf + kPBytes + p_off) = pack_bf16x4(pl);
    lds_barrier();  // P^T is complete (a plain __syncthreads would also wait for page c + 1)

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
  };
  // one pass over the block's pages with reference m (fixed once set); the
  // loop is unrolled by two so that each step reads a known buffer
  auto run_pass = [&]() __attribute__((always_inline)) {
    l = 0.f;
#pragma unroll
    for (int d = 0; d < 4; d++)
#pragma unroll
      for (int t = 0; t < 2; t++) acc[d][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (npages > 0) issue_page(0, (char *)kbuf0);
    if (npages > 1) issue_page(1, (char *)kbuf1);
    if (npages > 0) page_step(0, (char *)kbuf0, (char *)kbuf1);
    for (int c = 1; c < npages; c += 2) {
      page_step(c, (char *)kbuf1, (char *)kbuf0);
      if (c + 1 < npages) page_step(c + 1, (char *)kbuf0, (char *)kbuf1);
    }
  };
  // a second pass only if some weight could exceed 2^kHeadroom, then from
  // the largest score seen (one copy of the loop body in the code)
#pragma clang loop unroll(disable)
  for (int pass = 0; pass < 2; pass++) {
    run_pass();
    __syncthreads();
    if (pass == 1 || !sh.overflow) break;
    seen = fmaxf(seen, __shfl_xor(seen, 16, kWave));
    seen = fmaxf(seen, __shfl_xor(seen, 32, kWave));
    if (kg == 0) sh.red[tq][16 * ht + n] = seen;
    __syncthreads();
    m = fmaxf(fmaxf(sh.red[0][16 * ht + n], sh.red[1][16 * ht + n]),
              fmaxf(sh.red[2][16 * ht + n], sh.red[3][16 * ht + n]));
    __syncthreads();
  }
  // the heads' sums over the four token quarters
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);
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

// LDS the selection inside decode_mla_kernel<true> needs (laid over its first page buffer).
size_t mla_select_lds_bytes(int max_pages, int max_sel) {
  return ((sizeof(sel::SelShared<kWaves>) + 15) & ~(size_t)15) + (size_t)max_pages * 8 +
         2 * (size_t)((max_pages + 31) / 32) * 4 + (size_t)max_sel * 4;
}
bool mla_select_fits(const qasp_batch &bat, int max_sel) {
  return mla_select_lds_bytes(bat.max_pages > 0 ? bat.max_pages : 1, max_sel) <= (size_t)kBufBytes;
}

// scores != nullptr: the blocks select first (sel / sel_count, then written,
// receive the selection); else sel / sel_count are the given selection.
hipError_t launch_decode_mla(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                             const uint16_t *q, const uint16_t *k_pool, const int32_t *sel,
                             const int32_t *sel_count, int max_sel, float scale, float *out,
                             const Workspace &ws, hipStream_t stream, const qasp_score *scores,
                             const uint16_t *summ) {
  const float scale_log2 = scale * 1.4426950408889634f;
  if (bat.num_q_heads != kG * lay.num_kv_heads) return hipErrorInvalidValue;
  dim3 grid((unsigned)(kG / kHeads) * ws.splits * lay.num_kv_heads * bat.batch);
  if (scores != nullptr)
    hipLaunchKernelGGL(decode_mla_kernel<true>, grid, dim3(kThreads), 0, stream, q, k_pool, bat.page_table,
                       bat.seq_lens, (int32_t *)sel, (int32_t *)sel_count, ws.partial, ws.partial_ml, out,
                       bat.pt_stride, max_sel,
                       bat.num_q_heads, lay.num_kv_heads, ws.splits, scale_log2, pol.sink_tokens,
                       pol.window_tokens, pol.static_head_mask, scores, summ, bat.max_pages > 0 ? bat.max_pages : 1,
                       pol.n_sink_pages, pol.n_local_pages, pol.top_k);
  else
    hipLaunchKernelGGL(decode_mla_kernel<false>, grid, dim3(kThreads), 0, stream, q, k_pool, bat.page_table,
                       bat.seq_lens, (int32_t *)sel, (int32_t *)sel_count, ws.partial, ws.partial_ml, out,
                       bat.pt_stride, max_sel, bat.num_q_heads, lay.num_kv_heads, ws.splits, scale_log2,
                       pol.sink_tokens, pol.window_tokens, pol.static_head_mask, nullptr, nullptr, 0, 0, 0, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ws.splits == 1) return e;
  return launch_merge_splits(ws, bat.batch, bat.num_q_heads, kDV, out, stream);
}

}  // namespace qasp
