// score_pages for latent (MLA) heads: 128 query heads over one 576-channel
// latent KV head, pages of 64 tokens.
//
// The page bound is the one of score_core.h, U_h(j) = q_h^- . lo_j + q_h^+ .
// hi_j, here a real contraction: 128 heads x 1152 channels against every
// page.  A block of 8 waves stages the summary records of 16 pages in LDS and
// each wave contracts its 16 heads ([q^-, q^+] formed from q on the fly as
// the MFMA A operand, 36 steps of 16x16x32) against them, all in fp32.  The
// two MFMAs of a channel block are chained (the q^+ . hi product accumulates
// onto the q^- . lo result), three such pairs are summed per chunk and the
// six chunk sums in order.  Every bf16 product is exact, and each one passes
// through at most 63 roundings inside its pair (any order of its 64
// additions), 2 in its chunk and 5 across the chunks, each of unit 2^-23 on
// a partial sum bounded by S, so
//     |U_fp32 - U| <= 70 * 2^-23 * 1.01 * S + 2^-50.
// S comes from Cauchy-Schwarz instead of a second contraction on absolute
// values:
//     S_h(j) = sum_d |q_hd| |x_hd| <= |q_h|_2 * N_j,  N_j^2 = sum_d max(lo_d^2, hi_d^2)
// (times 1.01 for the fp32 evaluation of the norms).
// A block takes up to kMlaGroups consecutive 16-page groups of one sequence
// and stages their summary records in one LDS slab per group, through
// registers (16 bytes per lane and load): two groups are in flight while the
// one before them is contracted.  Chunk c (16 bytes) of page row n sits at
// slot c ^ (n % 16) of the row, so the 16 rows of an MFMA B fragment fall on
// different banks.  Before the first group, the slabs carry the sequence's q
// (loaded coalesced) into the MFMA layout.  The block also writes the row's
// non-candidate slots (-inf), so the score row needs no separate fill.
#include "launch.h"
#include "score_core.h"

namespace qasp {

namespace {

constexpr int kMlaD = 576;
constexpr int kMlaK2 = 2 * kMlaD;             // 1152 channels of [lo, hi]
constexpr int kMlaWaves = 8;                  // 8 x 16 = 128 heads
constexpr int kRecBytes = kMlaK2 * 2;         // LDS row of one page record (chunks swizzled)
constexpr int kGroupBytes = 16 * kRecBytes;
constexpr int kMlaGroups = 4;                 // 16-page groups per block (4 slabs: 144 KiB of LDS)
constexpr int kMlaChunk = 6;                  // MFMA results per chunk (three chained pairs)
constexpr float kErrRelMla = 70.0f * 1.1920928955078125e-07f * 1.01f;  // see the file comment

struct MlaScoreShared {
  float best[kMlaGroups][kMlaWaves][16];    // per group, wave and page: largest head value,
  float second[kMlaGroups][kMlaWaves][16];  // the runner-up,
  int arg[kMlaGroups][kMlaWaves][16];        // and the leading head
  float norm2[kMlaGroups][kMlaWaves][16];    // partial page norms per wave
  float qnorm[kMlaWaves];
  int phys[kMlaGroups][16];        // physical pages of the block's groups; -1 = not a candidate
  qasp_score out[kMlaGroups][16];  // the block's scores, stored at the end
};

constexpr int kRecU4 = kMlaK2 / 8;              // 144 chunks of 16 bytes per record
constexpr int kDmaPerGroup = 16 * kRecU4 / 64;  // 36 wave-wide 1 KB loads per group
static_assert(kRecU4 % 16 == 0 && (16 * kRecU4) % 64 == 0, "swizzle and transfer granularity");


// Workgroup barrier for LDS data: waits for this wave's LDS operations, not
// for its global loads and stores (a __syncthreads also waits for those,
// which here would hold the group loads up behind q's, or every load behind
// the first block's stores).  The empty asm statements keep the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // vmcnt and expcnt at their maximum, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Negative and non-negative parts of four bf16 pairs: an arithmetic shift of
// each 16-bit half by 15 gives its sign mask (one packed instruction), so
// neg = x & mask, pos = x ^ neg.
__device__ __forceinline__ void split_signs(const uint4 &x, uint4 &neg, uint4 &pos) {
  typedef short short2v __attribute__((ext_vector_type(2)));
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t n4[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const uint32_t m = __builtin_bit_cast(uint32_t, __builtin_bit_cast(short2v, w[k]) >> (short)15);
    n4[k] = w[k] & m;
  }
  neg = make_uint4(n4[0], n4[1], n4[2], n4[3]);
  pos = make_uint4(x.x ^ n4[0], x.y ^ n4[1], x.z ^ n4[2], x.w ^ n4[3]);
}

// LDS byte offset of chunk c of row n inside a slab
__device__ __forceinline__ int slab_off(int n, int c) { return n * kRecBytes + 16 * (c ^ (n & 15)); }

// Merges the top two (b1 >= b2, leader a1) with another top two.
__device__ __forceinline__ void top2_merge(float &b1, float &b2, int &a1, float ob1, float ob2, int oa) {
  if (ob1 > b1) {
    b2 = fmaxf(b1, ob2);
    b1 = ob1;
    a1 = oa;
  } else {
    b2 = fmaxf(b2, ob1);
  }
}

}  // namespace

__global__ __launch_bounds__(kMlaWaves * 64) void score_mla_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ summ,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    qasp_score *__restrict__ scores, int batch, int pt_stride, int max_pages, int Hq, int Hkv, int ps,
    int n_sink, int n_local, uint64_t static_mask, int groups_per_seq, TokenAppend ap) {
  // the four group slabs, one after the other (also q's way into the MFMA layout)
  __shared__ uint4 slabs[kMlaGroups * kGroupBytes / 16];
  static_assert(kMlaGroups == 4, "four slabs: two loading while two are contracted");
  __shared__ MlaScoreShared sh;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane & 15, kg = lane >> 4;
  const int g = 0;  // one latent KV head
  const int blocks_per_seq = (groups_per_seq + kMlaGroups - 1) / kMlaGroups;
  // the blocks of a sequence run on one XCD, which then reads its q once into L2
  const int item = xcd_contiguous_item(blockIdx.x, gridDim.x);
  const int b = item / blocks_per_seq;
  if (b >= batch) return;
  const int gfirst = (item % blocks_per_seq) * kMlaGroups;
  const int ng = min(kMlaGroups, groups_per_seq - gfirst);
  // the page-table entries of the block's groups are read together with the
  // length (assuming the usual cand_lo = n_sink; re-read if it is not)
  int pv = -1;
  {
    const int j = n_sink + gfirst * 16 + tid;
    if (tid < 16 * kMlaGroups && j < max_pages) pv = page_table[(size_t)b * pt_stride + j];
  }
  // q of the sequence's 128 heads (144 KB), loaded with the page-table
  // entries, coalesced: chunk c = tid + 512 k (16 bytes) of the heads'
  // contiguous rows.  It reaches the MFMA layout through LDS below (loading
  // that layout straight from memory touches 16 head rows per load and is
  // several us slower).
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // (a plain vector: arrays stay in registers)
  constexpr int kQChunks = kMlaWaves * 16 * kMlaD / 8;  // 9216
  static_assert(kQChunks % (kMlaWaves * 64) == 0 && kQChunks * 16 == kMlaGroups * kGroupBytes,
                "q fills the four slabs exactly");
  constexpr int kQLoads = kQChunks / (kMlaWaves * 64);  // 18
  u32x4 qc[kQLoads];
  {
    const uint16_t *qb = q + (size_t)b * Hq * kMlaD;
#pragma unroll
    for (int k = 0; k < kQLoads; k++) qc[k] = *(const u32x4 *)(qb + 8 * (tid + kMlaWaves * 64 * k));
  }
  const int L = seq_lens[b];
  const int P = num_pages_of(L, ps);
  const int cand_lo = min(n_sink, P);
  const int cand_hi = head_is_static(static_mask, g) ? cand_lo : max(cand_lo, P - n_local);
  qasp_score *row = scores + ((size_t)b * Hkv + g) * max_pages;
  const qasp_score none = {-INFINITY, 0.f, -1, 0};
  // the step's token (page L-1 is not a candidate here), by the row's first block
  if (ap.k_new != nullptr && gfirst == 0 && L > 0)
    ap.run(b, g, g + 1, page_table[(size_t)b * pt_stride + (L - 1) / ps], (L - 1) % ps, tid, kMlaWaves * 64);
  if (gfirst == 0) {  // the row's slots outside the candidates: sink pages, local pages, past the sequence
    for (int j = tid; j < cand_lo && j < max_pages; j += kMlaWaves * 64) row[j] = none;
    for (int j = cand_hi + tid; j < max_pages; j += kMlaWaves * 64) row[j] = none;
  }

  // physical pages of the block's groups (page j0 + 16 x + t of group x)
  const int j0 = cand_lo + gfirst * 16;
  if (tid < 16 * kMlaGroups) {
    const int x = tid / 16, j = j0 + tid;
    const bool cand = x < ng && j < cand_hi;
    if (cand_lo != n_sink) {  // short sequence: re-read (block-uniform; apart, so the usual path waits only for pv)
      const int pv2 = j < max_pages ? page_table[(size_t)b * pt_stride + j] : -1;
      sh.phys[x][tid % 16] = cand ? pv2 : -1;
    } else {
      sh.phys[x][tid % 16] = cand ? pv : -1;
    }
  }
  lds_barrier();  // sh.phys is complete

  // every record of group x, straight to its slab: transfer t fills slots
  // 64 t .. 64 t + 63 (row slot / 144), lane l loading the chunk whose
  // swizzled slot is 64 t + l; rows past the candidates read page 0 (their
  // columns are never stored)
  auto slab_of = [&](int x) -> char * { return (char *)slabs + x * kGroupBytes; };
  // the records of group x reach its slab through registers: load k of this
  // wave (t = wave + 8 k < 36) fills slots 64 t .. 64 t + 63, lane l loading
  // the chunk whose swizzled slot is 64 t + l.  (Loads straight into LDS
  // would make the compiler wait for every one still in flight before any LDS
  // read, so no group could be contracted while the next one loads.)
  constexpr int kLdPerWave = (kDmaPerGroup + kMlaWaves - 1) / kMlaWaves;
  // (every wave issues kLdPerWave loads: a load past the 36 of a group
  // repeats the group's last one and is not stored)
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // (a plain vector: the arrays stay in registers)
  auto load_group = [&](int x, u32x4 (&st)[kLdPerWave]) __attribute__((always_inline)) {
    int ph[kLdPerWave];  // the page ids are read from LDS before any load is issued
#pragma unroll
    for (int k = 0; k < kLdPerWave; k++) {
      const int t = min(wave + kMlaWaves * k, kDmaPerGroup - 1);
      ph[k] = max(sh.phys[x][(64 * t + lane) / kRecU4], 0);
    }
#pragma unroll
    for (int k = 0; k < kLdPerWave; k++) {
      const int t = min(wave + kMlaWaves * k, kDmaPerGroup - 1);
      const int slot = 64 * t + lane, r = slot / kRecU4, sl = slot % kRecU4;
      st[k] = *(const u32x4 *)(summ + summ_record(ph[k], g, Hkv) * kMlaK2 + 8 * (sl ^ (r & 15)));
    }
  };
  auto store_group = [&](int x, const u32x4 (&st)[kLdPerWave]) __attribute__((always_inline)) {
    char *slab = slab_of(x);
#pragma unroll
    for (int k = 0; k < kLdPerWave; k++) {
      const int t = wave + kMlaWaves * k;
      if (t < kDmaPerGroup) *(u32x4 *)(slab + 1024 * t + 16 * lane) = st[k];
    }
  };
  // two groups in flight: A holds groups 0 and 2, B groups 1 and 3.  Groups
  // past the block's (sh.phys -1) load page 0's record, never used, so that
  // the loads do not depend on ng.
  u32x4 stA[kLdPerWave], stB[kLdPerWave];
  load_group(0, stA);
  load_group(1, stB);

  // q into the MFMA layout: chunk c (head c / 72, piece p = c % 72) goes to
  // row c / 72 of the slab area at position p ^ (head % 8), so that the 8
  // rows of a wave's b128 reads fall on different banks; the wave then reads
  // q of its 16 heads, column n = head 16 wave + n, channels 32i + 8kg ..
  // (piece 4i + kg).  The slabs are free until group 0 is stored.
#pragma unroll
  for (int k = 0; k < kQLoads; k++) {
    const int c = tid + kMlaWaves * 64 * k, h = c / (kMlaD / 8), pc = c % (kMlaD / 8);
    *(u32x4 *)((char *)slabs + h * (2 * kMlaD) + 16 * (pc ^ (h & 7))) = qc[k];
  }
  lds_barrier();
  uint4 qraw[kMlaD / 32];
  {
    // piece 4i + kg of row 16 wave + n sits at 4 (i ^ (s >> 2)) + (kg ^ (s & 3)), s = n % 8
    const int sq = n & 7;
    const char *qrow = (const char *)slabs + (16 * wave + n) * (2 * kMlaD) + 16 * (kg ^ (sq & 3));
#pragma unroll
    for (int i = 0; i < kMlaD / 32; i++) qraw[i] = *(const uint4 *)(qrow + 64 * (i ^ (sq >> 2)));
  }
  lds_barrier();  // the slabs take the groups next

  // the largest |q_h| of the wave's heads
  {
    float s2 = 0.f;  // |q_h|^2 of head n over this lane's quarter of the channels
#pragma unroll
    for (int i = 0; i < kMlaD / 32; i++) {
      const uint32_t w4[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const float a = bf16_lo_to_f32(w4[k]), c = bf16_hi_to_f32(w4[k]);
        s2 += a * a + c * c;
      }
    }
    s2 += __shfl_xor(s2, 16, kWave);
    s2 += __shfl_xor(s2, 32, kWave);
    const float qmax = wave_max(sqrtf(s2));
    if (lane == 0) sh.qnorm[wave] = qmax;
  }

  // contracts group x: every wave's top two heads and partial norm per page
  auto contract = [&](int x) {
    const char *rec = slab_of(x);
    // page norms N_j^2 = sum_d max(lo_d^2, hi_d^2): wave w adds channel blocks
    // 32i + 8kg .. (i = w, w + 8, ...) of page n; the blocks sum in LDS below
    {
      float a = 0.f;
      for (int i = wave; i < kMlaD / 32; i += kMlaWaves) {
        const uint4 lo4 = *(const uint4 *)(rec + slab_off(n, 4 * i + kg));
        const uint4 hi4 = *(const uint4 *)(rec + slab_off(n, kMlaD / 8 + 4 * i + kg));
        const uint32_t lw[4] = {lo4.x, lo4.y, lo4.z, lo4.w}, hw[4] = {hi4.x, hi4.y, hi4.z, hi4.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const float l0 = bf16_lo_to_f32(lw[k]), l1 = bf16_hi_to_f32(lw[k]);
          const float h0 = bf16_lo_to_f32(hw[k]), h1 = bf16_hi_to_f32(hw[k]);
          a += fmaxf(l0 * l0, h0 * h0) + fmaxf(l1 * l1, h1 * h1);
        }
      }
      a += __shfl_xor(a, 16, kWave);
      a += __shfl_xor(a, 32, kWave);
      if (kg == 0) sh.norm2[x][wave][n] = a;
    }
    // contraction over [lo, hi]: q^- with lo channels 32i + 8kg ... and q^+
    // with the same hi channels, for i = 0 .. 17.  The fragments of three
    // channel blocks (one fp32 chunk of kMlaChunk MFMA results) are read from
    // LDS together, one chunk ahead of the MFMAs that use them.
    static_assert(kMlaChunk == 6 && (kMlaD / 32) % 3 == 0, "three channel blocks per fp32 chunk");
    constexpr int kChunks = kMlaD / 32 / 3;
    float u[4] = {0.f, 0.f, 0.f, 0.f};
    uint4 fl[2][3], fh[2][3];  // [buffer][block in chunk]: lo and hi fragments
    // chunk 4i + kg of row n is at frag_base[i % 4] + 256 (i / 4), hi chunk
    // 72 + 4i + kg at frag_base[(i + 2) % 4] + 256 (4 + (i + 2) / 4): four
    // per-lane bases, the rest immediate offsets
    static_assert(kMlaD / 8 == 72, "hi half starts at chunk 72");
    int frag_base[4];
#pragma unroll
    for (int m = 0; m < 4; m++) frag_base[m] = slab_off(n, 4 * m + kg);
    auto read_chunk = [&](int c, uint4 *l, uint4 *h) {
#pragma unroll
      for (int j = 0; j < 3; j++) {
        const int i = 3 * c + j;
        l[j] = *(const uint4 *)(rec + frag_base[i & 3] + 256 * (i >> 2));
        h[j] = *(const uint4 *)(rec + frag_base[(i + 2) & 3] + 256 * (4 + ((i + 2) >> 2)));
      }
    };
    read_chunk(0, fl[0], fh[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < kChunks; c++) {
      if (c + 1 < kChunks) read_chunk(c + 1, fl[(c + 1) & 1], fh[(c + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of this chunk's MFMAs
      floatx4 part;
#pragma unroll
      for (int j = 0; j < 3; j++) {
        const int i = 3 * c + j;
        uint4 qn, qp;  // q^- and q^+ (the rest of q's bits) of channel block i
        split_signs(qraw[i], qn, qp);
        const floatx4 t = mfma16x16x32(qp, fh[c & 1][j], mfma16x16x32(qn, fl[c & 1][j], floatx4{0.f, 0.f, 0.f, 0.f}));
        if (j == 0) {
          part = t;
        } else {
#pragma unroll
          for (int r = 0; r < 4; r++) part[r] += t[r];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; r++) u[r] = c == 0 ? part[r] : u[r] + part[r];
    }
    // lane (n, kg) holds heads 16 wave + 4kg + r of page n: top two of the
    // wave's heads for page n (value, runner-up, leading head)
    float b1 = -INFINITY, b2 = -INFINITY;
    int a1 = -1;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      if (u[r] > b1) {
        b2 = b1;
        b1 = u[r];
        a1 = 16 * wave + 4 * kg + r;
      } else {
        b2 = fmaxf(b2, u[r]);
      }
    }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float ob1 = __shfl_xor(b1, o, kWave), ob2 = __shfl_xor(b2, o, kWave);
      const int oa = __shfl_xor(a1, o, kWave);
      top2_merge(b1, b2, a1, ob1, ob2, oa);
    }
    if (kg == 0) {
      sh.best[x][wave][n] = b1;
      sh.second[x][wave][n] = b2;
      sh.arg[x][wave][n] = a1;
    }
  };
  // combines the waves' results of group x into its 16 scores (wave fw)
  auto finish = [&](int x, int fw) {
    if (wave == fw && lane < 16 && j0 + 16 * x + lane < cand_hi) {
      float m = sh.best[x][0][lane], m2 = sh.second[x][0][lane];
      int arg = sh.arg[x][0][lane];
      float qn = sh.qnorm[0], n2 = sh.norm2[x][0][lane];
#pragma unroll
      for (int w = 1; w < kMlaWaves; w++) {
        top2_merge(m, m2, arg, sh.best[x][w][lane], sh.second[x][w][lane], sh.arg[x][w][lane]);
        qn = fmaxf(qn, sh.qnorm[w]);
        n2 += sh.norm2[x][w][lane];
      }
      const float bound = qn * sqrtf(n2) * 1.01f;  // >= every head's S
      sh.out[x][lane] = score::make_score(m, bound, m2, arg, kErrRelMla);
    }
  };
  // group x goes to LDS once its loads have landed (the compiler waits for
  // exactly those registers), then group x + 2 loads into the same registers
  // and group x is contracted while x + 1 and x + 2 load
  store_group(0, stA);
  lds_barrier();
  load_group(2, stA);
  if (ng > 0) contract(0);
  store_group(1, stB);
  lds_barrier();
  load_group(3, stB);
  if (ng > 1) contract(1);
  store_group(2, stA);
  lds_barrier();
  if (ng > 2) contract(2);
  store_group(3, stB);
  lds_barrier();
  if (ng > 3) contract(3);
  lds_barrier();  // every wave's results of every group are in LDS
  if (wave < ng) finish(wave, wave);
  lds_barrier();
  for (int t = tid; t < 16 * ng; t += kMlaWaves * 64) {
    const int j = j0 + t;
    if (j < cand_hi) row[j] = sh.out[t / 16][t % 16];
  }
}

hipError_t launch_score_mla(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                            const uint16_t *q, const uint16_t *summ, qasp_score *scores, hipStream_t stream,
                            const TokenAppend &ap) {
  if (bat.batch == 0 || bat.max_pages == 0) return hipSuccess;
  // groups cover [cand_lo, cand_lo + 16 groups_per_seq), which holds every
  // candidate: cand_hi - cand_lo <= max_pages - n_sink - n_local when there are any
  const int max_cand = std::max(0, bat.max_pages - pol.n_sink_pages - pol.n_local_pages);
  const int groups_per_seq = std::max(1, (max_cand + 15) / 16);
  const int blocks_per_seq = (groups_per_seq + kMlaGroups - 1) / kMlaGroups;
  const int blocks = bat.batch * blocks_per_seq;
  hipLaunchKernelGGL(score_mla_kernel, dim3(blocks), dim3(kMlaWaves * 64), 0, stream, q,
                     summ, bat.page_table, bat.seq_lens, scores, bat.batch, bat.pt_stride, bat.max_pages,
                     bat.num_q_heads, lay.num_kv_heads, lay.page_size, pol.n_sink_pages, pol.n_local_pages,
                     pol.static_head_mask, groups_per_seq, ap);
  return hipGetLastError();
}

}  // namespace qasp
