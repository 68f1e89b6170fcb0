// score_pages for latent (MLA) heads: 128 query heads over one 576-channel
// latent KV head, pages of 64 tokens.
//
// The page bound is the one of score_core.h, U_h(j) = q_h^- . lo_j + q_h^+ .
// hi_j, here a real contraction: 128 heads x 1152 channels against every
// page.  A block of 8 waves stages the summary records of 16 pages in LDS
// (row stride padded by 16 bytes so the 16 page columns fall on different
// banks) and each wave contracts its 16 heads ([q^-, q^+] held as the MFMA A
// operand, 36 steps of 16x16x32) against them; every 32-product MFMA result
// is added in fp64.  The error bound uses Cauchy-Schwarz instead of a second
// contraction on absolute values:
//     S_h(j) = sum_d |q_hd| |x_hd| <= |q_h|_2 * N_j,  N_j^2 = sum_d max(lo_d^2, hi_d^2),
//     |U_fp32 - U| <= 65 * 2^-23 * 1.01 * max_h |q_h|_2 * N_j * 1.01 + 2^-50
// (the last 1.01 covers the fp32 evaluation of the norms).
// Blocks are persistent over the 16-page groups of the batch, in sequence
// order, with the next group's records loading while the current one is
// contracted.
#include "launch.h"
#include "score_core.h"

namespace qasp {

namespace {

constexpr int kMlaD = 576;
constexpr int kMlaK2 = 2 * kMlaD;             // 1152 channels of [lo, hi]
constexpr int kMlaSteps = kMlaK2 / 32;        // 36 MFMA steps
constexpr int kMlaWaves = 8;                  // 8 x 16 = 128 heads
constexpr int kRecBytes = kMlaK2 * 2 + 16;    // padded LDS row of one page record
constexpr int kGroupBytes = 16 * kRecBytes;

struct MlaScoreShared {
  double best[kMlaWaves][16];    // per wave and page: largest head value,
  double second[kMlaWaves][16];  // the runner-up,
  int arg[kMlaWaves][16];        // and the leading head
  float norm2[kMlaWaves][16];  // partial page norms per wave
  float qnorm[kMlaWaves];
  int phys[3][16];   // physical pages of groups gid, gid+1, gid+2 (slot gid % 3); -1 = not a candidate
};

constexpr int kRecU4 = kMlaK2 / 8;                                      // 144 uint4 per record
constexpr int kLoadsPerThread = (16 * kRecU4 + kMlaWaves * 64 - 1) / (kMlaWaves * 64);  // 5

// Merges the top two (b1 >= b2, leader a1) with another top two.
__device__ __forceinline__ void top2_merge(double &b1, double &b2, int &a1, double ob1, double ob2, int oa) {
  if (ob1 > b1) {
    b2 = fmax(b1, ob2);
    b1 = ob1;
    a1 = oa;
  } else {
    b2 = fmax(b2, ob1);
  }
}

}  // namespace

__global__ __launch_bounds__(kMlaWaves * 64) void score_mla_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ summ,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    qasp_score *__restrict__ scores, int batch, int pt_stride, int max_pages, int Hq, int Hkv, int ps,
    int n_sink, int n_local, uint64_t static_mask, int groups_per_seq, int groups_per_block) {
  extern __shared__ uint4 stage[];  // 2 x kGroupBytes
  __shared__ MlaScoreShared sh;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane & 15, kg = lane >> 4;
  const int g = 0;  // one latent KV head
  const int total = batch * groups_per_seq;
  // the blocks of a sequence run on one XCD, which then reads its q once into L2
  const int first = xcd_contiguous_item(blockIdx.x, gridDim.x) * groups_per_block;
  const int last = min(first + groups_per_block, total);
  if (first >= last) return;

  // group -> (sequence, first logical page, end of the candidates)
  auto group_pages = [&](int gid, int &b, int &j0, int &cand_hi) {
    b = gid / groups_per_seq;
    const int L = seq_lens[b];
    const int P = num_pages_of(L, ps);
    const int cand_lo = min(n_sink, P);
    cand_hi = head_is_static(static_mask, g) ? cand_lo : max(cand_lo, P - n_local);
    j0 = cand_lo + (gid % groups_per_seq) * 16;
  };
  // page-table entry of page tid (< 16) of group gid
  auto phys_of = [&](int gid) {
    if (gid >= last) return -1;
    int b, j0, cand_hi;
    group_pages(gid, b, j0, cand_hi);
    const int j = j0 + tid;
    return j < cand_hi ? page_table[(size_t)b * pt_stride + j] : -1;
  };
  // the group's 16 summary records, read into registers (5 uint4 per thread)
  auto load_regs = [&](int slot, uint4 *r) {
#pragma unroll
    for (int u = 0; u < kLoadsPerThread; u++) {
      const int e = tid + u * kMlaWaves * 64;
      const int p = e / kRecU4, c = e % kRecU4;
      const int phys = e < 16 * kRecU4 ? sh.phys[slot][p] : -1;
      r[u] = phys >= 0 ? *((const uint4 *)(summ + ((size_t)phys * Hkv + g) * kMlaK2) + c) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_regs = [&](int buf, const uint4 *r) {
    char *dst = (char *)stage + (size_t)buf * kGroupBytes;
#pragma unroll
    for (int u = 0; u < kLoadsPerThread; u++) {
      const int e = tid + u * kMlaWaves * 64;
      if (e < 16 * kRecU4) *(uint4 *)(dst + (size_t)(e / kRecU4) * kRecBytes + (e % kRecU4) * 16) = r[u];
    }
  };

  if (tid < 16) {
    sh.phys[first % 3][tid] = phys_of(first);
    sh.phys[(first + 1) % 3][tid] = phys_of(first + 1);
  }
  __syncthreads();
  uint4 regs[kLoadsPerThread];
  load_regs(first % 3, regs);
  store_regs(0, regs);

  uint4 qraw[kMlaD / 32];  // q of head 16 wave + (l % 16), channels 32i + 8(l / 16) ...
  int cur_b = -1;
  for (int gid = first; gid < last; gid++) {
    const int buf = (gid - first) & 1;
    int b, j0, cand_hi;
    group_pages(gid, b, j0, cand_hi);
    if (b != cur_b) {  // this wave's 16 heads of the sequence's query, and the largest |q_h|
      cur_b = b;
      const uint16_t *qg = q + ((size_t)b * Hq + (size_t)wave * 16) * kMlaD;
#pragma unroll
      for (int i = 0; i < kMlaD / 32; i++) qraw[i] = *(const uint4 *)(qg + (size_t)n * kMlaD + 32 * i + 8 * kg);
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
    __syncthreads();  // stage `buf` and sh.phys of gid+1 are complete
    // prefetch: page-table entries of gid+2, summary records of gid+1
    const int phys_ahead = tid < 16 ? phys_of(gid + 2) : -1;
    if (gid + 1 < last) load_regs((gid + 1) % 3, regs);
    const char *rec = (const char *)stage + (size_t)buf * kGroupBytes;
    // page norms N_j^2 = sum_d max(lo_d^2, hi_d^2): wave w adds channel blocks
    // 32i + 8kg .. (i = w, w + 8, ...) of page n; the blocks sum in LDS below
    {
      const char *rp = rec + (size_t)n * kRecBytes + 16 * kg;
      float a = 0.f;
      for (int i = wave; i < kMlaD / 32; i += kMlaWaves) {
        const uint4 lo4 = *(const uint4 *)(rp + 64 * i), hi4 = *(const uint4 *)(rp + 2 * kMlaD + 64 * i);
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
      if (kg == 0) sh.norm2[wave][n] = a;
    }
    // contraction over [lo, hi]: step i < 18 pairs q^- with lo channels
    // 32i + 8kg ..., step 18 + i pairs q^+ with the same hi channels
    double u64[4] = {0.0, 0.0, 0.0, 0.0};
    const char *bp = rec + (size_t)n * kRecBytes + 16 * kg;
#pragma unroll
    for (int i = 0; i < kMlaSteps; i++) {
      const uint4 bfrag = *(const uint4 *)(bp + 64 * i);
      const uint4 afrag = score::map4(qraw[i % (kMlaD / 32)], i < kMlaD / 32 ? 0 : 1);
      const floatx4 ui = mfma16x16x32(afrag, bfrag, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; r++) u64[r] += (double)ui[r];
    }
    // lane (n, kg) holds heads 16 wave + 4kg + r of page n: max over the wave's heads
    // top two of the wave's heads for page n: value, runner-up, leading head
    double b1 = -INFINITY, b2 = -INFINITY;
    int a1 = -1;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      if (u64[r] > b1) {
        b2 = b1;
        b1 = u64[r];
        a1 = 16 * wave + 4 * kg + r;
      } else {
        b2 = fmax(b2, u64[r]);
      }
    }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const double ob1 = __shfl_xor(b1, o, kWave), ob2 = __shfl_xor(b2, o, kWave);
      const int oa = __shfl_xor(a1, o, kWave);
      top2_merge(b1, b2, a1, ob1, ob2, oa);
    }
    if (kg == 0) {
      sh.best[wave][n] = b1;
      sh.second[wave][n] = b2;
      sh.arg[wave][n] = a1;
    }
    if (gid + 1 < last) store_regs(buf ^ 1, regs);
    if (tid < 16) sh.phys[(gid + 2) % 3][tid] = phys_ahead;
    __syncthreads();
    if (wave == 0 && lane < 16) {
      const int j = j0 + lane;
      if (j < cand_hi) {
        double m = sh.best[0][lane], m2 = sh.second[0][lane];
        int arg = sh.arg[0][lane];
        float qn = sh.qnorm[0], n2 = sh.norm2[0][lane];
#pragma unroll
        for (int w = 1; w < kMlaWaves; w++) {
          top2_merge(m, m2, arg, sh.best[w][lane], sh.second[w][lane], sh.arg[w][lane]);
          qn = fmaxf(qn, sh.qnorm[w]);
          n2 += sh.norm2[w][lane];
        }
        const float bound = qn * sqrtf(n2) * 1.01f;  // >= every head's S
        scores[((size_t)b * Hkv + g) * max_pages + j] = score::make_score(m, bound, m2, arg);
      }
    }
  }
}

// Fills every row with (-inf, 0); the candidates are overwritten by the scoring kernel.
__global__ void fill_scores_kernel(qasp_score *scores, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    scores[i] = qasp_score{-INFINITY, 0.f, -1, 0};
}

hipError_t launch_score_mla(const qasp_layout &lay, const qasp_batch &bat, const qasp_policy &pol,
                            const uint16_t *q, const uint16_t *summ, qasp_score *scores, hipStream_t stream) {
  const size_t n = (size_t)bat.batch * lay.num_kv_heads * bat.max_pages;
  size_t fill_blocks = (n + 255) / 256;
  if (fill_blocks > 2048) fill_blocks = 2048;
  hipLaunchKernelGGL(fill_scores_kernel, dim3((unsigned)fill_blocks), dim3(256), 0, stream, scores, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int groups_per_seq = (bat.max_pages + 15) / 16;
  const int total = bat.batch * groups_per_seq;
  int per_block = (total + 255) / 256;  // about one block per CU
  if (per_block < 1) per_block = 1;
  const int blocks = (total + per_block - 1) / per_block;
  hipLaunchKernelGGL(score_mla_kernel, dim3(blocks), dim3(kMlaWaves * 64), 2 * kGroupBytes, stream, q, summ,
                     bat.page_table, bat.seq_lens, scores, bat.batch, bat.pt_stride, bat.max_pages,
                     bat.num_q_heads, lay.num_kv_heads, lay.page_size, pol.n_sink_pages, pol.n_local_pages,
                     pol.static_head_mask, groups_per_seq, per_block);
  return hipGetLastError();
}

}  // namespace qasp
