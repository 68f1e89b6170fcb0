// select_topk: sink + local + top-k pages per (sequence, KV head), and the
// static A-shape page sets (sink tokens + local window; SCBench notes,
// notes.yuuk.io, "Tri-shape" paragraph).
//
// The top-k of the query-aware heads must be exactly the top-k of the exact
// group scores (largest first, equal scores to the lower page id).  The fp32
// scores of score_pages carry an error bound e, so with E the largest bound
// among the candidates and v_k, v_k1 the k-th and (k+1)-th largest fp32
// values:
//   v_j > v_k1 + 2E  -> certainly selected (at most k-1 pages can beat it),
//   v_j < v_k  - 2E  -> certainly not selected (k pages certainly beat it),
//   otherwise        -> in doubt ("band").
// The band pages get their exact score, the correctly rounded fp64 value of
// the exact real sum (an integer sum of the exact bf16 products, then one
// rounding), and the remaining places go to the best band pages by that
// score and then by lower page id.  The usual band is empty or a few pages.
//
// One block of 256 threads per (KV head, sequence).
#include <limits.h>

#include "common.h"
#include "launch.h"

namespace qasp {

namespace {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;

__device__ __forceinline__ uint32_t f32_order(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ uint64_t f64_order(double d) {
  if (d == 0.0) d = 0.0;  // one zero
  uint64_t u = (uint64_t)__double_as_longlong(d);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// ---------------------------------------------------------------------------
// block-wide helpers (256 threads)
// ---------------------------------------------------------------------------

constexpr int kQStageBytes = 8192;  // q rows of a group staged in LDS for exact re-scoring

struct SelShared {
  int hist[256];
  int ired[kSelWaves];
  float fred[kSelWaves];
  uint32_t ured[kSelWaves];
  uint64_t ared[kSelWaves], ored[kSelWaves];
  int digit, rem;
  uint16_t qstage[kQStageBytes / 2];
};

__device__ int block_sum_int(int v, SelShared &sh) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  __syncthreads();
  if (threadIdx.x % kWave == 0) sh.ired[threadIdx.x / kWave] = v;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < kSelWaves; w++) t += sh.ired[w];
  return t;
}

__device__ float block_max_float(float v, SelShared &sh) {
  v = wave_max(v);
  __syncthreads();
  if (threadIdx.x % kWave == 0) sh.fred[threadIdx.x / kWave] = v;
  __syncthreads();
  float t = sh.fred[0];
  for (int w = 1; w < kSelWaves; w++) t = fmaxf(t, sh.fred[w]);
  return t;
}

__device__ uint32_t block_max_u32(uint32_t v, SelShared &sh) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  __syncthreads();
  if (threadIdx.x % kWave == 0) sh.ured[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t t = sh.ured[0];
  for (int w = 1; w < kSelWaves; w++) t = max(t, sh.ured[w]);
  return t;
}

// Exclusive prefix of v over threads in order; *total gets the sum.
__device__ int block_exclusive_scan(int v, int *total, SelShared &sh) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int x = v;
  for (int o = 1; o < kWave; o <<= 1) {
    int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == kWave - 1) sh.ired[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kSelWaves; w++) {
    if (w < wave) base += sh.ired[w];
    tot += sh.ired[w];
  }
  *total = tot;
  return base + x - v;
}

// Given hist[256] (counts per digit) and the rank kk (1-based, from the
// top), finds the digit holding that rank: sh.digit, and the rank within
// that digit: sh.rem.  Wave 0 does it with a suffix scan, 4 bins per lane.
__device__ void find_digit_from_top(int kk, SelShared &sh) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    // lane l owns bins 255-4l .. 252-4l (descending)
    int c[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      c[i] = sh.hist[255 - 4 * lane - i];
      s += c[i];
    }
    int incl = s;
    for (int o = 1; o < kWave; o <<= 1) {
      int y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    const int excl = incl - s;
    if (excl < kk && incl >= kk) {  // exactly one lane
      int cum = excl;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        if (cum + c[i] >= kk) {
          sh.digit = 255 - 4 * lane - i;
          sh.rem = kk - cum;
          break;
        }
        cum += c[i];
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const int lo = __shfl_xor((int)(uint32_t)v, o, kWave);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), o, kWave);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Block-wide AND and OR of 64-bit values.
__device__ void block_and_or(uint64_t &a, uint64_t &o, SelShared &sh) {
  for (int s = 32; s > 0; s >>= 1) {
    a &= shfl_xor_u64(a, s);
    o |= shfl_xor_u64(o, s);
  }
  __syncthreads();
  if (threadIdx.x % kWave == 0) {
    sh.ared[threadIdx.x / kWave] = a;
    sh.ored[threadIdx.x / kWave] = o;
  }
  __syncthreads();
  a = ~0ull;
  o = 0;
  for (int w = 0; w < kSelWaves; w++) {
    a &= sh.ared[w];
    o |= sh.ored[w];
  }
}

// k-th largest (1-based) of the keys whose member bit is set (all keys when
// member_bits is null), keys in LDS.  The bits above the highest bit where
// the members differ are common to all of them and are skipped; the rest is
// resolved 8 bits per histogram pass, from the top.
template <typename U>
__device__ U kth_largest(const U *keys, const uint32_t *member_bits, int n, int k, SelShared &sh) {
  constexpr int kBits = 8 * sizeof(U);
  uint64_t a = ~0ull, o = 0;
  for (int i = threadIdx.x; i < n; i += kSelThreads) {
    if (member_bits && !((member_bits[i >> 5] >> (i & 31)) & 1u)) continue;
    a &= (uint64_t)keys[i];
    o |= (uint64_t)keys[i];
  }
  block_and_or(a, o, sh);
  const U all_and = (U)a, diff = (U)(a ^ o);
  if (diff == 0) return all_and;
  int hb = kBits - 1;
  while (!((diff >> hb) & 1)) hb--;
  U pmask = hb + 1 >= kBits ? (U)0 : (U)(~(U)0 << (hb + 1));
  U prefix = all_and & pmask;
  int kk = k;
  while (hb >= 0) {
    const int lo = hb >= 7 ? hb - 7 : 0;
    const U dmask = (U)((1u << (hb - lo + 1)) - 1u);
    sh.hist[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kSelThreads) {
      if (member_bits && !((member_bits[i >> 5] >> (i & 31)) & 1u)) continue;
      const U u = keys[i];
      if ((u & pmask) == prefix) atomicAdd(&sh.hist[(int)((u >> lo) & dmask)], 1);
    }
    __syncthreads();
    find_digit_from_top(kk, sh);
    prefix |= (U)sh.digit << lo;
    pmask |= dmask << lo;
    kk = sh.rem;
    __syncthreads();
    hb = lo - 1;
  }
  return prefix;
}

// ---------------------------------------------------------------------------
// exact page bound
// ---------------------------------------------------------------------------

// bf16 pattern -> (significand, exponent): value = m * 2^e, m < 2^8.
__device__ __forceinline__ void bf16_split(uint32_t bits, int &m, int &e) {
  const int ef = (bits >> 7) & 0xff, mant = bits & 0x7f;
  if (ef == 0) {
    m = mant;
    e = -133;
  } else {
    m = mant | 0x80;
    e = ef - 134;
  }
}

// Signed significand and exponent of the term q_d * x_d (bit patterns).
__device__ __forceinline__ void term_of(uint32_t qb, uint32_t xb, int &M, int &E) {
  int mq, eq, mx, ex;
  bf16_split(qb, mq, eq);
  bf16_split(xb, mx, ex);
  M = mq * mx;
  E = eq + ex;
  if ((qb ^ xb) & 0x8000u) M = -M;
}

// Channel-d term q_d * (q_d < 0 ? lo_d : hi_d).
__device__ __forceinline__ void bound_term(const uint16_t *qh, const uint16_t *lo, const uint16_t *hi,
                                           int d, int &M, int &E) {
  const uint32_t qb = qh[d];
  term_of(qb, (qb & 0x8000u) ? lo[d] : hi[d], M, E);
}

__device__ __forceinline__ double i64_to_f64_rn(int64_t x) {
  // both parts are exact doubles; their sum is rounded once
  const int32_t hi = (int32_t)(x >> 32);
  const uint32_t lo = (uint32_t)x;
  return (double)hi * 4294967296.0 + (double)lo;
}

// Exact sum with 32-bit digits; every lane runs it (rare path: some term is
// too small for the 64-bit window of exact_head_bound).
template <int D>
__device__ double exact_head_bound_digits(const uint16_t *qh, const uint16_t *lo, const uint16_t *hi) {
  constexpr int kDigits = 22;
  constexpr int kLow = -288;   // weight of bit 0 of digit 0: below 2^-266, the smallest term
  int64_t dg[kDigits];
  for (int i = 0; i < kDigits; i++) dg[i] = 0;
  for (int d = 0; d < D; d++) {
    int M, E;
    bound_term(qh, lo, hi, d, M, E);
    if (M == 0) continue;
    const int off = E - kLow;
    const int di = off >> 5, sh = off & 31;
    const int64_t v = (int64_t)M * ((int64_t)1 << sh);
    const int64_t low = v & 0xffffffffll;
    dg[di] += low;
    dg[di + 1] += (v - low) / ((int64_t)1 << 32);
  }
  // carries: digits into [0, 2^32), the top one keeps the sign
  for (int i = 0; i + 1 < kDigits; i++) {
    const int64_t low = dg[i] & 0xffffffffll;
    dg[i + 1] += (dg[i] - low) / ((int64_t)1 << 32);
    dg[i] = low;
  }
  bool neg = dg[kDigits - 1] < 0;
  if (neg) {
    for (int i = 0; i < kDigits; i++) dg[i] = -dg[i];
    for (int i = 0; i + 1 < kDigits; i++) {
      const int64_t low = dg[i] & 0xffffffffll;
      dg[i + 1] += (dg[i] - low) / ((int64_t)1 << 32);
      dg[i] = low;
    }
  }
  int top = kDigits - 1;
  while (top >= 0 && dg[top] == 0) top--;
  if (top < 0) return 0.0;
  // 64-bit window ending at the leading one; lower bits fold into a sticky bit
  const int lead = 32 * top + 31 - __builtin_clz((uint32_t)dg[top]);
  double r;
  if (lead < 64) {
    const uint64_t x = (uint64_t)dg[0] | ((uint64_t)dg[1] << 32);
    r = ldexp((double)(uint32_t)(x >> 32) * 4294967296.0 + (double)(uint32_t)x, kLow);
  } else {
    const int lo_bit = lead - 63;
    const int di = lo_bit >> 5, sh = lo_bit & 31;
    const uint64_t w0 = (uint64_t)dg[di] | ((uint64_t)dg[di + 1] << 32);
    const uint64_t w2 = di + 2 < kDigits ? (uint64_t)dg[di + 2] : 0;
    uint64_t x = sh == 0 ? w0 : ((w0 >> sh) | (w2 << (64 - sh)));
    bool sticky = sh != 0 && (dg[di] & ((1ll << sh) - 1)) != 0;
    for (int i = 0; i < di; i++) sticky |= dg[i] != 0;
    if (sticky) x |= 1;  // 11 bits below the rounding point: the sticky bit keeps RNE exact
    r = ldexp((double)(uint32_t)(x >> 32) * 4294967296.0 + (double)(uint32_t)x, lo_bit + kLow);
  }
  return neg ? -r : r;
}

// Correctly rounded fp64 value of the exact sum_d q_d * (q_d < 0 ? lo_d : hi_d).
// Wave-wide: lane l holds channels l, l+64, ... of the page rows (xl, xh, bit
// patterns); the terms are placed on one 64-bit integer grid just below the
// largest term and summed exactly across the wave.  qh may point to LDS.
template <int D>
__device__ double exact_head_bound(const uint16_t *qh, const uint32_t *xl, const uint32_t *xh,
                                   const uint16_t *lo, const uint16_t *hi, int lane) {
  constexpr int PER = (D + kWave - 1) / kWave;
  constexpr int LOGD = D <= 128 ? 7 : (D <= 1024 ? 10 : 16);
  constexpr int HEADROOM = 62 - 16 - LOGD;  // |sum| < D * 2^16 * 2^HEADROOM <= 2^62
  int Ms[PER], Es[PER];
  int emax = INT_MIN;
#pragma unroll
  for (int s = 0; s < PER; s++) {
    const int d = lane + kWave * s;
    Ms[s] = 0;
    Es[s] = 0;
    if (d < D) {
      const uint32_t qb = qh[d];
      term_of(qb, (qb & 0x8000u) ? xl[s] : xh[s], Ms[s], Es[s]);
      if (Ms[s] != 0) emax = max(emax, Es[s]);
    }
  }
  emax = wave_max_int(emax);
  if (emax == INT_MIN) return 0.0;
  const int base = emax - HEADROOM;
  int64_t acc = 0;
  int tiny = 0;
#pragma unroll
  for (int s = 0; s < PER; s++) {
    if (Ms[s] == 0) continue;
    const int sh = Es[s] - base;
    if (sh >= 0)
      acc += (int64_t)Ms[s] * ((int64_t)1 << sh);
    else
      tiny = 1;
  }
  if (__any(tiny)) return exact_head_bound_digits<D>(qh, lo, hi);
  acc = wave_sum_i64(acc);
  return ldexp(i64_to_f64_rn(acc), base);
}

// Exact group score of one page: max over the G heads (wave-wide).
template <int D>
__device__ double exact_page_key(const uint16_t *qg, int G, const uint16_t *lo, const uint16_t *hi, int lane) {
  constexpr int PER = (D + kWave - 1) / kWave;
  uint32_t xl[PER], xh[PER];
#pragma unroll
  for (int s = 0; s < PER; s++) {
    const int d = lane + kWave * s;
    xl[s] = d < D ? lo[d] : 0u;
    xh[s] = d < D ? hi[d] : 0u;
  }
  double best = -INFINITY;
  for (int m = 0; m < G; m++) best = fmax(best, exact_head_bound<D>(qg + (size_t)m * D, xl, xh, lo, hi, lane));
  return best;
}

}  // namespace

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ summ,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    const qasp_score *__restrict__ scores, int32_t *__restrict__ sel,
    int32_t *__restrict__ sel_count, int pt_stride, int max_pages,
    int max_sel, int Hq, int Hkv, int G, int ps, int n_sink, int n_local, int top_k,
    int sink_tokens, int window_tokens, uint64_t static_mask) {
  extern __shared__ uint64_t dyn[];
  __shared__ SelShared sh;
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int unit = b * Hkv + g;
  const int nwords = (max_pages + 31) / 32;
  uint64_t *keys64 = dyn;                                  // [max_pages]
  uint32_t *keys32 = (uint32_t *)dyn;                      // aliases keys64 until the band step
  uint32_t *sel_bits = (uint32_t *)(dyn + max_pages);      // [nwords]
  uint32_t *band_bits = sel_bits + nwords;                 // [nwords] (candidate index)

  const int L = seq_lens[b];
  const int P = num_pages_of(L, ps);
  for (int w = tid; w < nwords; w += kSelThreads) {
    sel_bits[w] = 0;
    band_bits[w] = 0;
  }
  __syncthreads();

  if (head_is_static(static_mask, g)) {
    const int sink_end = min(sink_tokens, L);
    const int win_begin = max(0, L - window_tokens);
    for (int j = tid; j < P; j += kSelThreads) {
      const int a = j * ps, e = min(a + ps, L);
      if (a < sink_end || e > win_begin) atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
    }
  } else {
    const int cand_lo = min(n_sink, P), cand_hi = max(cand_lo, P - n_local);
    const int n = cand_hi - cand_lo;
    for (int j = tid; j < P; j += kSelThreads)
      if (j < cand_lo || j >= cand_hi) atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
    const int k = top_k;
    if (k >= n) {
      for (int j = cand_lo + tid; j < cand_hi; j += kSelThreads) atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
    } else if (k > 0) {
      const qasp_score *row = scores + (size_t)unit * max_pages + cand_lo;
      float e_loc = 0.f;
      for (int i = tid; i < n; i += kSelThreads) {
        const qasp_score s = row[i];
        keys32[i] = f32_order(s.value);
        e_loc = fmaxf(e_loc, s.err);
      }
      const float emax = block_max_float(e_loc, sh);   // has a barrier before reading keys
      const uint32_t uk = kth_largest<uint32_t>(keys32, nullptr, n, k, sh);
      int c_ge = 0;
      uint32_t below = 0;
      for (int i = tid; i < n; i += kSelThreads) {
        const uint32_t u = keys32[i];
        c_ge += u >= uk;
        if (u < uk) below = max(below, u);
      }
      c_ge = block_sum_int(c_ge, sh);
      const uint32_t ubelow = block_max_u32(below, sh);
      const float vk = f32_from_order(uk);
      const float vk1 = c_ge > k ? vk : f32_from_order(ubelow);
      const double t_in = (double)vk1 + 2.0 * (double)emax;
      const double t_out = (double)vk - 2.0 * (double)emax;
      int n_in = 0, n_band = 0;
      for (int i = tid; i < n; i += kSelThreads) {
        const double v = (double)f32_from_order(keys32[i]);
        const int j = cand_lo + i;
        if (v > t_in) {
          atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
          n_in++;
        } else if (!(v < t_out)) {
          atomicOr(&band_bits[i >> 5], 1u << (i & 31));
          n_band++;
        }
      }
      n_in = block_sum_int(n_in, sh);
      n_band = block_sum_int(n_band, sh);
      const int need = k - n_in;
      if (need > 0 && need >= n_band) {
        for (int i = tid; i < n; i += kSelThreads)
          if ((band_bits[i >> 5] >> (i & 31)) & 1u) {
            const int j = cand_lo + i;
            atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
          }
      } else if (need > 0) {
        // exact scores of the band pages, one page per wave at a time
        __syncthreads();  // keys32 is dead from here; keys64 reuses the space
        const uint16_t *qb = q + ((size_t)b * Hq + (size_t)g * G) * D;
        if ((size_t)G * D * 2 <= kQStageBytes) {  // stage the group's q rows in LDS
          for (int i = tid; i < G * D / 2; i += kSelThreads)
            ((uint32_t *)sh.qstage)[i] = ((const uint32_t *)qb)[i];
          __syncthreads();
          qb = sh.qstage;
        }
        int seen = 0;
        for (int w = 0; w < (n + 31) / 32; w++) {
          uint32_t bits = band_bits[w];
          while (bits) {
            const int i = w * 32 + __builtin_ctz(bits);
            bits &= bits - 1;
            if ((seen++ % kSelWaves) != wave) continue;
            const int j = cand_lo + i;
            const int phys = page_table[(size_t)b * pt_stride + j];
            const uint16_t *lo = summ + ((size_t)phys * Hkv + g) * 2 * D;
            const uint16_t *hi = lo + D;
            const double best = exact_page_key<D>(qb, G, lo, hi, lane);
            if (lane == 0) keys64[i] = f64_order(best);
          }
        }
        __syncthreads();
        const uint64_t kth = kth_largest<uint64_t>(keys64, band_bits, n, need, sh);
        // all band pages above kth, then the lowest ids among those equal to it
        int above = 0;
        for (int i = tid; i < n; i += kSelThreads)
          if (((band_bits[i >> 5] >> (i & 31)) & 1u) && keys64[i] > kth) {
            const int j = cand_lo + i;
            atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
            above++;
          }
        above = block_sum_int(above, sh);
        int take = need - above;
        // ascending scan of the ties, 256 candidates per round
        for (int i0 = 0; i0 < n && take > 0; i0 += kSelThreads) {
          const int i = i0 + tid;
          const int tie = i < n && ((band_bits[i >> 5] >> (i & 31)) & 1u) && keys64[i] == kth;
          int total;
          const int before = block_exclusive_scan(tie, &total, sh);
          if (tie && before < take) {
            const int j = cand_lo + i;
            atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
          }
          take -= min(total, take);
        }
      }
    }
  }
  __syncthreads();

  // ascending list of the selected pages
  int32_t *out = sel + (size_t)unit * max_sel;
  int written = 0;
  for (int w0 = 0; w0 < nwords; w0 += kSelThreads) {
    const int w = w0 + tid;
    const uint32_t bits = w < nwords ? sel_bits[w] : 0u;
    int total;
    int pos = written + block_exclusive_scan(__popc(bits), &total, sh);
    uint32_t x = bits;
    while (x) {
      const int j = w * 32 + __builtin_ctz(x);
      x &= x - 1;
      if (pos < max_sel) out[pos] = j;
      pos++;
    }
    written += total;
  }
  const int count = min(written, max_sel);
  for (int i = count + tid; i < max_sel; i += kSelThreads) out[i] = -1;
  if (tid == 0) sel_count[unit] = count;
}

hipError_t launch_select_topk(const qasp_layout &lay, const qasp_batch &bat,
                              const qasp_policy &pol, const uint16_t *q, const uint16_t *summ,
                              const qasp_score *scores, int32_t *sel, int32_t *sel_count,
                              int max_sel, hipStream_t stream) {
  if (bat.batch == 0) return hipSuccess;
  const int G = bat.num_q_heads / lay.num_kv_heads;
  const int mp = bat.max_pages > 0 ? bat.max_pages : 1;
  const size_t lds = (size_t)mp * 8 + 2 * (size_t)((mp + 31) / 32) * 4;
  dim3 grid(lay.num_kv_heads, bat.batch);
#define QASP_SELECT_ARGS                                                                        \
  q, summ, bat.page_table, bat.seq_lens, scores, sel, sel_count,                                \
      bat.pt_stride, mp, max_sel, bat.num_q_heads, lay.num_kv_heads, G, lay.page_size,          \
      pol.n_sink_pages, pol.n_local_pages, pol.top_k, pol.sink_tokens, pol.window_tokens,        \
      pol.static_head_mask
  if (lay.head_dim_k == 128) {
    hipLaunchKernelGGL(select_topk_kernel<128>, grid, dim3(kSelThreads), lds, stream, QASP_SELECT_ARGS);
  } else if (lay.head_dim_k == 576) {
    hipLaunchKernelGGL(select_topk_kernel<576>, grid, dim3(kSelThreads), lds, stream, QASP_SELECT_ARGS);
  } else {
    return hipErrorInvalidValue;
  }
#undef QASP_SELECT_ARGS
  return hipGetLastError();
}

}  // namespace qasp
