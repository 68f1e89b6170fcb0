// Device building blocks of select_topk: per (sequence, KV head) block, the
// sink + local + top-k page selection with exact tie handling.
//
// The top-k of the query-aware heads must be exactly the top-k of the exact
// group scores (largest first, equal scores to the lower page id).  The fp32
// scores carry an error bound e, so with E the largest bound among the
// candidates and v_k, v_k1 the k-th and (k+1)-th largest fp32 values:
//   v_j > v_k1 + 2E  -> certainly selected (at most k-1 pages can beat it),
//   v_j < v_k  - 2E  -> certainly not selected (k pages certainly beat it),
//   otherwise        -> in doubt ("band").
// The band pages get their exact score, the correctly rounded fp64 value of
// the exact real sum (an integer sum of the exact bf16 products, then one
// rounding), and the remaining places go to the best band pages by that
// score and then by lower page id.  The usual band is empty or a few pages.
#pragma once

#include "common.h"

namespace qasp {
namespace sel {

constexpr int kQStageBytes = 8192;  // q rows of a group staged in LDS for exact re-scoring
constexpr int kSmallBand = 64;      // bands up to this size are ranked by one wave

// Order-preserving unsigned keys of fp32 / fp64 values (one zero).
__device__ __forceinline__ uint32_t f32_order(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ uint64_t f64_order(double d) {
  if (d == 0.0) d = 0.0;
  uint64_t u = (uint64_t)__double_as_longlong(d);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const int lo = __shfl_xor((int)(uint32_t)v, o, kWave);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), o, kWave);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

template <int NW>
struct SelShared {
  int hist[NW][256];          // one digit histogram per wave
  int red[NW][4];             // per-wave partials of block reductions
  int digit, rem, nlist, bincnt;
  int n_in, nsel;
  uint32_t kin, kib;          // smallest key above the band / of the band and above
  int kbin[2], krem[2], kcnt[2], nk[2];
  uint32_t uk, uk1;
  int list[kSmallBand];
  int bphys[kSmallBand], blead[kSmallBand];  // physical page and certified leading head of listed band pages
  uint32_t klist[kSmallBand];   // keys of one histogram bin
  uint32_t klist1[kSmallBand];  // keys of a second bin
  double lkey[kSmallBand];
  uint32_t rows[NW][128];     // one page's summary rows per wave (2 x 128 bf16)
  uint16_t qstage[kQStageBytes / 2];
};

// ---------------------------------------------------------------------------
// block-wide helpers: DPP inside a wave, one LDS exchange across waves
// ---------------------------------------------------------------------------

template <int NW>
__device__ void block_sum2(int &a, int &b, SelShared<NW> &sh) {
  a = wave_sum_dpp(a);
  b = wave_sum_dpp(b);
  __syncthreads();
  if (threadIdx.x % kWave == 0) {
    sh.red[threadIdx.x / kWave][0] = a;
    sh.red[threadIdx.x / kWave][1] = b;
  }
  __syncthreads();
  a = b = 0;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    a += sh.red[w][0];
    b += sh.red[w][1];
  }
}

// sum of c, max of m
template <int NW>
__device__ void block_sum_max(int &c, int &m, SelShared<NW> &sh) {
  c = wave_sum_dpp(c);
  m = wave_max_dpp(m);
  __syncthreads();
  if (threadIdx.x % kWave == 0) {
    sh.red[threadIdx.x / kWave][0] = c;
    sh.red[threadIdx.x / kWave][1] = m;
  }
  __syncthreads();
  c = 0;
  m = INT_MIN;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    c += sh.red[w][0];
    m = max(m, sh.red[w][1]);
  }
}

// max of f, AND and OR of the 32-bit a / o
template <int NW>
__device__ void block_max_and_or(float &f, uint32_t &a, uint32_t &o, SelShared<NW> &sh) {
  f = wave_max_dpp(f);
  a = wave_and_dpp(a);
  o = wave_or_dpp(o);
  __syncthreads();
  if (threadIdx.x % kWave == 0) {
    sh.red[threadIdx.x / kWave][0] = __float_as_int(f);
    sh.red[threadIdx.x / kWave][1] = (int)a;
    sh.red[threadIdx.x / kWave][2] = (int)o;
  }
  __syncthreads();
  f = __int_as_float(sh.red[0][0]);
  a = ~0u;
  o = 0;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    f = fmaxf(f, __int_as_float(sh.red[w][0]));
    a &= (uint32_t)sh.red[w][1];
    o |= (uint32_t)sh.red[w][2];
  }
}

// max of f, min and max of the unsigned keys lo / hi
template <int NW>
__device__ void block_max_min_max(float &f, uint32_t &lo, uint32_t &hi, SelShared<NW> &sh) {
  f = wave_max_dpp(f);
  const int nlo = wave_max_dpp((int)(~lo ^ 0x80000000u));  // max of ~lo = ~min(lo), biased to signed
  const int nhi = wave_max_dpp((int)(hi ^ 0x80000000u));
  __syncthreads();
  if (threadIdx.x % kWave == 0) {
    sh.red[threadIdx.x / kWave][0] = __float_as_int(f);
    sh.red[threadIdx.x / kWave][1] = nlo;
    sh.red[threadIdx.x / kWave][2] = nhi;
  }
  __syncthreads();
  f = __int_as_float(sh.red[0][0]);
  int a = INT_MIN, b = INT_MIN;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    f = fmaxf(f, __int_as_float(sh.red[w][0]));
    a = max(a, sh.red[w][1]);
    b = max(b, sh.red[w][2]);
  }
  lo = ~((uint32_t)a ^ 0x80000000u);
  hi = (uint32_t)b ^ 0x80000000u;
}

// AND and OR of 64-bit values
template <int NW>
__device__ void block_and_or64(uint64_t &a, uint64_t &o, SelShared<NW> &sh) {
  const uint32_t alo = wave_and_dpp((uint32_t)a), ahi = wave_and_dpp((uint32_t)(a >> 32));
  const uint32_t olo = wave_or_dpp((uint32_t)o), ohi = wave_or_dpp((uint32_t)(o >> 32));
  __syncthreads();
  if (threadIdx.x % kWave == 0) {
    int *r = sh.red[threadIdx.x / kWave];
    r[0] = (int)alo; r[1] = (int)ahi; r[2] = (int)olo; r[3] = (int)ohi;
  }
  __syncthreads();
  a = ~0ull;
  o = 0;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    a &= ((uint64_t)(uint32_t)sh.red[w][1] << 32) | (uint32_t)sh.red[w][0];
    o |= ((uint64_t)(uint32_t)sh.red[w][3] << 32) | (uint32_t)sh.red[w][2];
  }
}

// Exclusive prefix of v over threads in order; *total gets the sum.
template <int NW>
__device__ int block_exclusive_scan(int v, int *total, SelShared<NW> &sh) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int incl = wave_incl_sum(v);
  __syncthreads();
  if (lane == kWave - 1) sh.red[wave][0] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    if (w < wave) base += sh.red[w][0];
    tot += sh.red[w][0];
  }
  *total = tot;
  return base + incl - v;
}

// With the per-wave histograms filled, finds the digit holding rank kk
// (1-based, from the top): sh.digit, and the rank inside it: sh.rem.  Wave 0:
// lane l owns digits 255-4l .. 252-4l, summed over the waves' histograms.
template <int NW>
__device__ void find_digit_from_top(int kk, SelShared<NW> &sh) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int c[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int bin = 255 - 4 * lane - i;
      int t = 0;
#pragma unroll
      for (int w = 0; w < NW; w++) t += sh.hist[w][bin];
      c[i] = t;
      s += t;
    }
    const int incl = wave_incl_sum(s);
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

// k-th largest (1-based) of the keys whose member bit is set (all keys when
// member_bits is null); all_and / all_or are the AND and OR of the member
// keys.  The bits above the highest bit where the members differ are common
// to all of them; the rest is resolved 8 bits per histogram pass.
template <typename U, int NW>
__device__ U kth_largest(const U *keys, const uint32_t *member_bits, int n, int k, U all_and, U all_or,
                         SelShared<NW> &sh) {
  constexpr int kBits = 8 * sizeof(U);
  const U diff = all_and ^ all_or;
  if (diff == 0) return all_and;
  int hb = kBits - 1;
  while (!((diff >> hb) & 1)) hb--;
  U pmask = hb + 1 >= kBits ? (U)0 : (U)(~(U)0 << (hb + 1));
  U prefix = all_and & pmask;
  int kk = k;
  int *myhist = sh.hist[threadIdx.x / kWave];
  while (hb >= 0) {
    const int lo = hb >= 7 ? hb - 7 : 0;
    const U dmask = (U)((1u << (hb - lo + 1)) - 1u);
    for (int i = threadIdx.x % kWave; i < 256; i += kWave) myhist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NW * kWave) {
      if (member_bits && !((member_bits[i >> 5] >> (i & 31)) & 1u)) continue;
      const U u = keys[i];
      if ((u & pmask) == prefix) atomicAdd(&myhist[(int)((u >> lo) & dmask)], 1);
    }
    __syncthreads();
    find_digit_from_top(kk, sh);
    prefix |= (U)sh.digit << lo;
    pmask |= dmask << lo;
    kk = sh.rem;
    hb = lo - 1;
  }
  return prefix;
}

// k-th largest (1-based) of the 32-bit keys, all of which lie in [lo, hi].
// One pass spreads the keys of [lo, hi] over NW*256 equal bins (a shared
// LDS histogram: few keys per bin, so the atomics rarely collide), finds the
// bin holding rank k from the top, and either ranks that bin's keys in one
// wave (up to kSmallBand of them) or narrows [lo, hi] to the bin and repeats.
template <int NW>
__device__ uint32_t kth_largest_range(const uint32_t *keys, int n, int k, uint32_t lo, uint32_t hi,
                                      SelShared<NW> &sh) {
  constexpr int T = NW * kWave, NB = 4 * T;
  static_assert(NB * sizeof(int) <= sizeof(sh.hist), "histogram size");
  int *hist = &sh.hist[0][0];
  const int tid = threadIdx.x;
  int kk = k;
  for (;;) {
    if (lo == hi) return lo;
    int shift = 0;
    while (((hi - lo) >> shift) >= (uint32_t)NB) shift++;
    for (int i = tid; i < NB; i += T) hist[i] = 0;
    if (tid == 0) sh.nlist = 0;
    __syncthreads();
    for (int i = tid; i < n; i += T) {
      const uint32_t u = keys[i];
      if (u >= lo && u <= hi) atomicAdd(&hist[(u - lo) >> shift], 1);
    }
    __syncthreads();
    // thread t owns bins NB-1-4t .. NB-4-4t, scanned from the top
    int c[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      c[j] = hist[NB - 1 - 4 * tid - j];
      s += c[j];
    }
    int total;
    const int excl = block_exclusive_scan(s, &total, sh);
    if (excl < kk && excl + s >= kk) {  // exactly one thread
      int cum = excl;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (cum + c[j] >= kk) {
          sh.digit = NB - 1 - 4 * tid - j;
          sh.rem = kk - cum;
          sh.bincnt = c[j];
          break;
        }
        cum += c[j];
      }
    }
    __syncthreads();
    const uint32_t blo = lo + ((uint32_t)sh.digit << shift);
    const uint32_t bhi = shift == 0 ? blo : min(hi, blo + ((1u << shift) - 1u));
    const int cnt = sh.bincnt;
    kk = sh.rem;
    if (shift == 0) return blo;
    if (cnt > kSmallBand) {
      lo = blo;
      hi = bhi;
      continue;
    }
    // the bin's keys, ranked by one wave: the kk-th largest of them
    for (int i = tid; i < n; i += T) {
      const uint32_t u = keys[i];
      if (u >= blo && u <= bhi) sh.klist[atomicAdd(&sh.nlist, 1)] = u;
    }
    __syncthreads();
    if (tid == 0) sh.nlist = 0;  // free for the band list
    if (tid < kWave) {
      const uint32_t mine = tid < cnt ? sh.klist[tid] : 0u;
      int greater = 0, ge = 0;
      for (int e = 0; e < cnt; e++) {
        const uint32_t o = sh.klist[e];
        greater += o > mine;
        ge += o >= mine;
      }
      if (tid < cnt && greater < kk && ge >= kk) sh.digit = (int)mine;  // equal keys write the same value
    }
    __syncthreads();
    return (uint32_t)sh.digit;
  }
}

// The key of rank r (1-based, from the top) among the cnt <= 64 keys held
// one per lane (mine, lanes < cnt); lane-to-lane reads go through SGPRs.
__device__ __forceinline__ uint32_t rank_in_wave(uint32_t mine, int cnt, int r, int lane) {
  int greater = 0, ge = 0;
  for (int e = 0; e < cnt; e++) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)mine, e);
    greater += o > mine;
    ge += o >= mine;
  }
  const uint64_t hit = __ballot(lane < cnt && greater < r && ge >= r);  // equal keys: same value
  return (uint32_t)__shfl((int)mine, hit ? (int)__builtin_ctzll(hit) : 0, kWave);
}

// The k-th and (k+1)-th largest (1-based) of the n > k keys in [lo, hi].
// The block spreads the keys over NB = NW*256 equal bins (shared LDS
// histogram, which the caller has zeroed; few keys per bin, so the atomics
// rarely collide); a suffix scan over the bins locates the bins of ranks k
// and k+1; their keys are gathered and ranked by wave 0.  Five barriers.
// Bins of more than 64 keys (many equal or very close keys) fall back to
// kth_largest_range and a counting pass.
template <int NW>
__device__ void kth_pair(const uint32_t *keys, int n, int k, uint32_t lo, uint32_t hi, SelShared<NW> &sh,
                         uint32_t &uk, uint32_t &uk1) {
  constexpr int T = NW * kWave, NB = 4 * T;
  int *hist = &sh.hist[0][0];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  if (lo == hi) {  // block-uniform
    __syncthreads();
    uk = uk1 = lo;
    return;
  }
  int shift = 0;
  while (((hi - lo) >> shift) >= (uint32_t)NB) shift++;
  if (tid == 0) sh.nk[0] = sh.nk[1] = 0;
  for (int i = tid; i < n; i += T) atomicAdd(&hist[(keys[i] - lo) >> shift], 1);
  __syncthreads();
  // thread t owns bins NB-1-4t .. NB-4-4t, counted from the top
  int c[4], s = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    c[j] = hist[NB - 1 - 4 * tid - j];
    s += c[j];
  }
  const int incl = wave_incl_sum(s);
  if (lane == kWave - 1) sh.red[wave][3] = incl;
  __syncthreads();
  int excl = incl - s;
#pragma unroll
  for (int w = 0; w < NW; w++)
    if (w < wave) excl += sh.red[w][3];
#pragma unroll
  for (int x = 0; x < 2; x++) {
    const int r = k + x;
    if (excl < r && excl + s >= r) {
      int cum = excl;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (cum + c[j] >= r) {
          sh.kbin[x] = NB - 1 - 4 * tid - j;
          sh.krem[x] = r - cum;
          sh.kcnt[x] = c[j];
          break;
        }
        cum += c[j];
      }
    }
  }
  __syncthreads();
  const int bin0 = sh.kbin[0], bin1 = sh.kbin[1];
  const int cnt0 = sh.kcnt[0], cnt1 = bin1 == bin0 ? 0 : sh.kcnt[1];
  if (cnt0 <= kWave && cnt1 <= kWave) {  // block-uniform
    for (int i = tid; i < n; i += T) {
      const uint32_t u = keys[i];
      const int b = (int)((u - lo) >> shift);
      if (b == bin0) sh.klist[atomicAdd(&sh.nk[0], 1)] = u;
      else if (b == bin1) sh.klist1[atomicAdd(&sh.nk[1], 1)] = u;
    }
    __syncthreads();
    if (wave == 0) {
      const uint32_t k0 = lane < cnt0 ? sh.klist[lane] : 0u;
      const uint32_t a = rank_in_wave(k0, cnt0, sh.krem[0], lane);
      const uint32_t k1 = bin1 == bin0 ? k0 : (lane < cnt1 ? sh.klist1[lane] : 0u);
      const uint32_t b1 = rank_in_wave(k1, bin1 == bin0 ? cnt0 : cnt1, sh.krem[1], lane);
      if (lane == 0) {
        sh.uk = a;
        sh.uk1 = b1;
      }
    }
    __syncthreads();
    uk = sh.uk;
    uk1 = sh.uk1;
    return;
  }
  uk = kth_largest_range<NW>(keys, n, k, lo, hi, sh);
  // (k+1)-th largest: uk again if more than k keys reach it, else the largest below it
  int c_ge = 0;
  int below = INT_MIN;  // unsigned order keys, biased into the signed range
  for (int i = tid; i < n; i += T) {
    const uint32_t u = keys[i];
    c_ge += u >= uk;
    if (u < uk) below = max(below, (int)(u ^ 0x80000000u));
  }
  block_sum_max(c_ge, below, sh);
  uk1 = c_ge > k ? uk : ((uint32_t)below ^ 0x80000000u);
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

// Wave-uniform 64-bit read of lane src's value (src the same on every lane).
__device__ __forceinline__ int64_t readlane64(int64_t v, int src) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), src);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Digits into [0, 2^32), lane by lane from the lowest, the carries moving up;
// the top digit keeps the sign.  Lane i holds digit i.
template <int kDigits>
__device__ __forceinline__ int64_t carry_digits(int64_t dg, int lane) {
  for (int i = 0; i + 1 < kDigits; i++) {
    const int64_t x = readlane64(dg, i);
    const int64_t low = x & 0xffffffffll;
    if (lane == i) dg = low;
    if (lane == i + 1) dg += (x - low) / ((int64_t)1 << 32);
  }
  return dg;
}

// Exact sum with 32-bit digits, one digit per lane (lane i: weight
// 2^(-288 + 32 i), 22 digits from below 2^-266, the smallest term, to above
// the largest sum); wave-wide: every lane walks the same terms (the lanes of
// the two digits a term touches add its parts) and returns the result.  Call
// with every lane of the wave and wave-uniform arguments.  Rare path: some
// term is too small for the 64-bit window of exact_head_bound.
template <int D>
__device__ __forceinline__ double exact_head_bound_digits(const uint16_t *qh, const uint16_t *lo, const uint16_t *hi) {
  constexpr int kDigits = 22;
  constexpr int kLow = -288;   // weight of bit 0 of digit 0: below 2^-266, the smallest term
  static_assert(kDigits <= kWave, "one digit per lane");
  const int lane = threadIdx.x % kWave;
  int64_t dg = 0;
  for (int d = 0; d < D; d++) {
    int M, E;
    bound_term(qh, lo, hi, d, M, E);
    if (M == 0) continue;
    const int off = E - kLow;
    const int di = off >> 5, sh = off & 31;
    const int64_t v = (int64_t)M * ((int64_t)1 << sh);
    const int64_t low = v & 0xffffffffll;
    if (lane == di) dg += low;
    if (lane == di + 1) dg += (v - low) / ((int64_t)1 << 32);
  }
  dg = carry_digits<kDigits>(dg, lane);
  const bool neg = readlane64(dg, kDigits - 1) < 0;
  if (neg) dg = carry_digits<kDigits>(-dg, lane);
  const uint64_t nz = __ballot(lane < kDigits && dg != 0);
  if (nz == 0) return 0.0;
  const int top = 63 - __builtin_clzll(nz);
  // 64-bit window ending at the leading one; lower bits fold into a sticky bit
  const int lead = 32 * top + 31 - __builtin_clz((uint32_t)readlane64(dg, top));
  double r;
  if (lead < 64) {
    const uint64_t x = (uint64_t)readlane64(dg, 0) | ((uint64_t)readlane64(dg, 1) << 32);
    r = ldexp((double)(uint32_t)(x >> 32) * 4294967296.0 + (double)(uint32_t)x, kLow);
  } else {
    const int lo_bit = lead - 63;
    const int di = lo_bit >> 5, sh = lo_bit & 31;
    const uint64_t d0 = (uint64_t)readlane64(dg, di);
    const uint64_t w0 = d0 | ((uint64_t)readlane64(dg, di + 1) << 32);
    const uint64_t w2 = di + 2 < kDigits ? (uint64_t)readlane64(dg, di + 2) : 0;
    uint64_t x = sh == 0 ? w0 : ((w0 >> sh) | (w2 << (64 - sh)));
    bool sticky = sh != 0 && (d0 & ((1ull << sh) - 1)) != 0;
    sticky |= __ballot(lane < di && dg != 0) != 0;
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
__device__ __forceinline__ double exact_head_bound(const uint16_t *qh, const uint32_t *xl, const uint32_t *xh,
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
__device__ __forceinline__ double exact_page_key(const uint16_t *qg, int G, const uint16_t *lo, const uint16_t *hi, int lane) {
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

// Exact group score of one page for up to 64 / NP heads at once: lane l
// works on head l / NP and channels (l % NP) + NP t of the page rows (rows:
// lo then hi, bf16 pairs in LDS); the NP lanes of a head sum exactly on a
// common 64-bit grid, then the wave takes the max over heads.  Falls back to
// the per-head digit sum when some term lies below the grid.
template <int D, int NP>
__device__ __forceinline__ double exact_page_key_heads(const uint16_t *qg, int G, const uint16_t *rows,
                                       const uint16_t *lo_g, const uint16_t *hi_g, int lane) {
  constexpr int PER = D / NP;
  constexpr int LOGD = D <= 128 ? 7 : (D <= 1024 ? 10 : 16);
  constexpr int HEADROOM = 62 - 16 - LOGD;  // |sum of D terms| < 2^62
  const int m = lane / NP, part = lane % NP;
  const bool live = m < G;
  const uint16_t *qh = qg + (size_t)(live ? m : 0) * D;
  int Ms[PER], Es[PER];
  int emax = INT_MIN;
#pragma unroll
  for (int t = 0; t < PER; t++) {
    const int d = part + NP * t;
    const uint32_t qb = qh[d];
    term_of(qb, (qb & 0x8000u) ? rows[d] : rows[D + d], Ms[t], Es[t]);
    if (live && Ms[t] != 0) emax = max(emax, Es[t]);
  }
#pragma unroll
  for (int o = 1; o < NP; o <<= 1) emax = max(emax, __shfl_xor(emax, o, kWave));
  const int base = emax - HEADROOM;
  int64_t acc = 0;
  int tiny = 0;
  if (live && emax != INT_MIN) {
#pragma unroll
    for (int t = 0; t < PER; t++) {
      if (Ms[t] == 0) continue;
      const int sh = Es[t] - base;
      if (sh >= 0)
        acc += (int64_t)Ms[t] * ((int64_t)1 << sh);
      else
        tiny = 1;
    }
  }
  if (__any(tiny)) {
    double best = -INFINITY;
    for (int h = 0; h < G; h++) best = fmax(best, exact_head_bound_digits<D>(qg + (size_t)h * D, lo_g, hi_g));
    return best;
  }
#pragma unroll
  for (int o = 1; o < NP; o <<= 1) acc += (int64_t)shfl_xor_u64((uint64_t)acc, o);
  double v = -INFINITY;
  if (live) v = emax == INT_MIN ? 0.0 : ldexp(i64_to_f64_rn(acc), base);
  for (int o = NP; o < kWave; o <<= 1) v = fmax(v, __shfl_xor(v, o, kWave));
  return v;
}

// Keys per thread of a pass over the n candidate keys with T threads: the
// fewest (4, 8 or 16) that cover them in one round, so that small sets
// spread over many threads and large ones need no more barriers.
template <int T>
__device__ __forceinline__ int keys_per_thread(int n) {
  return n <= 4 * T ? 4 : (n <= 8 * T ? 8 : 16);
}

// Four-key chunks [i, i + PER) of the candidate keys that start below n, as
// 16-byte LDS loads (the keys area holds 8 bytes per page, so a chunk's tail
// past n is still inside it; callers mask those keys).  keys32 must be
// 16-byte aligned.
template <int PER>
__device__ __forceinline__ void load_key_chunks(uint32_t (&kr)[PER], const uint32_t *keys32, int i, int n) {
#pragma unroll
  for (int r = 0; r < PER / 4; r++) {
    const uint4 v = i + 4 * r < n ? *(const uint4 *)(keys32 + i + 4 * r) : make_uint4(0, 0, 0, 0);
    kr[4 * r] = v.x;
    kr[4 * r + 1] = v.y;
    kr[4 * r + 2] = v.z;
    kr[4 * r + 3] = v.w;
  }
}

// The classification pass of select_candidates over this thread's keys
// (PER per thread a round): counts the keys certainly in (value above t_in)
// and the smallest such key (kin) and the smallest key not certainly out
// (value not below t_out: kib); the keys in doubt go to band_bits and, the
// first kSmallBand of them, to sh.list (sh.nlist counts them all).
template <int NW, int PER>
__device__ __forceinline__ void classify_keys(SelShared<NW> &sh, const uint32_t *keys32, uint32_t *band_bits, int n,
                                              double t_in, double t_out, int &c_in, uint32_t &kin, uint32_t &kib) {
  constexpr int T = NW * kWave;
  for (int i0 = 0; i0 < n; i0 += PER * T) {
    const int i = i0 + PER * (int)threadIdx.x;
    uint32_t kr[PER];
    load_key_chunks<PER>(kr, keys32, i, n);
#pragma unroll
    for (int e = 0; e < PER; e++) {
      const int ie = i + e;
      if (ie >= n) continue;
      const uint32_t key = kr[e];
      const double v = (double)f32_from_order(key);
      if (v > t_in) {
        c_in++;
        kin = min(kin, key);
        kib = min(kib, key);
      } else if (!(v < t_out)) {
        kib = min(kib, key);
        atomicOr(&band_bits[ie >> 5], 1u << (ie & 31));
        const int pos = atomicAdd(&sh.nlist, 1);
        if (pos < kSmallBand) sh.list[pos] = ie;
      }
    }
  }
}

// Returns true when the top k are exactly the candidates whose key is >=
// *uk_fast (see emit_by_threshold): always when no candidate is in doubt
// (the k-th value beats the (k+1)-th by more than twice the largest error
// bound), and when the pages in doubt are few (at most kSmallBand) or all
// selected — the keys of re-scored band pages are then rewritten, winners to
// the largest key and losers to 0.  Otherwise (a larger band, re-scored
// through keys64) marks the top-k candidates in sel_bits and returns false.
// Called by every thread of the block.  Preconditions: keys32[0..n) hold the candidates' order keys (LDS,
// visible to all threads); band_bits and sh.hist are zero; emax, k_min and k_max are the
// block-wide max error bound and the smallest and largest key;
// 0 < k < n.  Candidate i is logical page cand_lo + i; pt_row is the
// sequence's page-table row; qg the group's first q row (global).  keys64
// aliases keys32 (8 bytes per candidate) for large bands.  cand_scores (may
// be null) holds the candidates' stored scores: a certified leading head
// reduces a page's exact re-score to that one head.  cand_phys (may be null,
// then pt_row is read) holds the candidates' physical pages.  qg may already
// point to sh.qstage.
template <int D, int NW>
__device__ bool select_candidates(SelShared<NW> &sh, uint32_t *keys32, uint64_t *keys64, uint32_t *sel_bits,
                                  uint32_t *band_bits, int n, int k, int cand_lo, float emax, uint32_t k_min,
                                  uint32_t k_max, const uint16_t *qg, int G, const uint16_t *summ,
                                  const int32_t *pt_row, int Hkv, int g, const qasp_score *cand_scores,
                                  const int32_t *cand_phys, uint32_t *uk_fast) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  uint32_t uk, uk1;
  if (tid == 0) {  // ordered before use by the barriers inside kth_pair
    sh.n_in = 0;
    sh.kin = sh.kib = ~0u;
  }
  kth_pair<NW>(keys32, n, k, k_min, k_max, sh, uk, uk1);
  const float vk = f32_from_order(uk), vk1 = f32_from_order(uk1);
  const double t_in = (double)vk1 + 2.0 * (double)emax;
  const double t_out = (double)vk - 2.0 * (double)emax;
  // block-uniform: every value >= vk is above t_in and every value <= vk1
  // below t_out, so no page is in doubt and the k keys >= uk are the top k
  if ((double)vk > t_in && (double)vk1 < t_out) {
    *uk_fast = uk;
    return true;
  }
  // one pass: count the pages certainly in, the smallest key among them and
  // among the pages not certainly out, and list the band (sh.nlist counts it;
  // the first kSmallBand indices land in sh.list, every one in band_bits)
  // (keys_per_thread keys per thread, 16-byte LDS loads, as in
  // emit_by_threshold)
  int c_in = 0;
  uint32_t kin = ~0u, kib = ~0u;
  const int per = keys_per_thread<NW * kWave>(n);  // block-uniform
  if (per == 4)
    classify_keys<NW, 4>(sh, keys32, band_bits, n, t_in, t_out, c_in, kin, kib);
  else if (per == 8)
    classify_keys<NW, 8>(sh, keys32, band_bits, n, t_in, t_out, c_in, kin, kib);
  else
    classify_keys<NW, 16>(sh, keys32, band_bits, n, t_in, t_out, c_in, kin, kib);
  c_in = wave_sum_dpp(c_in);
  kin = ~(uint32_t)wave_max_dpp((int)(~kin ^ 0x80000000u)) ^ 0x80000000u;  // wave min of unsigned keys
  kib = ~(uint32_t)wave_max_dpp((int)(~kib ^ 0x80000000u)) ^ 0x80000000u;
  if (lane == 0) {
    if (c_in) atomicAdd(&sh.n_in, c_in);
    atomicMin(&sh.kin, kin);
    atomicMin(&sh.kib, kib);
  }
  __syncthreads();
  const int n_in = sh.n_in, n_band = sh.nlist;
  const int need = k - n_in;
  if (need <= 0) {  // (block-uniform) no band page is needed: the pages above the band
    *uk_fast = sh.kin;
    return true;
  }
  if (need >= n_band) {  // every band page is needed: the band and the pages above it
    *uk_fast = sh.kib;
    return true;
  }
  // exact scores of the band pages
  const uint16_t *qb = qg;
  const bool stage = qg != sh.qstage && (size_t)G * D * 2 <= kQStageBytes;  // block-uniform
  if (stage) {  // the group's q rows to LDS
    for (int i = tid; i < G * D / 2; i += NW * kWave) ((uint32_t *)sh.qstage)[i] = ((const uint32_t *)qb)[i];
    qb = sh.qstage;
  }
  if (n_band <= kSmallBand) {
    // exact keys of the listed band (one page per wave), ranked by one wave;
    // the winners' keys become the largest key, the losers' 0.  The band
    // pages' physical pages and leading heads are fetched together first.
    if (tid < n_band) {
      const int i = sh.list[tid];
      sh.bphys[tid] = cand_phys ? cand_phys[i] : pt_row[cand_lo + i];
      sh.blead[tid] = cand_scores ? cand_scores[i].head : -1;
    }
    __syncthreads();  // the staged q rows, the band pages' entries
    for (int e = wave; e < n_band; e += NW) {
      const int phys = sh.bphys[e];
      const uint16_t *lo = summ + summ_record(phys, g, Hkv) * 2 * D;
      double key;
      const int lead = sh.blead[e];
      if (lead >= 0) {
        key = exact_page_key<D>(qb + (size_t)lead * D, 1, lo, lo + D, lane);
      } else if (D == 128 && G <= 16) {
        for (int x = lane; x < D; x += kWave) sh.rows[wave][x] = ((const uint32_t *)lo)[x];
        const uint16_t *rows = (const uint16_t *)sh.rows[wave];
        key = G <= 4 ? exact_page_key_heads<D, 16>(qb, G, rows, lo, lo + D, lane)
                     : (G <= 8 ? exact_page_key_heads<D, 8>(qb, G, rows, lo, lo + D, lane)
                               : exact_page_key_heads<D, 4>(qb, G, rows, lo, lo + D, lane));
      } else {
        key = exact_page_key<D>(qb, G, lo, lo + D, lane);
      }
      if (lane == 0) sh.lkey[e] = key;
    }
    __syncthreads();
    if (wave == 0 && lane < n_band) {
      const double kl = sh.lkey[lane];
      const int il = sh.list[lane];
      int rank = 0;  // band pages that beat this one: larger key, or equal key and lower id
      for (int e = 0; e < n_band; e++) {
        const double ke = sh.lkey[e];
        rank += ke > kl || (ke == kl && sh.list[e] < il);
      }
      keys32[il] = rank < need ? ~0u : 0u;
    }
    __syncthreads();  // the rewritten keys
    *uk_fast = sh.kin;  // the pages above the band and the winners (all keys >= it)
    return true;
  } else {
    // the pages above the band into sel_bits (their keys are >= sh.kin)
    const uint32_t kin_all = sh.kin;
    for (int i = tid; i < n; i += NW * kWave)
      if (keys32[i] >= kin_all) {
        const int j = cand_lo + i;
        atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
      }
    __syncthreads();  // keys32 is dead from here; keys64 reuses the space
    uint64_t b_and = ~0ull, b_or = 0;
    int seen = 0;
    for (int w = 0; w < (n + 31) / 32; w++) {
      uint32_t bits = band_bits[w];
      while (bits) {
        const int i = w * 32 + __builtin_ctz(bits);
        bits &= bits - 1;
        if ((seen++ % NW) != wave) continue;
        const int phys = cand_phys ? cand_phys[i] : pt_row[cand_lo + i];
        const uint16_t *lo = summ + summ_record(phys, g, Hkv) * 2 * D;
        const int lead = cand_scores ? cand_scores[i].head : -1;
        const uint64_t o = f64_order(lead >= 0 ? exact_page_key<D>(qb + (size_t)lead * D, 1, lo, lo + D, lane)
                                               : exact_page_key<D>(qb, G, lo, lo + D, lane));
        if (lane == 0) keys64[i] = o;
        b_and &= o;
        b_or |= o;
      }
    }
    block_and_or64(b_and, b_or, sh);
    const uint64_t kth = kth_largest<uint64_t, NW>(keys64, band_bits, n, need, b_and, b_or, sh);
    // all band pages above kth, then the lowest ids among those equal to it
    int above = 0, zero = 0;
    for (int i = tid; i < n; i += NW * kWave)
      if (((band_bits[i >> 5] >> (i & 31)) & 1u) && keys64[i] > kth) {
        const int j = cand_lo + i;
        atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
        above++;
      }
    block_sum2(above, zero, sh);
    int take = need - above;
    for (int i0 = 0; i0 < n && take > 0; i0 += NW * kWave) {
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
  return false;
}

// The candidates whose key is >= uk, ascending, from slot base on (see
// emit_by_threshold); thread t takes candidates PER t .. PER t + PER-1 of a
// round of PER T; returns the slot after the last.
template <int NW, int PER, typename Put>
__device__ __forceinline__ int emit_keys_at_least(SelShared<NW> &sh, const uint32_t *keys32, int n, uint32_t uk,
                                                  int cand_lo, int base, Put put) {
  constexpr int T = NW * kWave;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  for (int i0 = 0; i0 < n; i0 += PER * T) {
    const int i = i0 + PER * tid;
    uint32_t kr[PER];
    load_key_chunks<PER>(kr, keys32, i, n);
    uint32_t m = 0;  // bit e: candidate i + e is selected
#pragma unroll
    for (int e = 0; e < PER; e++)
      if (i + e < n && kr[e] >= uk) m |= 1u << e;
    const int c = __popc(m);
    const int incl = wave_incl_sum(c);
    if (lane == kWave - 1) sh.red[wave][2] = incl;
    __syncthreads();
    int pos = base + incl - c, round = 0;
#pragma unroll
    for (int x = 0; x < NW; x++) {
      const int t = sh.red[x][2];
      if (x < wave) pos += t;
      round += t;
    }
    while (m) {
      const int e = __builtin_ctz(m);
      m &= m - 1;
      put(pos++, cand_lo + i + e);
    }
    base += round;
    if (i0 + PER * T < n) __syncthreads();  // sh.red is rewritten next round
  }
  return base;
}

// The ascending selection when select_candidates returned true: the sink
// pages [0, cand_lo), the candidates whose key is >= uk, the local pages
// [cand_hi, P).  Written to out_global (followed by -1 up to max_sel) and/or
// out_lds; returns the count.  The candidates are counted in rounds of
// keys_per_thread keys per thread (16-byte LDS loads); a wave prefix sum and
// the wave totals in LDS give their slots, so a round costs one barrier.  No
// bit map is built.  keys32 must be 16-byte aligned.
template <int NW>
__device__ int emit_by_threshold(SelShared<NW> &sh, const uint32_t *keys32, int n, uint32_t uk, int cand_lo,
                                 int cand_hi, int P, int32_t *out_global, int32_t *out_lds, int max_sel) {
  constexpr int T = NW * kWave;
  const int tid = threadIdx.x;
  auto put = [&](int pos, int j) {
    if (pos < max_sel) {
      if (out_global) out_global[pos] = j;
      if (out_lds) out_lds[pos] = j;
    }
  };
  for (int j = tid; j < cand_lo; j += T) put(j, j);  // sink pages
  const int per = keys_per_thread<T>(n);  // block-uniform
  const int base = per == 4    ? emit_keys_at_least<NW, 4>(sh, keys32, n, uk, cand_lo, cand_lo, put)
                   : per == 8 ? emit_keys_at_least<NW, 8>(sh, keys32, n, uk, cand_lo, cand_lo, put)
                              : emit_keys_at_least<NW, 16>(sh, keys32, n, uk, cand_lo, cand_lo, put);
  const int nloc = P - cand_hi;
  for (int x = tid; x < nloc; x += T) put(base + x, cand_hi + x);  // local pages
  const int count = min(base + nloc, max_sel);
  if (out_global)
    for (int x = count + tid; x < max_sel; x += T) out_global[x] = -1;
  return count;
}

// Writes the pages marked in sel_bits, in ascending order, to out_global
// (followed by -1 up to max_sel) and/or out_lds.  Returns the count.
// Each thread takes one bit word per round; a wave prefix sum and the wave
// totals in LDS give the word's first slot.
template <int NW>
__device__ int emit_selection(SelShared<NW> &sh, const uint32_t *sel_bits, int nwords, int32_t *out_global,
                              int32_t *out_lds, int max_sel) {
  constexpr int T = NW * kWave;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  int written = 0;
  for (int w0 = 0; w0 < nwords; w0 += T) {
    const int w = w0 + tid;
    const uint32_t bits = w < nwords ? sel_bits[w] : 0u;
    const int c = __popc(bits);
    const int incl = wave_incl_sum(c);
    if (lane == kWave - 1) sh.red[wave][2] = incl;
    __syncthreads();
    int pos = written + incl - c, round = 0;
#pragma unroll
    for (int x = 0; x < NW; x++) {
      const int t = sh.red[x][2];
      if (x < wave) pos += t;
      round += t;
    }
    uint32_t m = bits;
    while (m) {
      const int j = w * 32 + __builtin_ctz(m);
      m &= m - 1;
      if (pos < max_sel) {
        if (out_global) out_global[pos] = j;
        if (out_lds) out_lds[pos] = j;
      }
      pos++;
    }
    written += round;
    if (w0 + T < nwords) __syncthreads();  // sh.red is rewritten next round
  }
  const int count = min(written, max_sel);
  if (out_global)
    for (int i = count + tid; i < max_sel; i += T) out_global[i] = -1;
  return count;
}

// The whole selection of one (sequence, KV head) unit by one block of NW
// waves, from the unit's stored scores: candidate keys into LDS, the
// certified top-k (pages in doubt re-scored exactly), sink and local pages,
// or a static head's sink + window pages.  The list goes, ascending, to
// out_global (followed by -1 up to max_sel; may be null) and/or out_lds.
// Returns the count on every thread.  Every thread of the block calls it.
//   keys64  LDS, 8 bytes per page of max_pages (keys32 aliases it);
//   bits    LDS, 2 * nwords words (nwords = ceil(max_pages / 32));
//   row     the unit's scores, indexed by logical page;
//   qg      the group's first q row (global; may be null for static heads);
//   pt_row  the sequence's page-table row;
//   after_issue  called once by every thread right after its score loads are
//           issued (before any is waited for): loads the caller issues there
//           complete behind the scores, not ahead of them.
struct NoHook {
  __device__ void operator()() const {}
};
template <int D, int NW, typename AfterIssue = NoHook>
__device__ int select_unit(SelShared<NW> &sh, uint64_t *keys64, uint32_t *bits, int nwords, const qasp_score *row,
                           int L, int ps, bool is_static, int n_sink, int n_local, int top_k, int sink_tokens,
                           int window_tokens, const uint16_t *qg, int G, const uint16_t *summ, const int32_t *pt_row,
                           int Hkv, int g, int32_t *out_global, int32_t *out_lds, int max_sel,
                           AfterIssue after_issue = AfterIssue()) {
  constexpr int THREADS = NW * kWave;
  const int tid = threadIdx.x;
  uint32_t *keys32 = (uint32_t *)keys64;  // aliases keys64 until the band step
  uint32_t *sel_bits = bits;
  uint32_t *band_bits = bits + nwords;    // candidate index
  const int P = num_pages_of(L, ps);
  const int cand_lo = min(n_sink, P), cand_hi = max(cand_lo, P - n_local);
  const int n = cand_hi - cand_lo;
  const int k = top_k;
  const bool ranked = !is_static && k > 0 && k < n;

  // issue the score loads first: eight per thread in flight
  constexpr int kLoadUnroll = 8;
  const qasp_score *crow = row + cand_lo;
  float e_loc = 0.f;
  uint32_t k_min = ~0u, k_max = 0;
  // a round issues kLoadUnroll score loads per thread, then turns them into
  // keys; after_issue comes between the first round's two halves, at one
  // call site (the empty asm keeps the compiler from moving the caller's
  // loads ahead of the scores')
  qasp_score sc[kLoadUnroll];
  auto issue = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kLoadUnroll; u++) {
      const int i = i0 + u * THREADS + tid;
      sc[u] = i < n ? crow[i] : qasp_score{-INFINITY, 0.f, -1, 0};
    }
  };
  auto to_keys = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kLoadUnroll; u++) {
      const int i = i0 + u * THREADS + tid;
      if (i < n) {
        const uint32_t o = f32_order(sc[u].value);
        keys32[i] = o;
        k_min = min(k_min, o);
        k_max = max(k_max, o);
        e_loc = fmaxf(e_loc, sc[u].err);
      }
    }
  };
  if (ranked) issue(0);
  asm volatile("" ::: "memory");
  after_issue();
  if (ranked) {
    to_keys(0);
    for (int i0 = kLoadUnroll * THREADS; i0 < n; i0 += kLoadUnroll * THREADS) {
      issue(i0);
      to_keys(i0);
    }
  }
  for (int w = tid; w < nwords; w += THREADS) {
    sel_bits[w] = 0;
    band_bits[w] = 0;
  }
  for (int w = tid; w < NW * 256; w += THREADS) (&sh.hist[0][0])[w] = 0;
  if (tid == 0) sh.nlist = 0;
  __syncthreads();

  bool fast = false;
  uint32_t uk_fast = 0;
  if (is_static) {
    const int sink_end = min(sink_tokens, L);
    const int win_begin = max(0, L - window_tokens);
    for (int j = tid; j < P; j += THREADS) {
      const int a = j * ps, e = min(a + ps, L);
      if (a < sink_end || e > win_begin) atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
    }
  } else {
    if (ranked) {
      block_max_min_max(e_loc, k_min, k_max, sh);
      fast = select_candidates<D, NW>(sh, keys32, keys64, sel_bits, band_bits, n, k, cand_lo, e_loc, k_min, k_max,
                                      qg, G, summ, pt_row, Hkv, g, crow, nullptr, &uk_fast);
    }
    if (!fast)
      for (int j = tid; j < P; j += THREADS)
        if (j < cand_lo || j >= cand_hi || (!ranked && k > 0)) atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  // without pages in doubt the list comes straight from the keys
  return fast ? emit_by_threshold(sh, keys32, n, uk_fast, cand_lo, cand_hi, P, out_global, out_lds, max_sel)
              : emit_selection(sh, sel_bits, nwords, out_global, out_lds, max_sel);
}

}  // namespace sel
}  // namespace qasp
