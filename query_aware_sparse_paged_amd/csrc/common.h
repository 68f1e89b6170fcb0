// Device-side helpers shared by the qasp kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "../../include/qasp.h"

namespace qasp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bf16 bit tricks
// ---------------------------------------------------------------------------

// Order-preserving signed key of a bf16 pattern: numeric order, -0 below +0.
// Negative patterns have their magnitude bits flipped so that a larger
// magnitude gives a smaller key.
__device__ __forceinline__ int bf16_order_key(uint32_t bits16) {
  int s = (int)(int16_t)(uint16_t)bits16;
  return s >= 0 ? s : (s ^ 0x7fff);
}
__device__ __forceinline__ uint32_t bf16_from_order_key(int key) {
  int s = key >= 0 ? key : (key ^ 0x7fff);
  return (uint32_t)(uint16_t)(int16_t)s;
}

// Two bf16 in a dword: keep each half whose sign bit is set / clear.
__device__ __forceinline__ uint32_t bf16x2_negative_part(uint32_t w) {
  uint32_t m = ((w & 0x80008000u) >> 15) * 0xffffu;
  return w & m;
}
__device__ __forceinline__ uint32_t bf16x2_positive_part(uint32_t w) {
  uint32_t m = ((w & 0x80008000u) >> 15) * 0xffffu;
  return w & ~m;
}
__device__ __forceinline__ uint32_t bf16x2_abs(uint32_t w) { return w & 0x7fff7fffu; }

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// MFMA wrappers (operands as raw dwords)
// ---------------------------------------------------------------------------

// D(16x16) += A(16x32) B(32x16), bf16 in, fp32 accumulate.  Lane l holds row
// (l % 16) of A and column (l % 16) of B, eight consecutive k each; the k
// blocks of lanes l and l' pair up when l / 16 == l' / 16.
__device__ __forceinline__ floatx4 mfma16x16x32(uint4 a, uint4 b, floatx4 c) {
  bf16x8 av = __builtin_bit_cast(bf16x8, a);
  bf16x8 bv = __builtin_bit_cast(bf16x8, b);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

// D(16x16) += A(16x16) B(16x16), bf16 in, fp32 accumulate, four k per lane.
// Output layout: lane l holds D[4 * (l / 16) + r][l % 16], r = 0..3.
__device__ __forceinline__ floatx4 mfma16x16x16(uint2 a, uint2 b, floatx4 c) {
  short4v av = __builtin_bit_cast(short4v, a);
  short4v bv = __builtin_bit_cast(short4v, b);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// wave reductions (wave64)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    int lo = __shfl_xor((int)(uint32_t)(uint64_t)v, o, kWave);
    int hi = __shfl_xor((int)(uint32_t)((uint64_t)v >> 32), o, kWave);
    v += (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
  }
  return v;
}

// ---------------------------------------------------------------------------
// DPP wave scans and reductions (GFX9 data-parallel primitives: row_shr
// within rows of 16 lanes, then row_bcast15 / row_bcast31 across rows).
// Each step is one VALU op with a DPP source, not a round trip through LDS.
// ---------------------------------------------------------------------------

constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_or(int identity, int x) {
  return __builtin_amdgcn_update_dpp(identity, x, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += dpp_or<kDppRowShr1>(0, x);
  x += dpp_or<kDppRowShr2>(0, x);
  x += dpp_or<kDppRowShr4>(0, x);
  x += dpp_or<kDppRowShr8>(0, x);
  x += dpp_or<kDppRowBcast15, 0xa>(0, x);
  x += dpp_or<kDppRowBcast31, 0xc>(0, x);
  return x;
}

// Sum / max over the wave, returned to every lane.
__device__ __forceinline__ int wave_sum_dpp(int x) {
  return __builtin_amdgcn_readlane(wave_incl_sum(x), 63);
}
__device__ __forceinline__ int wave_max_dpp(int x) {
  x = max(x, dpp_or<kDppRowShr1>(INT_MIN, x));
  x = max(x, dpp_or<kDppRowShr2>(INT_MIN, x));
  x = max(x, dpp_or<kDppRowShr4>(INT_MIN, x));
  x = max(x, dpp_or<kDppRowShr8>(INT_MIN, x));
  x = max(x, dpp_or<kDppRowBcast15, 0xa>(INT_MIN, x));
  x = max(x, dpp_or<kDppRowBcast31, 0xc>(INT_MIN, x));
  return __builtin_amdgcn_readlane(x, 63);
}
// max over floats without NaN: order-preserving int map, then integer max
__device__ __forceinline__ float wave_max_dpp(float f) {
  const int u = __float_as_int(f);
  const int key = u >= 0 ? u : (u ^ 0x7fffffff);
  const int m = wave_max_dpp(key);
  return __int_as_float(m >= 0 ? m : (m ^ 0x7fffffff));
}
__device__ __forceinline__ uint32_t wave_and_dpp(uint32_t x) {
  int v = (int)x;
  v &= dpp_or<kDppRowShr1>(-1, v);
  v &= dpp_or<kDppRowShr2>(-1, v);
  v &= dpp_or<kDppRowShr4>(-1, v);
  v &= dpp_or<kDppRowShr8>(-1, v);
  v &= dpp_or<kDppRowBcast15, 0xa>(-1, v);
  v &= dpp_or<kDppRowBcast31, 0xc>(-1, v);
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint32_t wave_or_dpp(uint32_t x) {
  int v = (int)x;
  v |= dpp_or<kDppRowShr1>(0, v);
  v |= dpp_or<kDppRowShr2>(0, v);
  v |= dpp_or<kDppRowShr4>(0, v);
  v |= dpp_or<kDppRowShr8>(0, v);
  v |= dpp_or<kDppRowBcast15, 0xa>(0, v);
  v |= dpp_or<kDppRowBcast31, 0xc>(0, v);
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}

// ---------------------------------------------------------------------------
// geometry
// ---------------------------------------------------------------------------

__device__ __forceinline__ int num_pages_of(int L, int ps) { return L <= 0 ? 0 : (L + ps - 1) / ps; }

// Work item of block `blk` (of `total`) when consecutive items should share
// an XCD: blocks are dealt to the 8 XCDs in turn (block b runs on XCD b % 8),
// so XCD x is given the contiguous items [x total / 8, (x + 1) total / 8).
// Identity when total is not a multiple of 8.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_contiguous_item(int blk, int total) {
  return total % kXcds == 0 ? (blk % kXcds) * (total / kXcds) + blk / kXcds : blk;
}

// Index of the summary record of KV head g of physical page phys in the
// summary pool, [pool][Hkv] records of [2][D] bf16 (lo row, hi row): the
// record sits in slot (g + phys) mod Hkv of the page's row.  Rotating the slot
// with the page spreads every head's records over all the slot offsets, so no
// head's reads fall on a fixed part of the address bits (with fixed slots the
// even heads' records sit at 1 KiB-aligned offsets and were read measurably
// slower than the odd heads').
__device__ __forceinline__ size_t summ_record(int phys, int g, int Hkv) {
  int slot = g + phys % Hkv;
  if (slot >= Hkv) slot -= Hkv;
  return (size_t)phys * Hkv + slot;
}

// The new token of a decode step, appended by one block for the KV heads
// [g0, g1) of sequence b: its key row and value column go into the page
// `phys` at slot t, and its key is folded into the page summary (slot 0
// starts it: elementwise min / max on bf16 order keys, -0 below +0).  The
// block's threads share the work (tid, nthreads); no synchronisation inside.
struct TokenAppend {
  const uint32_t *k_new;  // [B][Hkv][D / 2] bf16 pairs
  const uint16_t *v_new;  // [B][Hkv][Dv], or null (latent heads)
  uint32_t *k_pool;       // [pool][Hkv][ps][D / 2]
  uint16_t *v_pool;       // [pool][Hkv][Dv][ps], or null
  uint32_t *summ;         // [pool][Hkv][2][D / 2] (record slots: summ_record), or null
  int num_kv_heads, head_dim_k, head_dim_v, ps;

  __device__ void run(int b, int g0, int g1, int phys, int t, int tid, int nthreads) const {
    const int words = head_dim_k / 2;
    for (int item = tid; item < (g1 - g0) * words; item += nthreads) {
      const int g = g0 + item / words, w = item % words;
      const size_t ph = (size_t)phys * num_kv_heads + g;
      const uint32_t kv = k_new[((size_t)b * num_kv_heads + g) * words + w];
      k_pool[(ph * ps + t) * words + w] = kv;
      if (summ) {
        uint32_t *s = summ + summ_record(phys, g, num_kv_heads) * 2 * words;
        uint32_t lo = kv, hi = kv;
        if (t != 0) {
          const int v0 = bf16_order_key(kv & 0xffffu), v1 = bf16_order_key(kv >> 16);
          const uint32_t ol = s[w], oh = s[words + w];
          lo = bf16_from_order_key(min(v0, bf16_order_key(ol & 0xffffu))) |
               (bf16_from_order_key(min(v1, bf16_order_key(ol >> 16))) << 16);
          hi = bf16_from_order_key(max(v0, bf16_order_key(oh & 0xffffu))) |
               (bf16_from_order_key(max(v1, bf16_order_key(oh >> 16))) << 16);
        }
        s[w] = lo;
        s[words + w] = hi;
      }
    }
    if (v_pool)
      for (int item = tid; item < (g1 - g0) * head_dim_v; item += nthreads) {
        const int g = g0 + item / head_dim_v, dv = item % head_dim_v;
        const size_t ph = (size_t)phys * num_kv_heads + g;
        v_pool[(ph * head_dim_v + dv) * ps + t] = v_new[((size_t)b * num_kv_heads + g) * head_dim_v + dv];
      }
  }
};

__device__ __forceinline__ bool head_is_static(uint64_t mask, int g) {
  return (mask >> g) & 1ull;
}

// KV heads in dispatch order: the query-aware heads first, then the static
// ones.  Blocks start in index order as CUs free up, so when the units do not
// all fit on the chip at once the long (scored) units start first and the
// short static ones fill in behind them.  Returns the y-th head of that order.
__device__ __forceinline__ int head_in_dispatch_order(uint64_t static_mask, int Hkv, int y) {
  const uint64_t all = Hkv >= 64 ? ~0ull : ((1ull << Hkv) - 1);
  const uint64_t qa = all & ~static_mask, st = all & static_mask;
  const int n_qa = __popcll(qa);
  uint64_t m = y < n_qa ? qa : st;
  for (int r = y < n_qa ? y : y - n_qa; r > 0; r--) m &= m - 1;  // drop the r lowest set bits
  return __ffsll((long long)m) - 1;
}

}  // namespace qasp
