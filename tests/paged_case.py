"""Small seeded paged-KV cases for the tests, built with numpy.

A case keeps each sequence's tokens in logical order (for the brute-force
references) and the same tokens placed into a paged pool at a seeded
permutation (for the oracle and the GPU library).  Only placement happens
here; no summaries, scores or attention.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from brute import bf16_bits_to_f64, f32_to_bf16_bits


@dataclass
class Case:
    num_pool_pages: int
    page_size: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    v_from_k: bool
    num_q_heads: int
    seq_lens: np.ndarray        # int32 [B]
    page_table: np.ndarray      # int32 [B][stride], spare page at index P_b
    q_bits: np.ndarray          # uint16 [B][Hq][Dk]
    k_pool: np.ndarray          # uint16 [pool][Hkv][ps][Dk]
    v_pool: Optional[np.ndarray]  # uint16 [pool][Hkv][Dv][ps]
    K: List[np.ndarray]         # per sequence fp64 [L][Hkv][Dk]
    V: List[np.ndarray]         # per sequence fp64 [L][Hkv][Dv]

    @property
    def q(self):
        return bf16_bits_to_f64(self.q_bits)

    @property
    def batch(self):
        return int(self.seq_lens.shape[0])

    def layout_args(self):
        return dict(num_pool_pages=self.num_pool_pages, page_size=self.page_size,
                    num_kv_heads=self.num_kv_heads, head_dim_k=self.head_dim_k,
                    head_dim_v=self.head_dim_v, v_from_k=self.v_from_k)


def _draw(rng, shape, values):
    if values == "normal":
        return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    if values == "int":
        return f32_to_bf16_bits(rng.integers(-3, 4, size=shape).astype(np.float32))
    if values == "zero":
        return np.zeros(shape, np.uint16)
    raise ValueError(values)


def make_case(seed, B, Hq, Hkv, Dk, Dv, ps, lens, v_from_k=False, values="normal",
              q_values=None, garbage=True, pool_extra=3, perm_seed=None, key_scale=None) -> Case:
    rng = np.random.default_rng(seed)
    lens = [int(L) for L in lens]
    pages = [(L + ps - 1) // ps for L in lens]
    used = sum(pages)
    pool = used + B + pool_extra
    prng = np.random.default_rng(seed + 7919 if perm_seed is None else perm_seed)
    perm = prng.permutation(pool).astype(np.int32)
    stride = max(pages + [0]) + 1
    pt = np.full((B, stride), -1, np.int32)
    off = 0
    for b in range(B):
        pt[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    for b in range(B):
        pt[b, pages[b]] = perm[used + b]

    k_pool = np.zeros((pool, Hkv, ps, Dk), np.uint16)
    v_pool = None if v_from_k else np.zeros((pool, Hkv, Dv, ps), np.uint16)
    if garbage:  # every slot gets something; slots past L must never be read
        k_pool[:] = f32_to_bf16_bits((rng.standard_normal(k_pool.shape) * 1e4).astype(np.float32))
        if v_pool is not None:
            v_pool[:] = f32_to_bf16_bits((rng.standard_normal(v_pool.shape) * 1e4).astype(np.float32))
    K, V = [], []
    for b in range(B):
        L = lens[b]
        kb = _draw(rng, (L, Hkv, Dk), values)
        if key_scale is not None:
            kb = f32_to_bf16_bits((bf16_bits_to_f64(kb) * key_scale).astype(np.float32))
        vb = kb[:, :, :Dv] if v_from_k else _draw(rng, (L, Hkv, Dv), values)
        for t in range(L):
            phys = pt[b, t // ps]
            k_pool[phys, :, t % ps, :] = kb[t]
            if not v_from_k:
                v_pool[phys, :, :, t % ps] = vb[t]
        K.append(bf16_bits_to_f64(kb))
        V.append(bf16_bits_to_f64(vb))
    q_bits = _draw(rng, (B, Hq, Dk), q_values or values)
    return Case(pool, ps, Hkv, Dk, Dv, v_from_k, Hq, np.asarray(lens, np.int32), pt, q_bits,
                k_pool, v_pool, K, V)
