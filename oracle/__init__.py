"""Python access to the plain CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing here is imported by the GPU
library, and this package imports nothing from it.

Inputs are numpy arrays: bf16 tensors as ``uint16`` bit patterns, indices as
``int32``.  Layouts are the ones documented in ``oracle.h``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

OK, ERR_ARG, ERR_MAX_SEL, ERR_RANGE = 0, -1, -2, -3


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (IEEE fp64, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < max(os.path.getmtime(_SRC),
                                           os.path.getmtime(os.path.join(_HERE, "oracle.h")))):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
            "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm",
        ])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Layout(ctypes.Structure):
    _fields_ = [("num_pool_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim_k", ctypes.c_int32),
                ("head_dim_v", ctypes.c_int32), ("v_from_k", ctypes.c_int32)]


class _Batch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("pt_stride", ctypes.c_int32), ("page_table", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p)]


class _Policy(ctypes.Structure):
    _fields_ = [("n_sink_pages", ctypes.c_int32), ("n_local_pages", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("sink_tokens", ctypes.c_int32),
                ("window_tokens", ctypes.c_int32), ("static_heads", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("QASP_ORACLE_LIB") or build()
        _lib = ctypes.CDLL(path)
        P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        sigs = {
            "orc_exact_sum": (D, [P, I64, P]),
            "orc_summaries": (I32, [P, P, P, P]),
            "orc_append": (I32, [P, P, P, P, P, P]),
            "orc_scores": (I32, [P, P, P, P, P, P, I32]),
            "orc_select": (I32, [P, P, P, P, I32, P, P, I32]),
            "orc_attend": (I32, [P, P, P, P, P, P, P, P, I32, D, P]),
            "orc_decode": (I32, [P, P, P, P, P, P, P, D, P, P, P, I32, I32]),
            "orc_max_sel": (I32, [P, P, I32]),
            "orc_quantize": (I32, [P, P, I32, P, P, P, P, P, P]),
            "orc_attend_quant": (I32, [P, P, P, I32, P, P, P, P, P, P, P, P, P, I32, D, P]),
            "orc_half_bits": (ctypes.c_uint16, [D]),
            "orc_scores_multi": (I32, [P, P, P, I32, P, P, P, I32]),
            "orc_select_multi": (I32, [P, P, P, I32, P, I32, P, P, I32]),
            "orc_attend_multi": (I32, [P, P, P, I32, P, P, P, P, P, I32, D, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(_lib, name)
            fn.restype, fn.argtypes = res, args
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


@dataclass
class Layout:
    num_pool_pages: int
    page_size: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    v_from_k: bool = False

    def c(self) -> _Layout:
        return _Layout(self.num_pool_pages, self.page_size, self.num_kv_heads,
                       self.head_dim_k, self.head_dim_v, int(self.v_from_k))


@dataclass
class Policy:
    n_sink_pages: int = 1
    n_local_pages: int = 1
    top_k: int = 1
    sink_tokens: int = 0
    window_tokens: int = 0
    static_heads: Optional[Sequence[int]] = None


class _Keep:
    """Holds the numpy buffers a ctypes struct points into."""

    def __init__(self):
        self.refs = []

    def arr(self, a, dtype):
        a = np.ascontiguousarray(a, dtype=dtype)
        self.refs.append(a)
        return a


def _batch(keep, page_table, seq_lens, num_q_heads):
    pt = keep.arr(page_table, np.int32)
    sl = keep.arr(seq_lens, np.int32)
    assert pt.ndim == 2 and sl.ndim == 1 and pt.shape[0] == sl.shape[0]
    return _Batch(sl.shape[0], num_q_heads, pt.shape[1], _ptr(pt), _ptr(sl))


def _policy(keep, pol: Policy):
    sh = None
    if pol.static_heads is not None:
        sh = keep.arr(np.asarray(pol.static_heads, dtype=np.uint8), np.uint8)
    return _Policy(pol.n_sink_pages, pol.n_local_pages, pol.top_k, pol.sink_tokens,
                   pol.window_tokens, _ptr(sh))


def _check(rc, what):
    if rc != OK:
        raise RuntimeError("oracle %s failed with status %d" % (what, rc))


def exact_sum(x) -> float:
    x = np.ascontiguousarray(x, dtype=np.float64)
    st = ctypes.c_int32(0)
    r = lib().orc_exact_sum(_ptr(x), x.size, ctypes.byref(st))
    _check(st.value, "exact_sum")
    return r


def max_sel(layout: Layout, pol: Policy, max_pages: int) -> int:
    keep = _Keep()
    return lib().orc_max_sel(ctypes.byref(layout.c()), ctypes.byref(_policy(keep, pol)), max_pages)


def summaries(layout: Layout, page_table, seq_lens, num_q_heads, k_pool, summ_pool=None):
    """Returns the summary pool with every referenced page-head filled in."""
    keep = _Keep()
    k = keep.arr(k_pool, np.uint16)
    if summ_pool is None:
        summ_pool = np.zeros((layout.num_pool_pages, layout.num_kv_heads, 2, layout.head_dim_k), np.uint16)
    s = np.ascontiguousarray(summ_pool, dtype=np.uint16).copy()
    bat = _batch(keep, page_table, seq_lens, num_q_heads)
    _check(lib().orc_summaries(ctypes.byref(layout.c()), ctypes.byref(bat), _ptr(k), _ptr(s)), "summaries")
    return s


def append(layout: Layout, page_table, seq_lens_before, num_q_heads, k_new, v_new, k_pool, v_pool):
    """Returns (k_pool, v_pool) copies with the new tokens written."""
    keep = _Keep()
    k = np.ascontiguousarray(k_pool, dtype=np.uint16).copy()
    v = None if v_pool is None else np.ascontiguousarray(v_pool, dtype=np.uint16).copy()
    kn = keep.arr(k_new, np.uint16)
    vn = None if v_new is None else keep.arr(v_new, np.uint16)
    bat = _batch(keep, page_table, seq_lens_before, num_q_heads)
    _check(lib().orc_append(ctypes.byref(layout.c()), ctypes.byref(bat), _ptr(kn), _ptr(vn),
                            _ptr(k), _ptr(v)), "append")
    return k, v


def scores(layout: Layout, page_table, seq_lens, q, summ_pool, pol: Policy, max_pages=None):
    keep = _Keep()
    qq = keep.arr(q, np.uint16)
    s = keep.arr(summ_pool, np.uint16)
    bat = _batch(keep, page_table, seq_lens, qq.shape[1])
    if max_pages is None:
        max_pages = np.asarray(page_table).shape[1]
    out = np.empty((bat.batch, layout.num_kv_heads, max_pages), np.float64)
    _check(lib().orc_scores(ctypes.byref(layout.c()), ctypes.byref(bat),
                            ctypes.byref(_policy(keep, pol)), _ptr(qq), _ptr(s), _ptr(out),
                            max_pages), "scores")
    return out


def select(layout: Layout, page_table, seq_lens, num_q_heads, scores_arr, pol: Policy, max_sel_n=None):
    keep = _Keep()
    sc = keep.arr(scores_arr, np.float64)
    bat = _batch(keep, page_table, seq_lens, num_q_heads)
    max_pages = sc.shape[2]
    if max_sel_n is None:
        max_sel_n = max_sel(layout, pol, max_pages)
    sel = np.empty((bat.batch, layout.num_kv_heads, max_sel_n), np.int32)
    cnt = np.empty((bat.batch, layout.num_kv_heads), np.int32)
    _check(lib().orc_select(ctypes.byref(layout.c()), ctypes.byref(bat),
                            ctypes.byref(_policy(keep, pol)), _ptr(sc), max_pages, _ptr(sel),
                            _ptr(cnt), max_sel_n), "select")
    return sel, cnt


def attend(layout: Layout, page_table, seq_lens, q, k_pool, v_pool, sel, cnt, pol: Policy, scale):
    keep = _Keep()
    qq = keep.arr(q, np.uint16)
    k = keep.arr(k_pool, np.uint16)
    v = None if v_pool is None else keep.arr(v_pool, np.uint16)
    se = keep.arr(sel, np.int32)
    cn = keep.arr(cnt, np.int32)
    bat = _batch(keep, page_table, seq_lens, qq.shape[1])
    out = np.empty((bat.batch, qq.shape[1], layout.head_dim_v), np.float64)
    _check(lib().orc_attend(ctypes.byref(layout.c()), ctypes.byref(bat),
                            ctypes.byref(_policy(keep, pol)), _ptr(qq), _ptr(k), _ptr(v),
                            _ptr(se), _ptr(cn), se.shape[2], float(scale), _ptr(out)), "attend")
    return out


def decode(layout: Layout, page_table, seq_lens, q, k_pool, v_pool, summ_pool, pol: Policy, scale,
           num_threads=1, max_sel_n=None):
    """Scores + selection + attention in one pass over precomputed summaries.
    Returns (out fp64 [B][Hq][Dv], sel [B][Hkv][max_sel], count [B][Hkv])."""
    keep = _Keep()
    qq = keep.arr(q, np.uint16)
    k = keep.arr(k_pool, np.uint16)
    v = None if v_pool is None else keep.arr(v_pool, np.uint16)
    s = None if summ_pool is None else keep.arr(summ_pool, np.uint16)
    bat = _batch(keep, page_table, seq_lens, qq.shape[1])
    if max_sel_n is None:
        max_sel_n = max_sel(layout, pol, np.asarray(page_table).shape[1])
    out = np.empty((bat.batch, qq.shape[1], layout.head_dim_v), np.float64)
    sel = np.empty((bat.batch, layout.num_kv_heads, max_sel_n), np.int32)
    cnt = np.empty((bat.batch, layout.num_kv_heads), np.int32)
    _check(lib().orc_decode(ctypes.byref(layout.c()), ctypes.byref(bat),
                            ctypes.byref(_policy(keep, pol)), _ptr(qq), _ptr(k), _ptr(v), _ptr(s),
                            float(scale), _ptr(out), _ptr(sel), _ptr(cnt), max_sel_n,
                            int(num_threads)), "decode")
    return out, sel, cnt


# Multi-query step: nq draft tokens per sequence at positions L - nq ... L - 1
# (seq_lens count them); q [B][nq][Hq][Dk], out [B][nq][Hq][Dv].  The readings
# are stated in oracle.h beside orc_scores_multi.

def max_sel_multi(layout: Layout, pol: Policy, nq: int, max_pages: int) -> int:
    """Selection capacity of a multi-query step (static heads read a window of
    window_tokens + nq - 1 tokens when window_tokens >= 1)."""
    wide = pol.window_tokens + nq - 1 if pol.window_tokens > 0 else 0
    return max_sel(layout, dataclasses.replace(pol, window_tokens=wide), max_pages)


def scores_multi(layout: Layout, page_table, seq_lens, q, summ_pool, pol: Policy, max_pages=None):
    keep = _Keep()
    qq = keep.arr(q, np.uint16)
    nq = qq.shape[1]
    s = keep.arr(summ_pool, np.uint16)
    bat = _batch(keep, page_table, seq_lens, qq.shape[2])
    if max_pages is None:
        max_pages = np.asarray(page_table).shape[1]
    out = np.empty((bat.batch, layout.num_kv_heads, max_pages), np.float64)
    _check(lib().orc_scores_multi(ctypes.byref(layout.c()), ctypes.byref(bat), ctypes.byref(_policy(keep, pol)),
                                  nq, _ptr(qq), _ptr(s), _ptr(out), max_pages), "scores_multi")
    return out


def select_multi(layout: Layout, page_table, seq_lens, num_q_heads, nq, scores_arr, pol: Policy, max_sel_n=None):
    keep = _Keep()
    sc = keep.arr(scores_arr, np.float64)
    bat = _batch(keep, page_table, seq_lens, num_q_heads)
    max_pages = sc.shape[2]
    if max_sel_n is None:
        max_sel_n = max_sel_multi(layout, pol, nq, max_pages)
    sel = np.empty((bat.batch, layout.num_kv_heads, max_sel_n), np.int32)
    cnt = np.empty((bat.batch, layout.num_kv_heads), np.int32)
    _check(lib().orc_select_multi(ctypes.byref(layout.c()), ctypes.byref(bat), ctypes.byref(_policy(keep, pol)),
                                  int(nq), _ptr(sc), max_pages, _ptr(sel), _ptr(cnt), max_sel_n), "select_multi")
    return sel, cnt


def attend_multi(layout: Layout, page_table, seq_lens, q, k_pool, v_pool, sel, cnt, pol: Policy, scale):
    keep = _Keep()
    qq = keep.arr(q, np.uint16)
    nq = qq.shape[1]
    k = keep.arr(k_pool, np.uint16)
    v = None if v_pool is None else keep.arr(v_pool, np.uint16)
    se = keep.arr(sel, np.int32)
    cn = keep.arr(cnt, np.int32)
    bat = _batch(keep, page_table, seq_lens, qq.shape[2])
    out = np.empty((bat.batch, nq, qq.shape[2], layout.head_dim_v), np.float64)
    _check(lib().orc_attend_multi(ctypes.byref(layout.c()), ctypes.byref(bat), ctypes.byref(_policy(keep, pol)),
                                  nq, _ptr(qq), _ptr(k), _ptr(v), _ptr(se), _ptr(cn), se.shape[2], float(scale),
                                  _ptr(out)), "attend_multi")
    return out


# 2-bit quantised pages (readings stated beside orc_quantize in the oracle's
# header): logical layouts, one byte per code, binary16 (m, s) pairs.

@dataclass
class Quant:
    residual_pages: int
    k_codes: np.ndarray   # uint8  [pool][Hkv][ps][Dk]
    k_meta: np.ndarray    # uint16 [pool][Hkv][ps][Dk/32][2]
    v_codes: np.ndarray   # uint8  [pool][Hkv][ps][Dv]
    v_meta: np.ndarray    # uint16 [pool][Hkv][ps][Dv/32][2]


def half_bits(x: float) -> int:
    return int(lib().orc_half_bits(float(x)))


def quantize(layout: Layout, page_table, seq_lens, num_q_heads, residual_pages, k_pool, v_pool) -> Quant:
    """Quantised pool with the page-heads of logical pages j < P - residual_pages filled (others zero)."""
    keep = _Keep()
    k = keep.arr(k_pool, np.uint16)
    v = keep.arr(v_pool, np.uint16)
    L = layout
    kc = np.zeros((L.num_pool_pages, L.num_kv_heads, L.page_size, L.head_dim_k), np.uint8)
    km = np.zeros((L.num_pool_pages, L.num_kv_heads, L.page_size, L.head_dim_k // 32, 2), np.uint16)
    vc = np.zeros((L.num_pool_pages, L.num_kv_heads, L.page_size, L.head_dim_v), np.uint8)
    vm = np.zeros((L.num_pool_pages, L.num_kv_heads, L.page_size, L.head_dim_v // 32, 2), np.uint16)
    bat = _batch(keep, page_table, seq_lens, num_q_heads)
    _check(lib().orc_quantize(ctypes.byref(L.c()), ctypes.byref(bat), int(residual_pages), _ptr(k), _ptr(v),
                              _ptr(kc), _ptr(km), _ptr(vc), _ptr(vm)), "quantize")
    return Quant(int(residual_pages), kc, km, vc, vm)


def attend_quant(layout: Layout, page_table, seq_lens, q, k_pool, v_pool, quant: Quant, sel, cnt, pol: Policy,
                 scale):
    keep = _Keep()
    qq = keep.arr(q, np.uint16)
    k = keep.arr(k_pool, np.uint16)
    v = keep.arr(v_pool, np.uint16)
    kc, km = keep.arr(quant.k_codes, np.uint8), keep.arr(quant.k_meta, np.uint16)
    vc, vm = keep.arr(quant.v_codes, np.uint8), keep.arr(quant.v_meta, np.uint16)
    se = keep.arr(sel, np.int32)
    cn = keep.arr(cnt, np.int32)
    bat = _batch(keep, page_table, seq_lens, qq.shape[1])
    out = np.empty((bat.batch, qq.shape[1], layout.head_dim_v), np.float64)
    _check(lib().orc_attend_quant(ctypes.byref(layout.c()), ctypes.byref(bat), ctypes.byref(_policy(keep, pol)),
                                  int(quant.residual_pages), _ptr(qq), _ptr(k), _ptr(v), _ptr(kc), _ptr(km),
                                  _ptr(vc), _ptr(vm), _ptr(se), _ptr(cn), se.shape[2], float(scale), _ptr(out)),
           "attend_quant")
    return out
