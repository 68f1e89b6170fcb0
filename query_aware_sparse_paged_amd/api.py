"""Thin ctypes binding of ``include/qasp.h`` (argument marshalling only).

Every function takes torch tensors that already live on the GPU, checks
their dtype, shape (against the layout, the batch and the selection
capacity) and contiguity, and passes raw device pointers plus the current
HIP stream to ``libqasp.so``.  All computation happens in the HIP kernels;
there is no CPU path, and a missing library raises ``RuntimeError``.
bf16 tensors are passed as their 16-bit patterns.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QASP_LIB may point at another build of the same library (e.g. a tuning build)
LIB_PATH = os.environ.get("QASP_LIB") or os.path.join(_HERE, "libqasp.so")

OK, ERR_NULL_ARG, ERR_BAD_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_MAX_SEL, ERR_LAUNCH, ERR_ALLOC = \
    0, -1, -2, -3, -4, -5, -6, -7
ERR_BAD_PAGE_TABLE, ERR_SCRATCH = -8, -9


class QaspError(RuntimeError):
    def __init__(self, what, status):
        super().__init__("%s failed: %s (%d)" % (what, status_string(status), status))
        self.status = status


class CLayout(ctypes.Structure):
    _fields_ = [("num_pool_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim_k", ctypes.c_int32),
                ("head_dim_v", ctypes.c_int32), ("v_from_k", ctypes.c_int32)]


class CBatch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("pt_stride", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p)]


class CPolicy(ctypes.Structure):
    _fields_ = [("n_sink_pages", ctypes.c_int32), ("n_local_pages", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("sink_tokens", ctypes.c_int32),
                ("window_tokens", ctypes.c_int32), ("static_head_mask", ctypes.c_uint64)]


EXPORTS = {
    # name: (restype, argtypes)
    "qasp_version": (ctypes.c_char_p, []),
    "qasp_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "qasp_max_sel": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]),
    "qasp_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p] * 3 + [ctypes.c_int32]),
    "qasp_build_summaries": (ctypes.c_int32, [ctypes.c_void_p] * 5),
    "qasp_append_kv": (ctypes.c_int32, [ctypes.c_void_p] * 9),
    "qasp_score_pages": (ctypes.c_int32, [ctypes.c_void_p] * 7),
    "qasp_select_topk": (ctypes.c_int32, [ctypes.c_void_p] * 8 + [ctypes.c_int32, ctypes.c_void_p]),
    "qasp_sparse_paged_decode": (ctypes.c_int32, [ctypes.c_void_p] * 8 + [ctypes.c_int32, ctypes.c_float,
                                                                           ctypes.c_void_p, ctypes.c_void_p,
                                                                           ctypes.c_size_t, ctypes.c_void_p]),
    "qasp_decode_step": (ctypes.c_int32, [ctypes.c_void_p] * 9 + [ctypes.c_float] + [ctypes.c_void_p] * 3 +
                         [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "qasp_scratch_bytes": (ctypes.c_size_t, []),
    "qasp_decode_step_path": (ctypes.c_int32, [ctypes.c_void_p] * 3 + [ctypes.c_int32]),
    "qasp_decode_step_noalloc": (ctypes.c_int32, [ctypes.c_void_p] * 9 + [ctypes.c_float] + [ctypes.c_void_p] * 3 +
                                 [ctypes.c_int32, ctypes.c_void_p]),
    "qasp_decode_step_reuse": (ctypes.c_int32, [ctypes.c_void_p] * 9 + [ctypes.c_float] + [ctypes.c_void_p] * 2 +
                               [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                ctypes.c_void_p]),
    "qasp_quant_pool_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "qasp_quantize_pages": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32] +
                            [ctypes.c_void_p] * 4),
    "qasp_decode_step_quant": (ctypes.c_int32, [ctypes.c_void_p] * 3 + [ctypes.c_int32] + [ctypes.c_void_p] * 7 +
                               [ctypes.c_float] + [ctypes.c_void_p] * 3 +
                               [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "qasp_check_batch": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32] + [ctypes.c_void_p] * 2 +
                         [ctypes.c_int32, ctypes.c_void_p]),
    "qasp_host_alloc": (ctypes.c_int32, [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "qasp_host_free": (ctypes.c_int32, [ctypes.c_void_p]),
    "qasp_max_sel_multi": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]),
    "qasp_workspace_bytes_multi": (ctypes.c_size_t, [ctypes.c_void_p] * 3 + [ctypes.c_int32, ctypes.c_int32]),
    "qasp_decode_step_multi": (ctypes.c_int32, [ctypes.c_void_p] * 3 + [ctypes.c_int32] + [ctypes.c_void_p] * 6 +
                               [ctypes.c_float] + [ctypes.c_void_p] * 3 +
                               [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
}

_lib = None


def lib():
    """Loads libqasp.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libqasp.so is not built (run __graft_entry__.build() or "
                               "python query_aware_sparse_paged_amd/build.py); there is no fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().qasp_status_string(int(status)).decode()


def version() -> str:
    return lib().qasp_version().decode()


@dataclass
class Layout:
    num_pool_pages: int
    page_size: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    v_from_k: bool = False

    def c(self) -> CLayout:
        return CLayout(self.num_pool_pages, self.page_size, self.num_kv_heads, self.head_dim_k,
                       self.head_dim_v, int(self.v_from_k))


@dataclass
class Policy:
    n_sink_pages: int = 1
    n_local_pages: int = 1
    top_k: int = 1
    sink_tokens: int = 0
    window_tokens: int = 0
    static_heads: Optional[Sequence[int]] = None

    def mask(self) -> int:
        m = 0
        for g, s in enumerate(self.static_heads or []):
            if s:
                m |= 1 << g
        return m

    def c(self) -> CPolicy:
        return CPolicy(self.n_sink_pages, self.n_local_pages, self.top_k, self.sink_tokens,
                       self.window_tokens, self.mask())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class AtLeast(int):
    """A dimension that may be larger than the given size (a pool's pages)."""


def _check_args(*specs, devices=True):
    """Each spec is (tensor or None, dtype, name, shape); a shape entry is an
    int (exact), AtLeast(n) or None (any).  First every dtype, shape and
    contiguity is checked, then (devices) that every tensor lives on the GPU
    (or is a host-tier view), so a wrong shape is reported before the device."""
    for t, dtype, name, shape in specs:
        if t is None:
            continue
        if t.dtype != dtype:
            raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
        have = tuple(t.shape)
        if len(have) != len(shape):
            raise ValueError("%s must have %d dims, got shape %s" % (name, len(shape), have))
        for d, (h, want) in enumerate(zip(have, shape)):
            if want is None:
                continue
            if isinstance(want, AtLeast):
                if h < int(want):
                    raise ValueError("%s: dim %d is %d, needs at least %d" % (name, d, h, int(want)))
            elif h != want:
                raise ValueError("%s must have shape %s, got %s" % (
                    name, tuple("*" if w is None else (">=%d" % int(w) if isinstance(w, AtLeast) else w)
                                for w in shape), have))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if not devices:
        return
    for t, _, name, _ in specs:
        if t is None or isinstance(t, MappedTensor):  # a host-tier pool
            continue
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)


def _pool_specs(layout: "Layout", k_pool, v_pool, summ):
    P, H, ps = AtLeast(layout.num_pool_pages), layout.num_kv_heads, layout.page_size
    return [(k_pool, torch.bfloat16, "k_pool", (P, H, ps, layout.head_dim_k)),
            (v_pool, torch.bfloat16, "v_pool", (P, H, layout.head_dim_v, ps)),
            (summ, torch.bfloat16, "summ", (P, H, 2, layout.head_dim_k))]


def _check(status, what):
    if status != OK:
        raise QaspError(what, status)


class Batch:
    """Page table + sequence lengths (device int32) and the host bound max_pages."""

    def __init__(self, page_table: torch.Tensor, seq_lens: torch.Tensor, num_q_heads: int,
                 max_pages: Optional[int] = None):
        if page_table is None or seq_lens is None:
            raise ValueError("page_table and seq_lens are required")
        _check_args((page_table, torch.int32, "page_table", (None, None)),
                    (seq_lens, torch.int32, "seq_lens", (page_table.shape[0],)), devices=False)
        self.page_table, self.seq_lens = page_table, seq_lens
        self.num_q_heads = int(num_q_heads)
        self.max_pages = int(page_table.shape[1] if max_pages is None else max_pages)
        if not 0 <= self.max_pages <= page_table.shape[1]:
            raise ValueError("max_pages must lie in [0, page_table.shape[1]]")

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    def specs(self):
        return [(self.page_table, torch.int32, "page_table", (self.batch, None)),
                (self.seq_lens, torch.int32, "seq_lens", (self.batch,))]

    def c(self) -> CBatch:
        return CBatch(int(self.seq_lens.shape[0]), self.num_q_heads, int(self.page_table.shape[1]),
                      self.max_pages, self.page_table.data_ptr(), self.seq_lens.data_ptr())


def max_sel(layout: Layout, policy: Policy, max_pages: int) -> int:
    r = lib().qasp_max_sel(ctypes.byref(layout.c()), ctypes.byref(policy.c()), int(max_pages))
    _check(0 if r >= 0 else r, "qasp_max_sel")
    return r


def workspace_bytes(layout: Layout, batch: Batch, policy: Policy, max_sel_n: int) -> int:
    return int(lib().qasp_workspace_bytes(ctypes.byref(layout.c()), ctypes.byref(batch.c()),
                                          ctypes.byref(policy.c()), int(max_sel_n)))


def new_workspace(layout: Layout, batch: Batch, policy: Policy, max_sel_n: int, device) -> torch.Tensor:
    """Workspace of qasp_workspace_bytes bytes (no initialisation needed)."""
    n = workspace_bytes(layout, batch, policy, max_sel_n)
    if n == 0:
        raise ValueError("invalid arguments for the workspace size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _u16(t):
    return t.view(torch.int16) if t is not None else None


def summary_rows(summ: torch.Tensor, phys) -> torch.Tensor:
    """The summary records of the physical pages phys (indices, or a boolean
    mask over the pool) in KV-head order, [n][Hkv][2][Dk]: in the pool the
    record of KV head g of page p sits in slot (g + p) mod Hkv of row p."""
    phys = torch.as_tensor(phys, device=summ.device)
    if phys.dtype == torch.bool:
        phys = phys.nonzero().flatten()
    phys = phys.to(torch.int64)
    hkv = summ.shape[1]
    slot = (torch.arange(hkv, device=summ.device)[None, :] + phys[:, None]) % hkv
    return summ[phys[:, None], slot]


def build_summaries(layout: Layout, batch: Batch, k_pool: torch.Tensor, summ: torch.Tensor):
    _check_args(*batch.specs(), *_pool_specs(layout, k_pool, None, summ))
    _check(lib().qasp_build_summaries(ctypes.byref(layout.c()), ctypes.byref(batch.c()), _ptr(k_pool),
                                      _ptr(summ), _stream()), "qasp_build_summaries")


def _token_specs(layout: Layout, B: int, k_new, v_new, n_query=None):
    lead = (B,) if n_query is None else (B, n_query)
    return [(k_new, torch.bfloat16, "k_new", lead + (layout.num_kv_heads, layout.head_dim_k)),
            (v_new, torch.bfloat16, "v_new", lead + (layout.num_kv_heads, layout.head_dim_v))]


def _query_specs(layout: Layout, batch: Batch, q, out, n_query=None):
    lead = (batch.batch,) if n_query is None else (batch.batch, n_query)
    return [(q, torch.bfloat16, "q", lead + (batch.num_q_heads, layout.head_dim_k)),
            (out, torch.float32, "out", lead + (batch.num_q_heads, layout.head_dim_v))]


def _sel_specs(layout: Layout, batch: Batch, sel, sel_count, max_sel_n=None):
    return [(sel, torch.int32, "sel", (batch.batch, layout.num_kv_heads, max_sel_n)),
            (sel_count, torch.int32, "sel_count", (batch.batch, layout.num_kv_heads))]


def _ws_spec(workspace):
    if workspace is None:
        raise ValueError("workspace is required")
    return (workspace, torch.uint8, "workspace", (None,))


def append_kv(layout: Layout, batch_before: Batch, policy: Policy, k_new, v_new, k_pool, v_pool, summ):
    _check_args(*batch_before.specs(), *_token_specs(layout, batch_before.batch, k_new, v_new),
                *_pool_specs(layout, k_pool, v_pool, summ))
    _check(lib().qasp_append_kv(ctypes.byref(layout.c()), ctypes.byref(batch_before.c()),
                                ctypes.byref(policy.c()), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                                _ptr(v_pool), _ptr(summ), _stream()), "qasp_append_kv")


def _score_spec(layout: Layout, batch: Batch, scores):
    return (scores, torch.float32, "scores", (batch.batch, layout.num_kv_heads, batch.max_pages, 4))


def score_pages(layout: Layout, batch: Batch, policy: Policy, q, summ, scores=None) -> torch.Tensor:
    """Returns float32 [B][Hkv][max_pages][4], one qasp_score per page: (fp32
    score, error bound, certified leading head, 0); the last two are int32 bit
    patterns (view the tensor as int32 to read them)."""
    if scores is None:
        scores = torch.empty((batch.batch, layout.num_kv_heads, batch.max_pages, 4), dtype=torch.float32,
                             device=batch.seq_lens.device)
    _check_args(*batch.specs(), *_query_specs(layout, batch, q, None), *_pool_specs(layout, None, None, summ),
                _score_spec(layout, batch, scores))
    _check(lib().qasp_score_pages(ctypes.byref(layout.c()), ctypes.byref(batch.c()), ctypes.byref(policy.c()),
                                  _ptr(q), _ptr(summ), _ptr(scores), _stream()), "qasp_score_pages")
    return scores


def select_topk(layout: Layout, batch: Batch, policy: Policy, q, summ, scores, max_sel_n=None, sel=None,
                sel_count=None):
    """Returns (sel int32 [B][Hkv][max_sel], sel_count int32 [B][Hkv])."""
    dev = batch.seq_lens.device
    if sel is not None:
        if max_sel_n is not None and int(max_sel_n) != sel.shape[-1]:
            raise ValueError("max_sel_n disagrees with sel's last dimension")
        max_sel_n = int(sel.shape[-1])
    if max_sel_n is None:
        max_sel_n = max_sel(layout, policy, batch.max_pages)
    if sel is None:
        sel = torch.empty((batch.batch, layout.num_kv_heads, max_sel_n), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((batch.batch, layout.num_kv_heads), dtype=torch.int32, device=dev)
    _check_args(*batch.specs(), *_sel_specs(layout, batch, sel, sel_count, max_sel_n),
                *_query_specs(layout, batch, q, None), *_pool_specs(layout, None, None, summ),
                _score_spec(layout, batch, scores))
    _check(lib().qasp_select_topk(ctypes.byref(layout.c()), ctypes.byref(batch.c()), ctypes.byref(policy.c()),
                                  _ptr(q), _ptr(summ), _ptr(scores), _ptr(sel), _ptr(sel_count), int(max_sel_n),
                                  _stream()), "qasp_select_topk")
    return sel, sel_count


def _new_out(layout: Layout, batch: Batch, q, n_query=None):
    lead = (batch.batch,) if n_query is None else (batch.batch, n_query)
    return torch.empty(lead + (batch.num_q_heads, layout.head_dim_v), dtype=torch.float32,
                       device=q.device if q is not None else batch.seq_lens.device)


def sparse_paged_decode(layout: Layout, batch: Batch, policy: Policy, q, k_pool, v_pool, sel, sel_count,
                        scale: float, workspace: torch.Tensor, out=None) -> torch.Tensor:
    """Returns float32 [B][Hq][Dv]."""
    if sel is None or sel_count is None:
        raise ValueError("sel and sel_count are required")
    out = _new_out(layout, batch, q) if out is None else out
    _check_args(*batch.specs(), *_query_specs(layout, batch, q, out), *_pool_specs(layout, k_pool, v_pool, None),
                *_sel_specs(layout, batch, sel, sel_count), _ws_spec(workspace))
    _check(lib().qasp_sparse_paged_decode(ctypes.byref(layout.c()), ctypes.byref(batch.c()),
                                          ctypes.byref(policy.c()), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                          _ptr(sel), _ptr(sel_count), int(sel.shape[2]), float(scale),
                                          _ptr(out), _ptr(workspace), workspace.numel(), _stream()),
           "qasp_sparse_paged_decode")
    return out


def _step_specs(layout: Layout, batch: Batch, q, out, k_pool, v_pool, summ, k_new, v_new, sel, sel_count,
                max_sel_n, workspace, n_query=None, with_workspace=True):
    if sel is not None and int(max_sel_n) != sel.shape[-1]:
        raise ValueError("max_sel_n (%d) disagrees with sel's last dimension (%d)" % (max_sel_n, sel.shape[-1]))
    specs = [*batch.specs(), *_query_specs(layout, batch, q, out, n_query), *_pool_specs(layout, k_pool, v_pool, summ),
             *_token_specs(layout, batch.batch, k_new, v_new, n_query),
             *_sel_specs(layout, batch, sel, sel_count, int(max_sel_n))]
    return specs + [_ws_spec(workspace)] if with_workspace else specs


def decode_step(layout: Layout, batch: Batch, policy: Policy, q, k_pool, v_pool, summ, scale: float,
                workspace: torch.Tensor, max_sel_n: int, k_new=None, v_new=None, out=None, sel=None,
                sel_count=None) -> torch.Tensor:
    """Append (if k_new is given; batch.seq_lens then counts the new token),
    score, select, attend and merge in one call.  Returns out fp32 [B][Hq][Dv]."""
    out = _new_out(layout, batch, q) if out is None else out
    _check_args(*_step_specs(layout, batch, q, out, k_pool, v_pool, summ, k_new, v_new, sel, sel_count, max_sel_n,
                             workspace))
    _check(lib().qasp_decode_step(ctypes.byref(layout.c()), ctypes.byref(batch.c()), ctypes.byref(policy.c()),
                                  _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(summ),
                                  float(scale), _ptr(out), _ptr(sel), _ptr(sel_count), int(max_sel_n),
                                  _ptr(workspace), workspace.numel(), _stream()), "qasp_decode_step")
    return out


PATH_ONE_KERNEL, PATH_CHAIN = 1, 2


def decode_step_path(layout: Layout, batch: Batch, policy: Policy, max_sel_n: int) -> int:
    """PATH_ONE_KERNEL or PATH_CHAIN: the kernels decode_step launches here."""
    r = lib().qasp_decode_step_path(ctypes.byref(layout.c()), ctypes.byref(batch.c()), ctypes.byref(policy.c()),
                                    int(max_sel_n))
    _check(0 if r >= 0 else r, "qasp_decode_step_path")
    return r


def scratch_bytes() -> int:
    """Size of the library's static per-device workspace (decode_step_noalloc)."""
    return int(lib().qasp_scratch_bytes())


def decode_step_noalloc(layout: Layout, batch: Batch, policy: Policy, q, k_pool, v_pool, summ, scale: float,
                        max_sel_n: int, k_new=None, v_new=None, out=None, sel=None, sel_count=None) -> torch.Tensor:
    """decode_step with the library's static per-device workspace instead of a
    caller's: the library call allocates nothing (out is allocated here when
    not given).  Calls that overlap in time on one GPU race."""
    out = _new_out(layout, batch, q) if out is None else out
    _check_args(*_step_specs(layout, batch, q, out, k_pool, v_pool, summ, k_new, v_new, sel, sel_count, max_sel_n,
                             None, with_workspace=False))
    _check(lib().qasp_decode_step_noalloc(ctypes.byref(layout.c()), ctypes.byref(batch.c()),
                                          ctypes.byref(policy.c()), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                                          _ptr(v_pool), _ptr(summ), float(scale), _ptr(out), _ptr(sel),
                                          _ptr(sel_count), int(max_sel_n), _stream()), "qasp_decode_step_noalloc")
    return out


def decode_step_reuse(layout: Layout, batch: Batch, policy: Policy, q, k_pool, v_pool, summ, scale: float,
                      sel, sel_count, workspace: torch.Tensor, k_new=None, v_new=None, out=None) -> torch.Tensor:
    """A layer that reuses an earlier layer's selection (sel, sel_count of
    that layer's decode_step at the same step): append (if k_new is given;
    batch.seq_lens then counts the new token) and attention over the given
    pages, no scoring or selection.  summ may be None.  Returns out fp32
    [B][Hq][Dv]."""
    if sel is None or sel_count is None:
        raise ValueError("sel and sel_count are required")
    out = _new_out(layout, batch, q) if out is None else out
    _check_args(*_step_specs(layout, batch, q, out, k_pool, v_pool, summ, k_new, v_new, sel, sel_count,
                             sel.shape[-1], workspace))
    _check(lib().qasp_decode_step_reuse(ctypes.byref(layout.c()), ctypes.byref(batch.c()), ctypes.byref(policy.c()),
                                        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(summ),
                                        float(scale), _ptr(sel), _ptr(sel_count), int(sel.shape[2]), _ptr(out),
                                        _ptr(workspace), workspace.numel(), _stream()), "qasp_decode_step_reuse")
    return out


def check_batch(layout: Layout, batch: Batch, extra_tokens: int = 0, sel=None, sel_count=None):
    """Runs qasp_check_batch (and waits for it): raises QaspError with status
    ERR_BAD_PAGE_TABLE when a length, page-table entry or selected id is out
    of range.  Validate mode (environment variable QASP_VALIDATE=1) runs the
    same check inside every call that reads the pools."""
    max_sel_n = 0 if sel is None else int(sel.shape[-1])
    if (sel is None) != (sel_count is None):
        raise ValueError("sel and sel_count come together")
    _check_args(*batch.specs(), *([] if sel is None else _sel_specs(layout, batch, sel, sel_count, max_sel_n)))
    _check(lib().qasp_check_batch(ctypes.byref(layout.c()), ctypes.byref(batch.c()), int(extra_tokens), _ptr(sel),
                                  _ptr(sel_count), max_sel_n, _stream()), "qasp_check_batch")


def layout_of(w) -> Layout:
    """Layout of a generated workload (query_aware_sparse_paged_amd.workloads)."""
    s = w.spec
    return Layout(w.num_pool_pages, s.page_size, s.num_kv_heads, s.head_dim_k, s.head_dim_v, s.v_from_k)


def policy_of(w) -> Policy:
    s = w.spec
    return Policy(s.n_sink_pages, s.n_local_pages, s.top_k, s.sink_tokens, s.window_tokens, s.static_heads)


def max_sel_multi(layout: Layout, policy: Policy, n_query: int, max_pages: int) -> int:
    r = lib().qasp_max_sel_multi(ctypes.byref(layout.c()), ctypes.byref(policy.c()), int(n_query), int(max_pages))
    _check(0 if r >= 0 else r, "qasp_max_sel_multi")
    return r


def new_workspace_multi(layout: Layout, batch: Batch, policy: Policy, n_query: int, max_sel_n: int,
                        device) -> torch.Tensor:
    """Workspace of qasp_workspace_bytes_multi bytes (no initialisation needed)."""
    n = int(lib().qasp_workspace_bytes_multi(ctypes.byref(layout.c()), ctypes.byref(batch.c()),
                                             ctypes.byref(policy.c()), int(n_query), int(max_sel_n)))
    if n == 0:
        raise ValueError("invalid arguments for the multi-query workspace size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode_step_multi(layout: Layout, batch: Batch, policy: Policy, q, k_pool, v_pool, summ, scale: float,
                      workspace: torch.Tensor, max_sel_n: int, k_new=None, v_new=None, out=None, sel=None,
                      sel_count=None) -> torch.Tensor:
    """n_query = q.shape[1] draft tokens per sequence (batch.seq_lens counts
    them): append them (if k_new is given, [B][n][Hkv][Dk]), select once per
    (sequence, KV head) for all drafts, attend causally.  q [B][n][Hq][Dk];
    returns out fp32 [B][n][Hq][Dv]."""
    if q is None or q.dim() != 4:
        raise ValueError("q must be [B][n_query][Hq][Dk]")
    n = int(q.shape[1])
    out = _new_out(layout, batch, q, n) if out is None else out
    _check_args(*_step_specs(layout, batch, q, out, k_pool, v_pool, summ, k_new, v_new, sel, sel_count, max_sel_n,
                             workspace, n))
    _check(lib().qasp_decode_step_multi(ctypes.byref(layout.c()), ctypes.byref(batch.c()), ctypes.byref(policy.c()),
                                        int(n), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                                        _ptr(summ), float(scale), _ptr(out), _ptr(sel), _ptr(sel_count),
                                        int(max_sel_n), _ptr(workspace), workspace.numel(), _stream()),
           "qasp_decode_step_multi")
    return out


class MappedTensor:
    """A contiguous array in host-tier memory (qasp_host_alloc): `host` is a
    CPU tensor over the memory (to fill or read it), data_ptr() the address
    the kernels use.  Pass it where a pool tensor is expected."""

    def __init__(self, buf: "HostBuffer", shape, dtype, offset: int = 0):
        self.buf, self.shape, self.dtype, self.offset = buf, tuple(shape), dtype, offset
        n = 1
        for x in self.shape:
            n *= x
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        if offset + nbytes > buf.nbytes:
            raise ValueError("view past the end of the host buffer")
        raw = (ctypes.c_uint8 * nbytes).from_address(buf.host_ptr + offset)
        self.host = torch.frombuffer(raw, dtype=torch.uint8).view(dtype).view(self.shape)

    def data_ptr(self) -> int:
        return self.buf.device_ptr + self.offset

    def dim(self) -> int:
        return len(self.shape)

    def is_contiguous(self) -> bool:
        return True


class HostBuffer:
    """Pinned host memory mapped into the current GPU's address space (a
    host-tier KV pool).  Freed by free() or when garbage-collected; no queued
    work may still use it then."""

    def __init__(self, nbytes: int):
        h, d = ctypes.c_void_p(), ctypes.c_void_p()
        _check(lib().qasp_host_alloc(int(nbytes), ctypes.byref(h), ctypes.byref(d)), "qasp_host_alloc")
        self.host_ptr, self.device_ptr, self.nbytes = h.value, d.value, int(nbytes)

    def view(self, shape, dtype=torch.bfloat16, offset: int = 0) -> MappedTensor:
        return MappedTensor(self, shape, dtype, offset)

    def free(self):
        if self.host_ptr:
            _check(lib().qasp_host_free(ctypes.c_void_p(self.host_ptr)), "qasp_host_free")
            self.host_ptr = self.device_ptr = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def host_pool_like(t: torch.Tensor) -> MappedTensor:
    """A host-tier copy of pool tensor t (same shape and dtype, contents copied)."""
    buf = HostBuffer(t.numel() * t.element_size())
    m = buf.view(t.shape, t.dtype)
    m.host.copy_(t.cpu() if t.is_cuda else t)
    return m


def new_quant_pool(layout: Layout, device) -> torch.Tensor:
    """Zeroed quantised pool of qasp_quant_pool_bytes bytes ([pool][Hkv][1536] uint8)."""
    n = int(lib().qasp_quant_pool_bytes(ctypes.byref(layout.c())))
    if n == 0:
        raise ValueError("quantised pages need a grouped-query layout (page 16, head_dim 128)")
    return torch.zeros((layout.num_pool_pages, layout.num_kv_heads, n // (layout.num_pool_pages *
                                                                         layout.num_kv_heads)),
                       dtype=torch.uint8, device=device)


def _qpool_spec(layout: Layout, qpool):
    per = int(lib().qasp_quant_pool_bytes(ctypes.byref(layout.c()))) // max(1, layout.num_pool_pages *
                                                                            layout.num_kv_heads)
    return (qpool, torch.uint8, "qpool", (AtLeast(layout.num_pool_pages), layout.num_kv_heads, per or None))


def quantize_pages(layout: Layout, batch: Batch, residual_pages: int, k_pool, v_pool, qpool):
    """Quantises every page below the last residual_pages of each sequence."""
    _check_args(*batch.specs(), *_pool_specs(layout, k_pool, v_pool, None), _qpool_spec(layout, qpool))
    _check(lib().qasp_quantize_pages(ctypes.byref(layout.c()), ctypes.byref(batch.c()), int(residual_pages),
                                     _ptr(k_pool), _ptr(v_pool), _ptr(qpool), _stream()), "qasp_quantize_pages")


def decode_step_quant(layout: Layout, batch: Batch, policy: Policy, residual_pages: int, q, k_pool, v_pool, summ,
                      qpool, scale: float, workspace: torch.Tensor, max_sel_n: int, k_new=None, v_new=None, out=None,
                      sel=None, sel_count=None) -> torch.Tensor:
    """decode_step with the pages below the last residual_pages read from the
    2-bit quantised pool.  Returns out fp32 [B][Hq][Dv]."""
    out = _new_out(layout, batch, q) if out is None else out
    _check_args(*_step_specs(layout, batch, q, out, k_pool, v_pool, summ, k_new, v_new, sel, sel_count, max_sel_n,
                             workspace), _qpool_spec(layout, qpool))
    _check(lib().qasp_decode_step_quant(ctypes.byref(layout.c()), ctypes.byref(batch.c()), ctypes.byref(policy.c()),
                                        int(residual_pages), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                                        _ptr(v_pool), _ptr(summ), _ptr(qpool), float(scale), _ptr(out), _ptr(sel),
                                        _ptr(sel_count), int(max_sel_n), _ptr(workspace), workspace.numel(),
                                        _stream()), "qasp_decode_step_quant")
    return out
