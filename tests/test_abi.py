"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before touching HIP."""
import ctypes
import os
import re

import pytest
import torch

from query_aware_sparse_paged_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "qasp.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qasp_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(api.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return api.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert "qasp_decode_step" in names and len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(api.EXPORTS)


def test_version_and_status_strings(L):
    assert re.match(r"^\d+\.\d+\.\d+$", api.version())
    for s in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert api.status_string(s) != "unknown status"
    assert "page-table" in api.status_string(api.ERR_BAD_PAGE_TABLE)
    assert api.status_string(-99) == "unknown status"


GQA = api.Layout(512, 16, 8, 128, 128)
MLA = api.Layout(64, 64, 1, 576, 512, True)


def _batch(B=1, Hq=32, stride=300, max_pages=256, pt=0x1000, sl=0x2000):
    return api.CBatch(B, Hq, stride, max_pages, pt, sl)


def _call(fn, *args):
    return getattr(api.lib(), fn)(*args)


def test_null_and_shape_errors(L):
    b = ctypes.byref
    lay, pol = GQA.c(), api.Policy(1, 4, 32).c()
    bat = _batch()
    assert _call("qasp_build_summaries", None, b(bat), 1, 1, None) == api.ERR_NULL_ARG
    assert _call("qasp_build_summaries", b(lay), None, 1, 1, None) == api.ERR_NULL_ARG
    assert _call("qasp_build_summaries", b(lay), b(bat), None, 1, None) == api.ERR_NULL_ARG
    bad = api.CLayout(0, 16, 8, 128, 128, 0)
    assert _call("qasp_build_summaries", b(bad), b(bat), 1, 1, None) == api.ERR_BAD_SHAPE
    for shape in [(512, 32, 8, 128, 128, 0), (512, 16, 8, 64, 64, 0), (512, 64, 1, 576, 512, 0),
                  (512, 16, 80, 128, 128, 0)]:
        assert _call("qasp_build_summaries", b(api.CLayout(*shape)), b(bat), 1, 1, None) == api.ERR_UNSUPPORTED
    assert _call("qasp_score_pages", b(lay), b(_batch(Hq=30)), b(pol), 1, 1, 1, None) == api.ERR_BAD_SHAPE
    assert _call("qasp_score_pages", b(lay), b(_batch(Hq=8 * 17)), b(pol), 1, 1, 1, None) == api.ERR_UNSUPPORTED
    assert _call("qasp_score_pages", b(lay), b(_batch(stride=100)), b(pol), 1, 1, 1, None) == api.ERR_BAD_SHAPE
    assert _call("qasp_score_pages", b(lay), b(_batch(max_pages=20000, stride=20000)), b(pol), 1, 1, 1,
                 None) == api.ERR_UNSUPPORTED
    neg = api.Policy(1, -1, 3).c()
    assert _call("qasp_score_pages", b(lay), b(bat), b(neg), 1, 1, 1, None) == api.ERR_BAD_SHAPE
    stray = api.CPolicy(1, 1, 3, 0, 0, 1 << 9)   # static bit beyond the 8 KV heads
    assert _call("qasp_score_pages", b(lay), b(bat), b(stray), 1, 1, 1, None) == api.ERR_BAD_SHAPE
    assert _call("qasp_score_pages", b(lay), b(bat), b(pol), None, 1, 1, None) == api.ERR_NULL_ARG
    # MLA needs 128 q heads per latent head
    assert _call("qasp_score_pages", b(MLA.c()), b(_batch(Hq=64)), b(pol), 1, 1, 1, None) == api.ERR_UNSUPPORTED
    # and exactly one latent KV head
    mla2 = api.CLayout(64, 64, 2, 576, 512, 1)
    assert _call("qasp_score_pages", b(mla2), b(_batch(Hq=256)), b(pol), 1, 1, 1, None) == api.ERR_UNSUPPORTED


def test_max_sel_and_workspace_checks(L):
    b = ctypes.byref
    lay = GQA.c()
    pol = api.Policy(1, 4, 32)
    assert api.max_sel(GQA, pol, 256) == 37
    assert api.max_sel(GQA, pol, 20) == 20
    assert api.max_sel(GQA, api.Policy(1, 8, 55, 4, 1024, [1, 1, 1, 1, 0, 0, 0, 0]), 4097) == 66
    bat = _batch()
    # select with max_sel below the bound
    assert _call("qasp_select_topk", b(lay), b(bat), b(pol.c()), 1, 1, 1, 1, 1, 36, None) == api.ERR_MAX_SEL
    assert _call("qasp_decode_step", b(lay), b(bat), b(pol.c()), 1, None, None, 1, 1, 1, 1.0, 1, None, None,
                 36, 1, 1 << 30, None) == api.ERR_MAX_SEL
    need = _call("qasp_workspace_bytes", b(lay), b(bat), b(pol.c()), 37)
    assert need > 0
    assert _call("qasp_sparse_paged_decode", b(lay), b(bat), b(pol.c()), 1, 1, 1, 1, 1, 37, 1.0, 1, 1,
                 need - 1, None) == api.ERR_WORKSPACE
    assert _call("qasp_decode_step", b(lay), b(bat), b(pol.c()), 1, None, None, 1, 1, 1, 1.0, 1, None, None,
                 37, 1, need - 1, None) == api.ERR_WORKSPACE
    # sel and sel_count come together
    assert _call("qasp_decode_step", b(lay), b(bat), b(pol.c()), 1, None, None, 1, 1, 1, 1.0, 1, 1, None,
                 37, 1, need, None) == api.ERR_NULL_ARG
    assert _call("qasp_workspace_bytes", None, b(bat), b(pol.c()), 37) == 0


def test_static_only_heads_need_no_summaries(L):
    b = ctypes.byref
    lay = GQA.c()
    pol = api.Policy(0, 0, 0, 4, 64, [1] * 8).c()
    # empty batch: valid and returns before any launch, even with NULL summaries
    empty = _batch(B=0)
    assert _call("qasp_decode_step", b(lay), b(empty), b(pol), 1, None, None, 1, 1, None, 1.0, 1, None, None,
                 6, 1, 1 << 20, None) == api.OK
    qa = api.Policy(1, 1, 1).c()
    assert _call("qasp_decode_step", b(lay), b(_batch()), b(qa), 1, None, None, 1, 1, None, 1.0, 1, None,
                 None, 256, 1, 1 << 30, None) == api.ERR_NULL_ARG
    assert _call("qasp_append_kv", b(lay), b(_batch()), b(qa), 1, 1, 1, 1, None, None) == api.ERR_NULL_ARG


def test_empty_batch_is_a_no_op(L):
    b = ctypes.byref
    lay, pol = GQA.c(), api.Policy(1, 4, 32).c()
    empty = _batch(B=0)
    assert _call("qasp_build_summaries", b(lay), b(empty), None, None, None) == api.OK
    assert _call("qasp_score_pages", b(lay), b(empty), b(pol), None, None, None, None) == api.OK
    assert _call("qasp_select_topk", b(lay), b(empty), b(pol), None, None, None, None, None, 37, None) == api.OK
    assert _call("qasp_sparse_paged_decode", b(lay), b(empty), b(pol), None, None, None, None, None, 37, 1.0,
                 None, None, 0, None) == api.OK


def test_reuse_step_argument_checks(L):
    """qasp_decode_step_reuse: the given selection is required, summaries are
    not; the workspace bound and the empty batch behave as in decode_step."""
    b = ctypes.byref
    lay, pol = GQA.c(), api.Policy(1, 4, 32).c()
    bat = _batch()
    need = _call("qasp_workspace_bytes", b(lay), b(bat), b(pol), 37)
    # (lay, bat, pol, q, k_new, v_new, k_pool, v_pool, summ, scale, sel, sel_count, max_sel, out, ws, bytes, stream)
    args = lambda **kw: [kw.get(k, v) for k, v in (("q", 1), ("k_new", None), ("v_new", None), ("k_pool", 1),
                                                    ("v_pool", 1), ("summ", None), ("scale", 1.0), ("sel", 1),
                                                    ("sel_count", 1), ("max_sel", 37), ("out", 1), ("ws", 1),
                                                    ("bytes", need), ("stream", None))]
    call = lambda lay_=lay, bat_=bat, **kw: _call("qasp_decode_step_reuse", b(lay_), b(bat_), b(pol), *args(**kw))
    assert call(sel=None) == api.ERR_NULL_ARG
    assert call(sel_count=None) == api.ERR_NULL_ARG
    assert call(q=None) == api.ERR_NULL_ARG
    assert call(out=None) == api.ERR_NULL_ARG
    assert call(v_pool=None) == api.ERR_NULL_ARG
    assert call(k_new=1, v_new=None) == api.ERR_NULL_ARG   # a value row goes with the key row
    assert call(bytes=need - 1) == api.ERR_WORKSPACE
    assert call(max_sel=-1) == api.ERR_BAD_SHAPE
    assert call(bat_=_batch(Hq=30)) == api.ERR_BAD_SHAPE
    # no launch for an empty batch, whatever the pointers
    assert _call("qasp_decode_step_reuse", b(lay), b(_batch(B=0)), b(pol), None, None, None, None, None, None, 1.0,
                 None, None, 37, None, None, 0, None) == api.OK


def test_multi_step_argument_checks(L):
    """qasp_decode_step_multi: draft count limits, the widened selection
    capacity of static heads, the multi-query workspace, null arguments."""
    b = ctypes.byref
    lay, pol = GQA.c(), api.Policy(1, 4, 32).c()
    bat = _batch(Hq=32)   # 8 KV heads: 4 heads per group, so at most 4 drafts
    ms = _call("qasp_max_sel_multi", b(lay), b(pol), 4, 256)
    assert ms == 37
    need = _call("qasp_workspace_bytes_multi", b(lay), b(bat), b(pol), 4, ms)
    assert need > _call("qasp_workspace_bytes", b(lay), b(bat), b(pol), ms)
    # (lay, bat, pol, n, q, k_new, v_new, k_pool, v_pool, summ, scale, out, sel, cnt, max_sel, ws, bytes, stream)
    args = lambda **kw: [kw.get(k, v) for k, v in (("n", 4), ("q", 1), ("k_new", None), ("v_new", None),
                                                    ("k_pool", 1), ("v_pool", 1), ("summ", 1), ("scale", 1.0),
                                                    ("out", 1), ("sel", None), ("cnt", None), ("max_sel", ms),
                                                    ("ws", 1), ("bytes", need), ("stream", None))]
    call = lambda lay_=lay, bat_=bat, pol_=pol, **kw: _call("qasp_decode_step_multi", b(lay_), b(bat_), b(pol_),
                                                            *args(**kw))
    assert call(n=0) == api.ERR_BAD_SHAPE
    assert call(n=5) == api.ERR_UNSUPPORTED          # 5 drafts x 4 heads > 16 columns
    assert call(n=17) == api.ERR_UNSUPPORTED
    assert call(lay_=MLA.c(), bat_=_batch(Hq=128)) == api.ERR_UNSUPPORTED
    assert call(q=None) == api.ERR_NULL_ARG
    assert call(summ=None) == api.ERR_NULL_ARG
    assert call(out=None) == api.ERR_NULL_ARG
    assert call(v_pool=None) == api.ERR_NULL_ARG
    assert call(k_new=1, v_new=None) == api.ERR_NULL_ARG
    assert call(sel=1, cnt=None) == api.ERR_NULL_ARG
    assert call(bytes=need - 1) == api.ERR_WORKSPACE
    assert call(max_sel=-1) == api.ERR_BAD_SHAPE
    # static heads: the drafts' windows widen the page set (window 32 + 3 tokens: up to 4 pages of 16)
    spol = api.Policy(0, 0, 0, sink_tokens=4, window_tokens=32, static_heads=[1] * 8).c()
    assert _call("qasp_max_sel", b(lay), b(spol), 256) == 4
    assert _call("qasp_max_sel_multi", b(lay), b(spol), 4, 256) == 5
    need_s = _call("qasp_workspace_bytes_multi", b(lay), b(bat), b(spol), 4, 5)
    assert call(pol_=spol, max_sel=4, bytes=need_s) == api.ERR_MAX_SEL
    # no launch for an empty batch, whatever the pointers
    assert _call("qasp_decode_step_multi", b(lay), b(_batch(B=0)), b(pol), 2, None, None, None, None, None, None,
                 1.0, None, None, None, ms, None, 0, None) == api.OK


def test_host_tier_allocation_argument_checks(L):
    """qasp_host_alloc / qasp_host_free: argument errors come before any HIP
    call (here, without a GPU, a valid request reports QASP_ERR_ALLOC with both
    pointers cleared)."""
    h, d = ctypes.c_void_p(1), ctypes.c_void_p(1)
    assert _call("qasp_host_alloc", 1024, None, ctypes.byref(d)) == api.ERR_NULL_ARG
    assert _call("qasp_host_alloc", 1024, ctypes.byref(h), None) == api.ERR_NULL_ARG
    assert _call("qasp_host_alloc", 0, ctypes.byref(h), ctypes.byref(d)) == api.ERR_BAD_SHAPE
    assert h.value is None and d.value is None
    assert _call("qasp_host_free", None) == api.ERR_NULL_ARG
    import torch
    if not torch.cuda.is_available():
        h, d = ctypes.c_void_p(1), ctypes.c_void_p(1)
        assert _call("qasp_host_alloc", 1024, ctypes.byref(h), ctypes.byref(d)) == api.ERR_ALLOC
        assert h.value is None and d.value is None


def test_quant_step_argument_checks(L):
    """Quantised pages: grouped-query layouts only, residual_pages >= 1, the
    pool size, null arguments."""
    b = ctypes.byref
    lay, pol = GQA.c(), api.Policy(1, 4, 32).c()
    bat = _batch()
    assert _call("qasp_quant_pool_bytes", b(lay)) == 512 * 8 * 1536
    assert _call("qasp_quant_pool_bytes", b(MLA.c())) == 0
    assert _call("qasp_quantize_pages", b(lay), b(bat), 0, 1, 1, 1, None) == api.ERR_BAD_SHAPE
    assert _call("qasp_quantize_pages", b(lay), b(bat), 1, 1, None, 1, None) == api.ERR_NULL_ARG
    assert _call("qasp_quantize_pages", b(MLA.c()), b(_batch(Hq=128)), 1, 1, 1, 1, None) == api.ERR_UNSUPPORTED
    need = _call("qasp_workspace_bytes", b(lay), b(bat), b(pol), 37)
    # (lay, bat, pol, R, q, k_new, v_new, k_pool, v_pool, summ, qpool, scale, out, sel, cnt, max_sel, ws, bytes, st)
    args = lambda **kw: [kw.get(k, v) for k, v in (("R", 2), ("q", 1), ("k_new", None), ("v_new", None),
                                                    ("k_pool", 1), ("v_pool", 1), ("summ", 1), ("qpool", 1),
                                                    ("scale", 1.0), ("out", 1), ("sel", None), ("cnt", None),
                                                    ("max_sel", 37), ("ws", 1), ("bytes", need), ("stream", None))]
    call = lambda lay_=lay, bat_=bat, **kw: _call("qasp_decode_step_quant", b(lay_), b(bat_), b(pol), *args(**kw))
    assert call(R=0) == api.ERR_BAD_SHAPE
    assert call(qpool=None) == api.ERR_NULL_ARG
    assert call(summ=None) == api.ERR_NULL_ARG
    assert call(v_pool=None) == api.ERR_NULL_ARG
    assert call(k_new=1, v_new=None) == api.ERR_NULL_ARG
    assert call(bytes=need - 1) == api.ERR_WORKSPACE
    assert call(max_sel=36) == api.ERR_MAX_SEL
    assert call(lay_=MLA.c(), bat_=_batch(Hq=128)) == api.ERR_UNSUPPORTED
    assert _call("qasp_decode_step_quant", b(lay), b(_batch(B=0)), b(pol), 1, None, None, None, None, None, None,
                 None, 1.0, None, None, None, 37, None, 0, None) == api.OK


# ----------------------------------------------------------------------------
# the Python binding's shape checks (run before any device check, so CPU
# tensors of the wrong shape are reported by name)
# ----------------------------------------------------------------------------

def _cpu_args(B=2, Hq=32, max_sel_n=37, nq=None):
    import torch
    lay = api.Layout(64, 16, 8, 128, 128)
    pt = torch.zeros((B, 10), dtype=torch.int32)
    bat = api.Batch(pt, torch.full((B,), 100, dtype=torch.int32), Hq, max_pages=9)
    lead = (B,) if nq is None else (B, nq)
    bf = torch.bfloat16
    a = dict(
        q=torch.zeros(lead + (Hq, 128), dtype=bf),
        out=torch.zeros(lead + (Hq, 128), dtype=torch.float32),
        k_pool=torch.zeros((64, 8, 16, 128), dtype=bf),
        v_pool=torch.zeros((64, 8, 128, 16), dtype=bf),
        summ=torch.zeros((64, 8, 2, 128), dtype=bf),
        k_new=torch.zeros(lead + (8, 128), dtype=bf),
        v_new=torch.zeros(lead + (8, 128), dtype=bf),
        sel=torch.zeros((B, 8, max_sel_n), dtype=torch.int32),
        sel_count=torch.zeros((B, 8), dtype=torch.int32),
        workspace=torch.zeros(16, dtype=torch.uint8),
    )
    return lay, bat, api.Policy(1, 4, 32), a


def _raises(fn, match):
    with pytest.raises((ValueError, TypeError), match=match):
        fn()


def test_binding_rejects_wrong_shapes(L):
    import torch
    lay, bat, pol, a = _cpu_args()

    def step(**kw):
        x = dict(a, **kw)
        return lambda: api.decode_step(lay, bat, pol, x["q"], x["k_pool"], x["v_pool"], x["summ"], 0.1,
                                       x["workspace"], 37, k_new=x["k_new"], v_new=x["v_new"], out=x["out"],
                                       sel=x["sel"], sel_count=x["sel_count"])

    # every argument right: the first complaint is the device
    _raises(step(), "GPU tensor")
    bf = torch.bfloat16
    wrong = dict(
        q=torch.zeros((2, 31, 128), dtype=bf),                  # heads
        out=torch.zeros((3, 32, 128), dtype=torch.float32),      # batch
        k_pool=torch.zeros((63, 8, 16, 128), dtype=bf),          # fewer pages than the layout
        v_pool=torch.zeros((64, 8, 16, 128), dtype=bf),          # untransposed value tile
        summ=torch.zeros((64, 8, 1, 128), dtype=bf),
        k_new=torch.zeros((2, 4, 128), dtype=bf),
        v_new=torch.zeros((2, 8, 64), dtype=bf),
        sel=torch.zeros((2, 8, 36), dtype=torch.int32),          # capacity disagrees with max_sel_n
        sel_count=torch.zeros((2, 7), dtype=torch.int32),
    )
    for name, t in wrong.items():
        _raises(step(**{name: t}), name if name != "sel" else "max_sel_n|sel")
    _raises(step(q=a["q"].float()), "q must be")
    _raises(step(out=torch.zeros((2, 128, 32), dtype=torch.float32).transpose(1, 2)), "out must be contiguous")
    # larger pools than the layout declares are fine (the device check comes next)
    _raises(step(k_pool=torch.zeros((65, 8, 16, 128), dtype=bf)), "GPU tensor")


def test_binding_shape_checks_of_the_other_calls(L):
    import torch
    lay, bat, pol, a = _cpu_args()
    bf = torch.bfloat16
    bad_scores = torch.zeros((2, 8, 8, 4), dtype=torch.float32)   # max_pages is 9
    _raises(lambda: api.score_pages(lay, bat, pol, a["q"], a["summ"], scores=bad_scores), "scores")
    _raises(lambda: api.select_topk(lay, bat, pol, a["q"], a["summ"], bad_scores), "scores")
    good_scores = torch.zeros((2, 8, 9, 4), dtype=torch.float32)
    _raises(lambda: api.select_topk(lay, bat, pol, a["q"], a["summ"], good_scores, max_sel_n=40, sel=a["sel"]),
            "max_sel_n")
    _raises(lambda: api.sparse_paged_decode(lay, bat, pol, a["q"], a["k_pool"], a["v_pool"], a["sel"],
                                            torch.zeros((2,), dtype=torch.int32), 0.1, a["workspace"]), "sel_count")
    _raises(lambda: api.decode_step_reuse(lay, bat, pol, a["q"], a["k_pool"], a["v_pool"], None, 0.1,
                                          a["sel"][:1], a["sel_count"], a["workspace"]), "sel")
    _raises(lambda: api.build_summaries(lay, bat, a["k_pool"], torch.zeros((64, 8, 2, 64), dtype=bf)), "summ")
    _raises(lambda: api.append_kv(lay, bat, pol, a["k_new"][:1], a["v_new"], a["k_pool"], a["v_pool"],
                                  a["summ"]), "k_new")
    q4 = torch.zeros((64, 8, 1000), dtype=torch.uint8)
    _raises(lambda: api.quantize_pages(lay, bat, 2, a["k_pool"], a["v_pool"], q4), "qpool")
    _raises(lambda: api.decode_step_quant(lay, bat, pol, 2, a["q"], a["k_pool"], a["v_pool"], a["summ"],
                                          torch.zeros((63, 8, 1536), dtype=torch.uint8), 0.1, a["workspace"], 37),
            "qpool")
    # multi-query: [B][n] leading dimensions
    lay, bat, pol, m = _cpu_args(nq=3, max_sel_n=40)
    _raises(lambda: api.decode_step_multi(lay, bat, pol, m["q"], m["k_pool"], m["v_pool"], m["summ"], 0.1,
                                          m["workspace"], 40, k_new=m["k_new"][:, :2], v_new=m["v_new"]), "k_new")
    _raises(lambda: api.decode_step_multi(lay, bat, pol, m["q"], m["k_pool"], m["v_pool"], m["summ"], 0.1,
                                          m["workspace"], 40, out=torch.zeros((2, 32, 128))), "out")
    _raises(lambda: api.decode_step_multi(lay, bat, pol, m["q"], m["k_pool"], m["v_pool"], m["summ"], 0.1,
                                          m["workspace"], 40, k_new=m["k_new"], v_new=m["v_new"]), "GPU tensor")
    # the batch itself
    _raises(lambda: api.Batch(torch.zeros((2, 10), dtype=torch.int32), torch.zeros((3,), dtype=torch.int32), 32),
            "seq_lens")
    _raises(lambda: api.Batch(torch.zeros((2, 10), dtype=torch.int64), torch.zeros((2,), dtype=torch.int32), 32),
            "page_table")
    _raises(lambda: api.Batch(torch.zeros((2, 10), dtype=torch.int32), torch.zeros((2,), dtype=torch.int32), 32,
                              max_pages=11), "max_pages")


def test_check_batch_host_errors(L):
    """qasp_check_batch's host-side argument errors come before any HIP call."""
    b = ctypes.byref
    lay, bat = GQA.c(), _batch()
    assert _call("qasp_check_batch", None, b(bat), 0, None, None, 0, None) == api.ERR_NULL_ARG
    assert _call("qasp_check_batch", b(lay), None, 0, None, None, 0, None) == api.ERR_NULL_ARG
    assert _call("qasp_check_batch", b(lay), b(bat), -1, None, None, 0, None) == api.ERR_BAD_SHAPE
    assert _call("qasp_check_batch", b(lay), b(bat), 17, None, None, 0, None) == api.ERR_BAD_SHAPE
    assert _call("qasp_check_batch", b(lay), b(bat), 0, None, None, -1, None) == api.ERR_BAD_SHAPE
    assert _call("qasp_check_batch", b(lay), b(bat), 0, 0x10, None, 4, None) == api.ERR_NULL_ARG
    assert _call("qasp_check_batch", b(lay), b(_batch(stride=100)), 0, None, None, 0, None) == api.ERR_BAD_SHAPE
    # an empty batch has nothing to check
    assert _call("qasp_check_batch", b(lay), b(_batch(B=0)), 0, None, None, 0, None) == api.OK


def test_validate_mode_keeps_host_checks_first(L, monkeypatch):
    """In validate mode the host-side argument errors are still returned
    before the device check would run."""
    monkeypatch.setenv("QASP_VALIDATE", "1")
    b = ctypes.byref
    lay, pol, bat = GQA.c(), api.Policy(1, 4, 32).c(), _batch()
    assert _call("qasp_decode_step", b(lay), b(bat), b(pol), 1, None, None, 1, 1, 1, 1.0, 1, None, None,
                 36, 1, 1 << 30, None) == api.ERR_MAX_SEL
    assert _call("qasp_sparse_paged_decode", b(lay), b(bat), b(pol), 1, 1, 1, 1, 1, 37, 1.0, 1, 1,
                 1, None) == api.ERR_WORKSPACE
    assert _call("qasp_build_summaries", b(lay), b(bat), None, 1, None) == api.ERR_NULL_ARG


def test_noalloc_step_rejects_sizes_beyond_its_scratch(L):
    """qasp_decode_step_noalloc refuses, before any HIP call, a call whose
    workspace would not fit the static scratch buffer."""
    b = ctypes.byref
    lay, pol = GQA.c(), api.Policy(1, 4, 32).c()
    limit = api.scratch_bytes()
    assert limit == 32 << 20
    small = _batch()
    assert _call("qasp_workspace_bytes", b(lay), b(small), b(pol), 37) <= limit
    # 4000 sequences x 8 KV heads x 4097 pages of 16-byte score records: far beyond the scratch
    big = _batch(B=4000, stride=4097, max_pages=4097)
    assert _call("qasp_workspace_bytes", b(lay), b(big), b(pol), 37) > limit
    assert _call("qasp_decode_step_noalloc", b(lay), b(big), b(pol), 1, None, None, 1, 1, 1, 1.0, 1, None, None,
                 37, None) == api.ERR_SCRATCH
    assert "scratch" in api.status_string(api.ERR_SCRATCH)
    # the other argument errors as qasp_decode_step
    assert _call("qasp_decode_step_noalloc", b(lay), b(small), b(pol), 1, None, None, 1, 1, 1, 1.0, 1, None, None,
                 36, None) == api.ERR_MAX_SEL
    assert _call("qasp_decode_step_noalloc", b(lay), b(small), b(pol), None, None, None, 1, 1, 1, 1.0, 1, None,
                 None, 37, None) == api.ERR_NULL_ARG


def test_decode_step_path(L):
    """The library's own dispatch rule, as the benchmark reads it."""
    pol = api.Policy(1, 8, 119)
    b = lambda B, mp: api.CBatch(B, 32, mp + 1, mp, 0x1000, 0x2000)
    path = lambda lay, bat, p, msel: _call("qasp_decode_step_path", ctypes.byref(lay.c()), ctypes.byref(bat),
                                           ctypes.byref(p.c()), msel)
    big = api.Layout(131072, 16, 8, 128, 128)
    assert path(big, b(32, 2048), pol, 128) == api.PATH_ONE_KERNEL      # 32K x 32: 256 units
    assert path(big, b(25, 2048), pol, 128) == api.PATH_ONE_KERNEL      # 200 units
    assert path(big, b(24, 2048), pol, 128) == api.PATH_CHAIN           # 192 units
    assert path(big, b(8, 8192), pol, 256) == api.PATH_CHAIN            # needle: 64 units, 8192 pages
    tiny = api.Layout(512, 16, 8, 128, 128)
    assert path(tiny, b(1, 256), api.Policy(1, 4, 32), 37) == api.PATH_ONE_KERNEL   # 8 small units
    assert path(big, b(3, 190), pol, 128) == api.PATH_CHAIN             # 24 units of 1.1 MB each
    assert path(big, b(64, 4097), pol, 128) == api.PATH_CHAIN           # page list past the kernel's arrays
    assert path(big, b(64, 4096), pol, 4096) == api.PATH_ONE_KERNEL     # 98 KB of on-chip arrays
    # 16 heads per group: the merge area grows, and with every page selected the arrays pass 160 KB
    assert path(big, api.CBatch(64, 128, 4097, 4096, 0x1000, 0x2000), pol, 4096) == api.PATH_CHAIN
    assert path(big, api.CBatch(64, 128, 4097, 4096, 0x1000, 0x2000), pol, 128) == api.PATH_ONE_KERNEL
    mla = api.Layout(32768, 64, 1, 576, 512, True)
    assert path(mla, api.CBatch(256, 128, 1025, 1024, 0x1000, 0x2000), pol, 32) == api.PATH_CHAIN
    assert path(big, b(32, 2048), pol, -1) == api.ERR_BAD_SHAPE


def test_summary_rows_undo_the_slot_rotation():
    """The summary pool keeps the record of KV head g of page p in slot
    (g + p) mod Hkv of row p; summary_rows returns records in head order."""
    pool, hkv, d = 11, 8, 4
    summ = torch.zeros((pool, hkv, 2, d), dtype=torch.float32)
    for p in range(pool):
        for g in range(hkv):
            summ[p, (g + p) % hkv] = 100 * p + g  # the record of (page p, head g)
    phys = torch.tensor([3, 0, 10, 7])
    rows = api.summary_rows(summ, phys)
    assert rows.shape == (4, hkv, 2, d)
    for i, p in enumerate(phys.tolist()):
        for g in range(hkv):
            assert (rows[i, g] == 100 * p + g).all()
    mask = torch.zeros(pool, dtype=torch.bool)
    mask[[2, 5]] = True
    assert torch.equal(api.summary_rows(summ, mask), api.summary_rows(summ, torch.tensor([2, 5])))
    one = torch.arange(6.0).reshape(3, 1, 2, 1)  # one KV head: no rotation
    assert torch.equal(api.summary_rows(one, torch.tensor([2, 0])), one[[2, 0]])
