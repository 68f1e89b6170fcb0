"""Validate mode (QASP_VALIDATE=1) and qasp_check_batch on the GPU.

Every case that must be rejected keeps all its memory accesses inside
allocated buffers even if the check did not exist: the bad page ids lie in a
gap of pool pages that the tensors hold but the layout does not declare, and
the lengths and selections that are out of range are only given to
qasp_check_batch itself, whose reads stay inside the stated array shapes.
Accepted inputs must give bit-identical results with and without the check."""
import numpy as np
import pytest
import torch

from query_aware_sparse_paged_amd import api, workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_cases import DEV

GAP = 8  # pool pages held by the tensors beyond the layout's num_pool_pages


def _case(batch, seq_len=900):
    """A workload whose pools hold GAP more pages than the layout declares."""
    w = workloads.make("llama8b_b32_32k", device=DEV, batch=batch, seq_len=seq_len, seq_len_min=seq_len - 300)
    lay = api.layout_of(w)
    pad = lambda t: torch.cat([t, torch.zeros((GAP,) + tuple(t.shape[1:]), dtype=t.dtype, device=DEV)])
    w.k_pool, w.v_pool = pad(w.k_pool), pad(w.v_pool)
    assert lay.num_pool_pages + GAP == w.k_pool.shape[0]
    return w, lay, api.policy_of(w)


def _step(w, lay, pol, page_table=None):
    pt = w.page_table if page_table is None else page_table
    bat = api.Batch(pt, w.seq_lens, w.spec.num_q_heads)
    msel = api.max_sel(lay, pol, bat.max_pages)
    summ = torch.zeros((w.k_pool.shape[0], lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16, device=DEV)
    ws = api.new_workspace(lay, bat, pol, msel, DEV)
    out = torch.full((w.spec.batch, w.spec.num_q_heads, 128), 7.0, dtype=torch.float32, device=DEV)
    sel = torch.full((w.spec.batch, lay.num_kv_heads, msel), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((w.spec.batch, lay.num_kv_heads), -7, dtype=torch.int32, device=DEV)
    return bat, msel, summ, ws, out, sel, cnt


@pytest.mark.parametrize("batch", [3, 32])   # kernel chain; one-kernel step
def test_validate_mode_accepts_good_batches_bit_identically(batch, monkeypatch):
    print("validate mode, good batch", batch, flush=True)
    w, lay, pol = _case(batch)
    runs = []
    for mode in ("0", "1"):
        monkeypatch.setenv("QASP_VALIDATE", mode)
        bat, msel, summ, ws, out, sel, cnt = _step(w, lay, pol)
        api.build_summaries(lay, bat, w.k_pool, summ)
        api.decode_step(lay, bat, pol, w.q, w.k_pool, w.v_pool, summ, w.scale, ws, msel, k_new=w.k_new,
                        v_new=w.v_new, out=out, sel=sel, sel_count=cnt)
        torch.cuda.synchronize()
        runs.append((out.cpu(), sel.cpu(), cnt.cpu()))
    assert torch.equal(runs[0][1], runs[1][1]) and torch.equal(runs[0][2], runs[1][2])
    assert torch.equal(runs[0][0].view(torch.int32), runs[1][0].view(torch.int32))
    api.check_batch(lay, bat)
    api.check_batch(lay, bat, sel=sel, sel_count=cnt)


@pytest.mark.parametrize("batch", [3, 32])
def test_validate_mode_rejects_a_page_in_the_gap(batch, monkeypatch):
    """An entry naming a pool page the layout does not declare: every
    pool-reading call returns QASP_ERR_BAD_PAGE_TABLE and writes nothing."""
    print("validate mode, page in the gap", batch, flush=True)
    w, lay, pol = _case(batch)
    monkeypatch.setenv("QASP_VALIDATE", "1")
    good = api.Batch(w.page_table, w.seq_lens, w.spec.num_q_heads)
    _, msel, summ, ws, out, sel, cnt = _step(w, lay, pol)
    api.build_summaries(lay, good, w.k_pool, summ)
    api.decode_step(lay, good, pol, w.q, w.k_pool, w.v_pool, summ, w.scale, ws, msel, out=out, sel=sel,
                    sel_count=cnt)
    torch.cuda.synchronize()
    pt = w.page_table.clone()
    b = batch - 1
    pt[b, 5] = lay.num_pool_pages + 3                     # in the gap: allocated, not declared
    bat = api.Batch(pt, w.seq_lens, w.spec.num_q_heads)
    snap = [t.clone() for t in (out, sel, cnt, summ, w.k_pool, w.v_pool)]

    def rejected(fn):
        with pytest.raises(api.QaspError) as e:
            fn()
        assert e.value.status == api.ERR_BAD_PAGE_TABLE
    rejected(lambda: api.decode_step(lay, bat, pol, w.q, w.k_pool, w.v_pool, summ, w.scale, ws, msel,
                                     k_new=w.k_new, v_new=w.v_new, out=out, sel=sel, sel_count=cnt))
    rejected(lambda: api.build_summaries(lay, bat, w.k_pool, summ))
    rejected(lambda: api.append_kv(lay, bat, pol, w.k_new, w.v_new, w.k_pool, w.v_pool, summ))
    rejected(lambda: api.score_pages(lay, bat, pol, w.q, summ))
    sc = api.score_pages(lay, good, pol, w.q, summ)
    rejected(lambda: api.select_topk(lay, bat, pol, w.q, summ, sc, max_sel_n=msel))
    rejected(lambda: api.sparse_paged_decode(lay, bat, pol, w.q, w.k_pool, w.v_pool, sel, cnt, w.scale, ws,
                                             out=out))
    rejected(lambda: api.decode_step_reuse(lay, bat, pol, w.q, w.k_pool, w.v_pool, None, w.scale, sel, cnt, ws,
                                           out=out))
    qpool = torch.zeros((w.k_pool.shape[0], lay.num_kv_heads, 1536), dtype=torch.uint8, device=DEV)
    rejected(lambda: api.quantize_pages(lay, bat, 2, w.k_pool, w.v_pool, qpool))
    rejected(lambda: api.decode_step_quant(lay, bat, pol, 2, w.q, w.k_pool, w.v_pool, summ, qpool, w.scale, ws,
                                           msel, out=out))
    nq = 2
    dq, dk, dv = workloads.drafts(w, nq, 5, device=DEV)
    mmsel = api.max_sel_multi(lay, pol, nq, bat.max_pages)
    mws = api.new_workspace_multi(lay, bat, pol, nq, mmsel, DEV)
    rejected(lambda: api.decode_step_multi(lay, bat, pol, dq, w.k_pool, w.v_pool, summ, w.scale, mws, mmsel,
                                           k_new=dk, v_new=dv))
    rejected(lambda: api.check_batch(lay, bat))
    torch.cuda.synchronize()
    for before, after in zip(snap, (out, sel, cnt, summ, w.k_pool, w.v_pool)):
        assert torch.equal(before, after), "a rejected call wrote something"
    assert (qpool == 0).all()


def test_check_batch_finds_each_kind_of_bad_entry():
    """Lengths, negative ids and selections out of range, given to the check
    alone (its reads stay inside the arrays' stated shapes)."""
    print("qasp_check_batch cases", flush=True)
    w, lay, pol = _case(4, seq_len=600)
    Hq = w.spec.num_q_heads
    stride = int(w.page_table.shape[1])
    P = ((w.seq_lens + 15) // 16).cpu()

    def status(pt=None, sl=None, max_pages=None, extra=0, sel=None, cnt=None):
        bat = api.Batch(w.page_table if pt is None else pt, w.seq_lens if sl is None else sl, Hq, max_pages)
        try:
            api.check_batch(lay, bat, extra, sel, cnt)
            return api.OK
        except api.QaspError as e:
            return e.status

    bad = api.ERR_BAD_PAGE_TABLE
    assert status() == api.OK
    pt = w.page_table.clone()
    pt[1, 0] = -1
    assert status(pt=pt) == bad
    pt = w.page_table.clone()
    pt[2, int(P[2]) - 1] = lay.num_pool_pages           # the last page of a sequence
    assert status(pt=pt) == bad
    pt = w.page_table.clone()
    pt[2, int(P[2])] = -1                               # past the length: not read
    assert status(pt=pt) == api.OK
    assert status(extra=1) == api.OK                    # the spare page holds the append
    # an append at a page boundary needs the next entry
    assert status(pt=pt, extra=1) == (bad if int(w.seq_lens[2]) % 16 == 0 else api.OK)
    sl = w.seq_lens.clone()
    sl[0] = -3
    assert status(sl=sl) == bad
    full = w.page_table.clone()
    full[3] = torch.arange(stride, dtype=torch.int32, device=DEV)   # a whole row of valid pages
    sl = w.seq_lens.clone()
    sl[3] = (stride - 1) * 16 + 1                       # more pages than max_pages = stride - 1
    assert status(pt=full, sl=sl, max_pages=stride - 1) == bad
    assert status(pt=full, sl=sl) == api.OK             # max_pages = stride
    sl[3] = stride * 16
    assert status(pt=full, sl=sl) == api.OK
    assert status(pt=full, sl=sl, extra=1) == bad       # the append would go past the row
    msel = 20
    sel = torch.zeros((4, 8, msel), dtype=torch.int32, device=DEV)
    cnt = torch.full((4, 8), 3, dtype=torch.int32, device=DEV)
    sel[:, :, 1], sel[:, :, 2] = 1, 2
    assert status(sel=sel, cnt=cnt) == api.OK
    s2 = sel.clone()
    s2[2, 5, 1] = int(P[2])                             # one past the sequence's pages
    assert status(sel=s2, cnt=cnt) == bad
    s2 = sel.clone()
    s2[0, 0, 0] = -1
    assert status(sel=s2, cnt=cnt) == bad
    s2[0, 0, 0] = 0
    s2[0, 0, 3] = 10 ** 6                               # past the count: not read
    assert status(sel=s2, cnt=cnt) == api.OK
    c2 = cnt.clone()
    c2[1, 1] = msel + 1
    assert status(sel=sel, cnt=c2) == bad
    c2[1, 1] = -1
    assert status(sel=sel, cnt=c2) == bad
