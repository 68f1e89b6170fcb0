"""GPU parity of the cross-layer reuse step (qasp_decode_step_reuse): a layer
appends its token and attends over the pages that an earlier layer selected
at the same step, with no scoring or selection of its own (the OmniKV /
DeltaKV family named in the SparseEngine article's decode-hook paragraph).

Oracle: the selecting layer's selection (oracle.scores / select, compared
with the GPU's), this layer's pools with the token written, attention over
that selection (oracle.attend), summaries from scratch (oracle.summaries).  Bar:
pools and summaries bit-exact, outputs within 5e-3 max-abs, the selection
left untouched."""
import numpy as np
import pytest
import torch

from query_aware_sparse_paged_amd import api, workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    from gpu_cases import DEV, OUT_TOL, olayout, opolicy, run_oracle


def _case(name, batch, big=False):
    """Layer A and layer B share the page table, the lengths and the pool
    size (a pool's size follows the lengths it was drawn for, so B's pools are
    built from A's shape); B's contents differ: keys with their channels
    reversed, values negated (exact in bf16), its own queries."""
    if name.startswith("mla"):
        kw = dict(batch=batch, seq_len=6000, seq_len_min=4000)
    elif big:
        kw = dict(batch=batch, seq_len=9000, seq_len_min=8700)
    else:
        kw = dict(batch=batch, seq_len=900, seq_len_min=600)
    a = workloads.make(name, device="cpu", seed=11, **kw)   # the layer that selects
    other = workloads.make(name, device="cpu", seed=23, **kw)
    b = workloads.Workload(a.spec, a.seq_lens, a.page_table, other.q, a.k_pool.flip(-1).contiguous(),
                           None if a.v_pool is None else (-a.v_pool).contiguous(), a.k_new.flip(-1).contiguous(),
                           None if a.v_new is None else (-a.v_new).contiguous(), None)
    return a, b


@pytest.mark.parametrize("name,batch,top_k", [("llama8b_b32_32k", 32, None),   # one kernel per (sequence, KV head)
                                              ("llama8b_b32_32k", 3, None),    # append + decode kernels
                                              ("llama8b_b32_32k", 32, 530),    # > 512 pages per unit, one kernel
                                              ("mla_b16_64k", 2, None)])
@pytest.mark.parametrize("with_summ", [True, False])
def test_reuse_step(name, batch, top_k, with_summ):
    print("reuse case", name, batch, top_k, with_summ, flush=True)
    A, B = _case(name, batch, big=top_k is not None)
    lay, pol = api.layout_of(A), api.policy_of(A)
    if top_k is not None:
        pol = api.Policy(pol.n_sink_pages, pol.n_local_pages, top_k)
    Hq = A.spec.num_q_heads
    pt, sl = A.page_table, A.seq_lens                # shared page table and lengths
    assert int(pt.max()) < B.k_pool.shape[0] == A.k_pool.shape[0]
    bat = api.Batch(pt.to(DEV), sl.to(DEV), Hq)
    msel = api.max_sel(lay, pol, bat.max_pages)
    t = lambda x: None if x is None else x.to(DEV)

    # layer A: a whole step, its selection kept
    summ_a = torch.zeros((lay.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16,
                         device=DEV)
    ka, va = t(A.k_pool), t(A.v_pool)
    api.build_summaries(lay, bat, ka, summ_a)
    ws = api.new_workspace(lay, bat, pol, msel, DEV)
    sel = torch.full((batch, lay.num_kv_heads, msel), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((batch, lay.num_kv_heads), -7, dtype=torch.int32, device=DEV)
    api.decode_step(lay, bat, pol, t(A.q), ka, va, summ_a, A.scale, ws, msel, k_new=t(A.k_new),
                    v_new=t(A.v_new), sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    sel_np, cnt_np = sel.cpu().numpy(), cnt.cpu().numpy()
    # the selection layer B reuses is the oracle's (the token A appends is the
    # value already at L-1, so A's pools and summaries are unchanged)
    ra = run_oracle(A, pol, msel)
    assert np.array_equal(cnt_np, ra.cnt) and np.array_equal(sel_np, ra.sel)

    # layer B: a new token (not yet in its pools), its summaries before the token
    gen = torch.Generator().manual_seed(3)
    new_k = torch.randn(B.k_new.shape, generator=gen).to(torch.bfloat16)
    new_v = None if B.v_pool is None else torch.randn(B.v_new.shape, generator=gen).to(torch.bfloat16)
    kb, vb = t(B.k_pool), t(B.v_pool)
    summ_b = None
    if with_summ:
        summ_b = torch.zeros_like(summ_a)
        api.build_summaries(lay, api.Batch(bat.page_table, (bat.seq_lens - 1).contiguous(), Hq), kb, summ_b)
    out = api.decode_step_reuse(lay, bat, pol, t(B.q), kb, vb, summ_b, B.scale, sel, cnt, ws,
                                k_new=t(new_k), v_new=t(new_v))
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), sel_np) and np.array_equal(cnt.cpu().numpy(), cnt_np)

    # oracle: the token written into B's pools, attention over A's selection
    ps = lay.page_size
    for b in range(batch):
        L = int(sl[b])
        phys = int(pt[b, (L - 1) // ps])
        B.k_pool[phys, :, (L - 1) % ps, :] = new_k[b]
        if B.v_pool is not None:
            B.v_pool[phys, :, :, (L - 1) % ps] = new_v[b]
    assert torch.equal(kb.cpu().view(torch.int16), B.k_pool.view(torch.int16))
    if B.v_pool is not None:
        assert torch.equal(vb.cpu().view(torch.int16), B.v_pool.view(torch.int16))
    olay, opol = olayout(lay), opolicy(pol)
    pt_np, sl_np = pt.numpy(), sl.numpy()
    kbits = workloads.bits(B.k_pool)
    vbits = None if B.v_pool is None else workloads.bits(B.v_pool)
    ref = oracle.attend(olay, pt_np, sl_np, workloads.bits(B.q), kbits, vbits, ra.sel, ra.cnt, opol, B.scale)
    gout = out.cpu().numpy()
    assert np.isfinite(gout).all()
    assert np.abs(gout.astype(np.float64) - ref).max() <= OUT_TOL
    if with_summ:
        rs = oracle.summaries(olay, pt_np, sl_np, Hq, kbits)
        used = pt[pt >= 0].long()
        assert np.array_equal(workloads.bits(api.summary_rows(summ_b.cpu(), used)), rs[used.numpy()])
    assert (cnt_np > 0).all()
    if top_k is not None:
        assert cnt_np.min() > 512
