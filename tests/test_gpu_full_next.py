"""Full-size parity of the multi-query, quantised-page and cross-layer reuse
steps on the 32K x 32 workload, in the launch configuration bench.py times
(256 units: the one-kernel forms), against the oracle on sampled sequences
(re-packed into a small pool; logical page ids unchanged).

Bars as in the small tests: pools, summaries, selections and quantised
page-heads bit-exact, outputs within 5e-3."""
import numpy as np
import pytest
import torch

from query_aware_sparse_paged_amd import api, workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    from gpu_cases import DEV, OUT_TOL, olayout, opolicy
    from test_gpu_quant import unpack

SEQS = [0, 17, 31]


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _repack(w, k_pool, v_pool, seqs=SEQS):
    """Sub-batch of sequences seqs: (page table into a small pool, lengths,
    physical pages used (device order), k bits, v bits) from the given pools."""
    pt_full = w.page_table[seqs]
    valid = pt_full >= 0
    phys = pt_full[valid].long()
    k = workloads.bits(k_pool[phys])
    v = None if v_pool is None else workloads.bits(v_pool[phys])
    pt = np.full(tuple(pt_full.shape), -1, np.int32)
    pt[valid.cpu().numpy()] = np.arange(phys.numel(), dtype=np.int32)
    return pt, w.seq_lens[seqs].cpu().numpy(), phys, k, v


def _small_layout(lay, n_pages):
    return oracle.Layout(int(n_pages), lay.page_size, lay.num_kv_heads, lay.head_dim_k, lay.head_dim_v, lay.v_from_k)


def test_full_multi_query_4_drafts():
    print("full-size multi-query step", flush=True)
    w = workloads.make("llama8b_b32_32k", device=DEV)
    nq = 4
    dq, dk, dv = workloads.drafts(w, nq, 77, device=DEV)
    lay, pol = api.layout_of(w), api.policy_of(w)
    Hq = w.spec.num_q_heads
    bat = api.Batch(w.page_table, w.seq_lens, Hq)
    msel = api.max_sel_multi(lay, pol, nq, bat.max_pages)
    summ = torch.zeros((lay.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16, device=DEV)
    api.build_summaries(lay, api.Batch(bat.page_table, (bat.seq_lens - nq).contiguous(), Hq), w.k_pool, summ)
    _, _, phys, k_before, v_before = _repack(w, w.k_pool, w.v_pool)
    ws = api.new_workspace_multi(lay, bat, pol, nq, msel, DEV)
    sel = torch.empty((w.spec.batch, lay.num_kv_heads, msel), dtype=torch.int32, device=DEV)
    cnt = torch.empty((w.spec.batch, lay.num_kv_heads), dtype=torch.int32, device=DEV)
    out = api.decode_step_multi(lay, bat, pol, dq, w.k_pool, w.v_pool, summ, w.scale, ws, msel, k_new=dk, v_new=dv,
                                sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    pt, sl, phys, k_after, v_after = _repack(w, w.k_pool, w.v_pool)
    # expected pools: the drafts written over the sampled sequences' last positions
    k_exp, v_exp = k_before.copy(), v_before.copy()
    dkb, dvb = workloads.bits(dk), workloads.bits(dv)
    for s, b in enumerate(SEQS):
        L = int(sl[s])
        for i in range(nq):
            pos = L - nq + i
            p = pt[s, pos // 16]
            k_exp[p, :, pos % 16, :] = dkb[b, i]
            v_exp[p, :, :, pos % 16] = dvb[b, i]
    assert np.array_equal(k_after, k_exp) and np.array_equal(v_after, v_exp)
    olay, opol = _small_layout(lay, phys.numel()), opolicy(pol)
    rs = oracle.summaries(olay, pt, sl, Hq, k_exp)
    assert np.array_equal(workloads.bits(summ[phys]), rs)
    qb = workloads.bits(dq[SEQS])
    sc = oracle.scores_multi(olay, pt, sl, qb, rs, opol)
    rsel, rcnt = oracle.select_multi(olay, pt, sl, Hq, nq, sc, opol, max_sel_n=msel)
    assert np.array_equal(cnt[SEQS].cpu().numpy(), rcnt)
    assert np.array_equal(sel[SEQS].cpu().numpy(), rsel)
    ref = oracle.attend_multi(olay, pt, sl, qb, k_exp, v_exp, rsel, rcnt, opol, w.scale)
    assert np.abs(out[SEQS].cpu().numpy().astype(np.float64) - ref).max() <= OUT_TOL
    del w, summ, ws, out
    _free()


def test_full_quantised_pages():
    print("full-size quantised-page step", flush=True)
    R = 8
    w = workloads.make("llama8b_b32_32k", device=DEV)
    lay, pol = api.layout_of(w), api.policy_of(w)
    Hq = w.spec.num_q_heads
    bat = api.Batch(w.page_table, w.seq_lens, Hq)
    msel = api.max_sel(lay, pol, bat.max_pages)
    summ = torch.zeros((lay.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16, device=DEV)
    api.build_summaries(lay, bat, w.k_pool, summ)
    qpool = api.new_quant_pool(lay, DEV)
    api.quantize_pages(lay, api.Batch(bat.page_table, (bat.seq_lens - 1).contiguous(), Hq), R, w.k_pool, w.v_pool,
                       qpool)
    ws = api.new_workspace(lay, bat, pol, msel, DEV)
    sel = torch.empty((w.spec.batch, lay.num_kv_heads, msel), dtype=torch.int32, device=DEV)
    cnt = torch.empty((w.spec.batch, lay.num_kv_heads), dtype=torch.int32, device=DEV)
    out = api.decode_step_quant(lay, bat, pol, R, w.q, w.k_pool, w.v_pool, summ, qpool, w.scale, ws, msel,
                                k_new=w.k_new, v_new=w.v_new, sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    pt, sl, phys, kb, vb = _repack(w, w.k_pool, w.v_pool)
    olay, opol = _small_layout(lay, phys.numel()), opolicy(pol)
    rs = oracle.summaries(olay, pt, sl, Hq, kb)
    assert np.array_equal(workloads.bits(summ[phys]), rs)
    qb = workloads.bits(w.q[SEQS])
    sc = oracle.scores(olay, pt, sl, qb, rs, opol)
    rsel, rcnt = oracle.select(olay, pt, sl, Hq, sc, opol, max_sel_n=msel)
    assert np.array_equal(cnt[SEQS].cpu().numpy(), rcnt)
    assert np.array_equal(sel[SEQS].cpu().numpy(), rsel)
    qz = oracle.quantize(olay, pt, sl, Hq, R, kb, vb)
    kc, km, vc, vm = unpack(qpool[phys].cpu().numpy())
    n_q = 0
    for s in range(len(SEQS)):
        P = (int(sl[s]) + 15) // 16
        rows = pt[s, :P - R]
        assert np.array_equal(kc[rows], qz.k_codes[rows]) and np.array_equal(km[rows], qz.k_meta[rows])
        assert np.array_equal(vc[rows], qz.v_codes[rows]) and np.array_equal(vm[rows], qz.v_meta[rows])
        n_q += len(rows)
    assert n_q > 0
    ref = oracle.attend_quant(olay, pt, sl, qb, kb, vb, qz, rsel, rcnt, opol, w.scale)
    assert np.abs(out[SEQS].cpu().numpy().astype(np.float64) - ref).max() <= OUT_TOL
    del w, summ, qpool, ws, out
    _free()


def test_full_cross_layer_reuse():
    print("full-size cross-layer reuse step", flush=True)
    a = workloads.make("llama8b_b32_32k", device=DEV)
    lay, pol = api.layout_of(a), api.policy_of(a)
    Hq = a.spec.num_q_heads
    bat = api.Batch(a.page_table, a.seq_lens, Hq)
    msel = api.max_sel(lay, pol, bat.max_pages)
    summ = torch.zeros((lay.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16, device=DEV)
    api.build_summaries(lay, bat, a.k_pool, summ)
    ws = api.new_workspace(lay, bat, pol, msel, DEV)
    sel = torch.empty((a.spec.batch, lay.num_kv_heads, msel), dtype=torch.int32, device=DEV)
    cnt = torch.empty((a.spec.batch, lay.num_kv_heads), dtype=torch.int32, device=DEV)
    api.decode_step(lay, bat, pol, a.q, a.k_pool, a.v_pool, summ, a.scale, ws, msel, k_new=a.k_new, v_new=a.v_new,
                    sel=sel, sel_count=cnt)
    # the reusing layer: the same page table, its own pools (keys reversed, values negated) and query
    kb_pool, vb_pool = a.k_pool.flip(-1).contiguous(), (-a.v_pool).contiguous()
    qb = a.q.flip(-1).contiguous()
    out = api.decode_step_reuse(lay, bat, pol, qb, kb_pool, vb_pool, None, a.scale, sel, cnt, ws,
                                k_new=a.k_new.flip(-1).contiguous(), v_new=(-a.v_new).contiguous())
    torch.cuda.synchronize()
    pt, sl, phys, kb, vb = _repack(a, kb_pool, vb_pool)
    olay, opol = _small_layout(lay, phys.numel()), opolicy(pol)
    s_sel, s_cnt = sel[SEQS].cpu().numpy(), cnt[SEQS].cpu().numpy()
    assert (s_cnt == 128).all()
    ref = oracle.attend(olay, pt, sl, workloads.bits(qb[SEQS]), kb, vb, s_sel, s_cnt, opol, a.scale)
    assert np.abs(out[SEQS].cpu().numpy().astype(np.float64) - ref).max() <= OUT_TOL
    del a, summ, ws, out, kb_pool, vb_pool
    _free()
