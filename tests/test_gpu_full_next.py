"""Full-size parity of the multi-query, quantised-page and cross-layer reuse
steps on the 32K x 32 workload, in the launch configuration bench.py times
(256 units: the one-kernel forms), against the oracle on every sequence
(chunks of sequences re-packed into small pools, run on worker threads;
logical page ids unchanged).

Bars as in the small tests: pools, summaries, selections and quantised
page-heads bit-exact, outputs within 5e-3."""
import numpy as np
import pytest
import torch

from query_aware_sparse_paged_amd import api, workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    from gpu_cases import DEV, OUT_TOL, chunked, map_chunks, opolicy, oracle_inputs
    from test_gpu_quant import unpack

CHUNK = 2


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


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
    k_before, v_before = w.k_pool.clone(), w.v_pool.clone()
    ws = api.new_workspace_multi(lay, bat, pol, nq, msel, DEV)
    sel = torch.empty((w.spec.batch, lay.num_kv_heads, msel), dtype=torch.int32, device=DEV)
    cnt = torch.empty((w.spec.batch, lay.num_kv_heads), dtype=torch.int32, device=DEV)
    out = api.decode_step_multi(lay, bat, pol, dq, w.k_pool, w.v_pool, summ, w.scale, ws, msel, k_new=dk, v_new=dv,
                                sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    g_sel, g_cnt, g_out = sel.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    dkb, dvb = workloads.bits(dk), workloads.bits(dv)
    opol = opolicy(pol)

    def gather(seqs):
        after = oracle_inputs(w, seqs, q=dq)
        before = oracle_inputs(w, seqs, k_pool=k_before, v_pool=v_before, q=dq)
        return after, before, workloads.bits(api.summary_rows(summ, after.phys))

    def job(seqs, gathered):
        after, before, gsumm = gathered
        pt, sl, olay = after.pt, after.sl, after.olay
        # expected pools: the drafts written over each sequence's last positions
        k_exp, v_exp = before.k.copy(), before.v.copy()
        for s, b in enumerate(seqs):
            L = int(sl[s])
            for i in range(nq):
                pos = L - nq + i
                p = pt[s, pos // 16]
                k_exp[p, :, pos % 16, :] = dkb[b, i]
                v_exp[p, :, :, pos % 16] = dvb[b, i]
        assert np.array_equal(after.k, k_exp) and np.array_equal(after.v, v_exp), "pools differ %s" % seqs
        rs = oracle.summaries(olay, pt, sl, Hq, k_exp)
        assert np.array_equal(gsumm, rs), "summaries differ %s" % seqs
        sc = oracle.scores_multi(olay, pt, sl, after.q, rs, opol)
        rsel, rcnt = oracle.select_multi(olay, pt, sl, Hq, nq, sc, opol, max_sel_n=msel)
        assert np.array_equal(g_cnt[seqs], rcnt) and np.array_equal(g_sel[seqs], rsel), "selection differs %s" % seqs
        ref = oracle.attend_multi(olay, pt, sl, after.q, k_exp, v_exp, rsel, rcnt, opol, w.scale)
        err = np.abs(g_out[seqs].astype(np.float64) - ref).max()
        assert err <= OUT_TOL, "max abs error %.3g %s" % (err, seqs)
        return err

    map_chunks(chunked(w.spec.batch, CHUNK), gather, job)
    del w, summ, ws, out, k_before, v_before
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
    g_sel, g_cnt, g_out = sel.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    opol = opolicy(pol)

    def gather(seqs):
        inp = oracle_inputs(w, seqs)
        return inp, workloads.bits(api.summary_rows(summ, inp.phys)), qpool[inp.phys].cpu().numpy()

    def job(seqs, gathered):
        inp, gsumm, gq = gathered
        pt, sl, olay = inp.pt, inp.sl, inp.olay
        rs = oracle.summaries(olay, pt, sl, Hq, inp.k)
        assert np.array_equal(gsumm, rs), "summaries differ %s" % seqs
        sc = oracle.scores(olay, pt, sl, inp.q, rs, opol)
        rsel, rcnt = oracle.select(olay, pt, sl, Hq, sc, opol, max_sel_n=msel)
        assert np.array_equal(g_cnt[seqs], rcnt) and np.array_equal(g_sel[seqs], rsel), "selection differs %s" % seqs
        qz = oracle.quantize(olay, pt, sl, Hq, R, inp.k, inp.v)
        kc, km, vc, vm = unpack(gq)
        n_q = 0
        for s in range(len(seqs)):
            P = (int(sl[s]) + 15) // 16
            rows = pt[s, :P - R]
            assert np.array_equal(kc[rows], qz.k_codes[rows]) and np.array_equal(km[rows], qz.k_meta[rows])
            assert np.array_equal(vc[rows], qz.v_codes[rows]) and np.array_equal(vm[rows], qz.v_meta[rows])
            n_q += len(rows)
        assert n_q > 0
        ref = oracle.attend_quant(olay, pt, sl, inp.q, inp.k, inp.v, qz, rsel, rcnt, opol, w.scale)
        err = np.abs(g_out[seqs].astype(np.float64) - ref).max()
        assert err <= OUT_TOL, "max abs error %.3g %s" % (err, seqs)
        return err

    map_chunks(chunked(w.spec.batch, CHUNK), gather, job)
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
    out_a = api.decode_step(lay, bat, pol, a.q, a.k_pool, a.v_pool, summ, a.scale, ws, msel, k_new=a.k_new,
                            v_new=a.v_new, sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    g_out_a = out_a.cpu().numpy()
    # the reusing layer: the same page table, its own pools (keys reversed, values negated) and query
    kb_pool, vb_pool = a.k_pool.flip(-1).contiguous(), (-a.v_pool).contiguous()
    qb = a.q.flip(-1).contiguous()
    out = api.decode_step_reuse(lay, bat, pol, qb, kb_pool, vb_pool, None, a.scale, sel, cnt, ws,
                                k_new=a.k_new.flip(-1).contiguous(), v_new=(-a.v_new).contiguous())
    torch.cuda.synchronize()
    g_sel, g_cnt, g_out = sel.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    assert (g_cnt == 128).all()
    opol = opolicy(pol)

    def gather(seqs):
        ia = oracle_inputs(a, seqs)
        return ia, oracle_inputs(a, seqs, k_pool=kb_pool, v_pool=vb_pool, q=qb), workloads.bits(api.summary_rows(summ, ia.phys))

    def job(seqs, gathered):
        ia, ib, gsumm = gathered
        pt, sl, olay = ia.pt, ia.sl, ia.olay
        # the selecting layer: its selection (the one layer B reuses) and output
        rs = oracle.summaries(olay, pt, sl, Hq, ia.k)
        assert np.array_equal(gsumm, rs), "summaries differ %s" % seqs
        ra, rsel, rcnt = oracle.decode(olay, pt, sl, ia.q, ia.k, ia.v, rs, opol, a.scale, max_sel_n=msel)
        assert np.array_equal(g_cnt[seqs], rcnt) and np.array_equal(g_sel[seqs], rsel), "selection differs %s" % seqs
        assert np.abs(g_out_a[seqs].astype(np.float64) - ra).max() <= OUT_TOL
        # the reusing layer over the oracle's selection
        ref = oracle.attend(olay, pt, sl, ib.q, ib.k, ib.v, rsel, rcnt, opol, a.scale)
        err = np.abs(g_out[seqs].astype(np.float64) - ref).max()
        assert err <= OUT_TOL, "max abs error %.3g %s" % (err, seqs)
        return err

    map_chunks(chunked(a.spec.batch, CHUNK), gather, job)
    del a, summ, ws, out, out_a, kb_pool, vb_pool
    _free()
