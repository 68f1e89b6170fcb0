"""GPU parity of the multi-query step (qasp_decode_step_multi): n draft
tokens per sequence, appended, one shared selection per (sequence, KV head),
causal attention per draft (speculative decoding of multi-token-prediction
drafts; the llama.cpp draft-head fix article on aikeizai.jp, the section on
why it matters).

Oracle: the drafts written into the pools, summaries from scratch
(oracle.summaries), oracle.scores_multi, oracle.select_multi and
oracle.attend_multi.  Bar: pools, summaries and selections bit-exact, outputs
within 5e-3 max-abs."""
import numpy as np
import pytest
import torch

from query_aware_sparse_paged_amd import api, workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    from gpu_cases import DEV, OUT_TOL, olayout, opolicy


def _run(name, batch, nq, seq_len, seq_len_min, seed=31, **overrides):
    print("multi-query case", name, batch, nq, seq_len, overrides, flush=True)
    w = workloads.make(name, device="cpu", seed=seed, batch=batch, seq_len=seq_len, seq_len_min=seq_len_min,
                       **overrides)
    dq, dk, dv = workloads.drafts(w, nq, seed + 1)
    lay, pol = api.layout_of(w), api.policy_of(w)
    Hq = w.spec.num_q_heads
    pt, sl = w.page_table, w.seq_lens
    t = lambda x: None if x is None else x.to(DEV)
    bat = api.Batch(t(pt), t(sl), Hq)
    msel = api.max_sel_multi(lay, pol, nq, bat.max_pages)
    kp, vp = t(w.k_pool), t(w.v_pool)
    # summaries of the sequences before the drafts
    summ = torch.zeros((lay.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16, device=DEV)
    api.build_summaries(lay, api.Batch(bat.page_table, (bat.seq_lens - nq).clamp(min=0).contiguous(), Hq), kp, summ)
    ws = api.new_workspace_multi(lay, bat, pol, nq, msel, DEV)
    sel = torch.full((batch, lay.num_kv_heads, msel), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((batch, lay.num_kv_heads), -7, dtype=torch.int32, device=DEV)
    out = api.decode_step_multi(lay, bat, pol, t(dq), kp, vp, summ, w.scale, ws, msel, k_new=t(dk), v_new=t(dv),
                                sel=sel, sel_count=cnt)
    torch.cuda.synchronize()

    # oracle: drafts written at L - nq ... L - 1
    ps = lay.page_size
    for b in range(batch):
        L = int(sl[b])
        for i in range(nq):
            pos = L - nq + i
            if pos < 0:
                continue
            phys = int(pt[b, pos // ps])
            w.k_pool[phys, :, pos % ps, :] = dk[b, i]
            w.v_pool[phys, :, :, pos % ps] = dv[b, i]
    assert torch.equal(kp.cpu().view(torch.int16), w.k_pool.view(torch.int16))
    assert torch.equal(vp.cpu().view(torch.int16), w.v_pool.view(torch.int16))
    olay, opol = olayout(lay), opolicy(pol)
    pt_np, sl_np = pt.numpy(), sl.numpy()
    kbits, vbits = workloads.bits(w.k_pool), workloads.bits(w.v_pool)
    rs = oracle.summaries(olay, pt_np, sl_np, Hq, kbits)
    used = pt[pt >= 0].long()
    used = used[used < lay.num_pool_pages]
    assert np.array_equal(workloads.bits(api.summary_rows(summ.cpu(), used)), rs[used.numpy()])
    qbits = workloads.bits(dq)
    sc = oracle.scores_multi(olay, pt_np, sl_np, qbits, rs, opol)
    rsel, rcnt = oracle.select_multi(olay, pt_np, sl_np, Hq, nq, sc, opol, max_sel_n=msel)
    gsel, gcnt = sel.cpu().numpy(), cnt.cpu().numpy()
    assert np.array_equal(gcnt, rcnt)
    for b in range(batch):
        for g in range(lay.num_kv_heads):
            assert np.array_equal(gsel[b, g, :gcnt[b, g]], rsel[b, g, :rcnt[b, g]]), (b, g)
    ref = oracle.attend_multi(olay, pt_np, sl_np, qbits, kbits, vbits, rsel, rcnt, opol, w.scale)
    gout = out.cpu().numpy()
    assert np.isfinite(gout).all()
    err = np.abs(gout.astype(np.float64) - ref).max()
    assert err <= OUT_TOL, err
    return gout, ref


@pytest.mark.parametrize("nq", [1, 2, 4])
def test_multi_step_few_sequences(nq):
    _run("llama8b_b32_32k", 3, nq, 900, 600)


def test_multi_step_one_draft_many_units():
    # one draft on the one-kernel path: the draft is the step's token, appended at L - 1
    _run("llama8b_b32_32k", 32, 1, 1100, 400)


def test_multi_step_many_units_ragged_tail():
    # 64 sequences x 8 KV heads: 512 units, one kernel per unit after the draft append; lengths not page-aligned
    _run("llama8b_b32_32k", 64, 4, 1000, 300)


@pytest.mark.parametrize("nq,window", [(3, 1024), (2, 0)])
def test_multi_step_many_units_static_heads(nq, window):
    # 32 sequences x 8 KV heads (one kernel per unit), A-shape heads beside query-aware heads
    _run("ragged_b64_mixed", 32, nq, 2600, 900, window_tokens=window)


@pytest.mark.parametrize("nq", [2, 3])
def test_multi_step_static_heads(nq):
    # A-shape heads (sink 4 tokens, window 1024) beside query-aware heads
    _run("ragged_b64_mixed", 6, nq, 3000, 1100)


def test_multi_step_zero_window_and_two_heads_per_group():
    # static heads with no window (sink only); 16 q / 8 KV heads: 2 heads per group, 8 drafts
    _run("ragged_b64_mixed", 4, 8, 2500, 700, window_tokens=0, num_q_heads=16)


@pytest.mark.parametrize("nq,kw", [
    (8, dict(num_q_heads=16)),        # 8 drafts x 2 heads: the drafts are written in the kernel's prologue
    (3, dict(n_local_pages=0)),       # no local pages: the drafts' pages are candidates, scored with them
])
def test_multi_step_many_units_prologue_append(nq, kw):
    _run("llama8b_b32_32k", 32, nq, 1100, 400, **kw)


def test_multi_step_drafts_differ():
    gout, ref = _run("llama8b_b32_32k", 2, 3, 700, 500, seed=37)
    assert np.abs(gout[:, 0] - gout[:, 2]).max() > 1e-3


def test_multi_step_large_selection():
    # 32 x 8 units (one kernel per unit), 2 drafts, about 530 pages selected per unit: more than 64 per wave
    _run("llama8b_b32_32k", 32, 2, 9000, 8700, top_k=520)
