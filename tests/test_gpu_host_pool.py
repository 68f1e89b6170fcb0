"""GPU parity of the host-tier KV pool: the K/V pools live in pinned host
memory mapped into the GPU (qasp_host_alloc); summaries, page tables and
workspaces stay in device memory (CPU-GPU cooperative loading: SCBench notes,
the discussion of CPU-GPU cooperation for Quest / RetrievalAttention).

The same kernels run on the same data as with device pools, so the bar is
bit-equality with the device-pool run: outputs, selections and the pools
after the step's append; and against the oracle: summaries and selections
bit-exact, outputs within 5e-3."""
import numpy as np
import pytest
import torch

from query_aware_sparse_paged_amd import api, workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_cases import DEV, OUT_TOL, run_oracle


def _step(w, lay, pol, kp, vp, summ, bat, msel):
    ws = api.new_workspace(lay, bat, pol, msel, DEV)
    sel = torch.full((w.spec.batch, lay.num_kv_heads, msel), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((w.spec.batch, lay.num_kv_heads), -7, dtype=torch.int32, device=DEV)
    out = api.decode_step(lay, bat, pol, w.q.to(DEV), kp, vp, summ, w.scale, ws, msel, k_new=w.k_new.to(DEV),
                          v_new=None if w.v_new is None else w.v_new.to(DEV), sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    return out.cpu(), sel.cpu(), cnt.cpu()


@pytest.mark.parametrize("name,batch,seq_len", [("llama8b_b32_32k", 3, 1500),    # kernel chain
                                                ("llama8b_b32_32k", 32, 1200),   # one kernel per unit
                                                ("ragged_b64_mixed", 32, 3000),  # static heads, one kernel
                                                ("mla_b16_64k", 2, 6000)])       # latent heads
def test_host_tier_pools_match_device_pools(name, batch, seq_len):
    print("host-tier case", name, batch, seq_len, flush=True)
    w = workloads.make(name, device="cpu", seed=5, batch=batch, seq_len=seq_len, seq_len_min=seq_len // 2)
    lay, pol = api.layout_of(w), api.policy_of(w)
    bat = api.Batch(w.page_table.to(DEV), w.seq_lens.to(DEV), w.spec.num_q_heads)
    msel = api.max_sel(lay, pol, bat.max_pages)
    # the token at L-1 is written again by the append with a new value, so the
    # pools after the step show the append went through
    gen = torch.Generator().manual_seed(9)
    w.k_new = torch.randn(w.k_new.shape, generator=gen).to(torch.bfloat16)
    if w.v_new is not None:
        w.v_new = torch.randn(w.v_new.shape, generator=gen).to(torch.bfloat16)

    summ_d = torch.zeros((lay.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16,
                         device=DEV)
    kd = w.k_pool.to(DEV)
    vd = None if w.v_pool is None else w.v_pool.to(DEV)
    # summaries of the cache before the step's token (lengths L - 1)
    api.build_summaries(lay, api.Batch(bat.page_table, (bat.seq_lens - 1).contiguous(), w.spec.num_q_heads), kd,
                        summ_d)
    summ_h = summ_d.clone()
    kh = api.host_pool_like(w.k_pool)
    vh = None if w.v_pool is None else api.host_pool_like(w.v_pool)

    out_d, sel_d, cnt_d = _step(w, lay, pol, kd, vd, summ_d, bat, msel)
    out_h, sel_h, cnt_h = _step(w, lay, pol, kh, vh, summ_h, bat, msel)
    assert torch.equal(cnt_h, cnt_d) and torch.equal(sel_h, sel_d)
    assert torch.equal(out_h.view(torch.int32), out_d.view(torch.int32))
    assert torch.equal(kh.host.view(torch.int16), kd.cpu().view(torch.int16))
    if vh is not None:
        assert torch.equal(vh.host.view(torch.int16), vd.cpu().view(torch.int16))
    assert torch.equal(summ_h.cpu().view(torch.int16), summ_d.cpu().view(torch.int16))

    # and the oracle: the token written into a host copy of the pools,
    # summaries from scratch, scores, selection and attention
    ps = lay.page_size
    for b in range(batch):
        L = int(w.seq_lens[b])
        phys = int(w.page_table[b, (L - 1) // ps])
        w.k_pool[phys, :, (L - 1) % ps, :] = w.k_new[b]
        if w.v_pool is not None:
            w.v_pool[phys, :, :, (L - 1) % ps] = w.v_new[b]
    assert torch.equal(kh.host.view(torch.int16), w.k_pool.view(torch.int16))
    r = run_oracle(w, pol, msel)
    used = w.page_table[w.page_table >= 0].long()
    assert np.array_equal(workloads.bits(api.summary_rows(summ_h.cpu(), used)), r.summ[used.numpy()])
    assert np.array_equal(cnt_h.numpy(), r.cnt) and np.array_equal(sel_h.numpy(), r.sel)
    assert np.abs(out_h.numpy().astype(np.float64) - r.out).max() <= OUT_TOL


def test_host_tier_quantised_pages_match_device_pools():
    """2-bit pages in the host tier as well: the quantised pool and the bf16
    pools in host memory give the device-pool results bit for bit."""
    print("host-tier quantised case", flush=True)
    R = 4
    w = workloads.make("llama8b_b32_32k", device="cpu", seed=6, batch=32, seq_len=1500, seq_len_min=700)
    lay, pol = api.layout_of(w), api.policy_of(w)
    bat = api.Batch(w.page_table.to(DEV), w.seq_lens.to(DEV), w.spec.num_q_heads)
    msel = api.max_sel(lay, pol, bat.max_pages)
    kd, vd = w.k_pool.to(DEV), w.v_pool.to(DEV)
    summ_d = torch.zeros((lay.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16,
                         device=DEV)
    api.build_summaries(lay, bat, kd, summ_d)
    summ_h = summ_d.clone()
    qd = api.new_quant_pool(lay, DEV)
    api.quantize_pages(lay, bat, R, kd, vd, qd)
    kh, vh, qh = api.host_pool_like(w.k_pool), api.host_pool_like(w.v_pool), api.host_pool_like(qd)
    runs = []
    for kp, vp, qp, summ in ((kd, vd, qd, summ_d), (kh, vh, qh, summ_h)):
        ws = api.new_workspace(lay, bat, pol, msel, DEV)
        sel = torch.empty((32, lay.num_kv_heads, msel), dtype=torch.int32, device=DEV)
        cnt = torch.empty((32, lay.num_kv_heads), dtype=torch.int32, device=DEV)
        out = api.decode_step_quant(lay, bat, pol, R, w.q.to(DEV), kp, vp, summ, qp, w.scale, ws, msel,
                                    k_new=w.k_new.to(DEV), v_new=w.v_new.to(DEV), sel=sel, sel_count=cnt)
        torch.cuda.synchronize()
        runs.append((out.cpu(), sel.cpu(), cnt.cpu()))
    assert torch.equal(runs[0][1], runs[1][1]) and torch.equal(runs[0][2], runs[1][2])
    assert torch.equal(runs[0][0].view(torch.int32), runs[1][0].view(torch.int32))
    assert torch.equal(qh.host, qd.cpu())
    assert torch.equal(kh.host.view(torch.int16), kd.cpu().view(torch.int16))
