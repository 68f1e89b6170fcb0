"""qasp_decode_step_noalloc (the step with the library's static per-device
workspace) against qasp_decode_step with a caller's workspace: two calls in
a row, the second with a smaller input, each bit-identical to the existing
entry point on the same inputs (same kernels, same launch shapes)."""
import pytest
import torch

from query_aware_sparse_paged_amd import api, workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_cases import DEV


def _inputs(name, batch, seq_len):
    w = workloads.make(name, device=DEV, batch=batch, seq_len=seq_len, seq_len_min=seq_len // 2)
    lay, pol = api.layout_of(w), api.policy_of(w)
    bat = api.Batch(w.page_table, w.seq_lens, w.spec.num_q_heads)
    msel = api.max_sel(lay, pol, bat.max_pages)
    summ = torch.zeros((lay.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16, device=DEV)
    api.build_summaries(lay, bat, w.k_pool, summ)
    return w, lay, pol, bat, msel, summ


def _outputs(w, lay, msel):
    out = torch.full((w.spec.batch, w.spec.num_q_heads, lay.head_dim_v), float("nan"), device=DEV)
    sel = torch.full((w.spec.batch, lay.num_kv_heads, msel), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((w.spec.batch, lay.num_kv_heads), -7, dtype=torch.int32, device=DEV)
    return out, sel, cnt


@pytest.mark.parametrize("name,first,second", [
    ("llama8b_b32_32k", (4, 3000), (2, 1500)),     # kernel chain: scores, selection, partials in the scratch
    ("mla_b16_64k", (2, 9000), (1, 4000)),         # latent heads: split partials in the scratch
    ("llama8b_b32_32k", (32, 1200), (26, 900)),    # one-kernel step (no scratch used)
])
def test_noalloc_step_matches_decode_step(name, first, second):
    for batch, seq_len in (first, second):
        print("no-alloc step", name, batch, seq_len, flush=True)
        w, lay, pol, bat, msel, summ = _inputs(name, batch, seq_len)
        ws = api.new_workspace(lay, bat, pol, msel, DEV)
        assert ws.numel() <= api.scratch_bytes()
        ref = _outputs(w, lay, msel)
        api.decode_step(lay, bat, pol, w.q, w.k_pool, w.v_pool, summ, w.scale, ws, msel, k_new=w.k_new,
                        v_new=w.v_new, out=ref[0], sel=ref[1], sel_count=ref[2])
        got = _outputs(w, lay, msel)
        api.decode_step_noalloc(lay, bat, pol, w.q, w.k_pool, w.v_pool, summ, w.scale, msel, k_new=w.k_new,
                                v_new=w.v_new, out=got[0], sel=got[1], sel_count=got[2])
        torch.cuda.synchronize()
        assert torch.equal(got[2], ref[2]) and torch.equal(got[1], ref[1])
        assert torch.equal(got[0].view(torch.int32), ref[0].view(torch.int32))
        assert not torch.isnan(got[0]).any()
        del w, summ, ws, ref, got
    torch.cuda.synchronize()
