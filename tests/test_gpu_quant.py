"""GPU parity of the 2-bit quantised pages (qasp_quantize_pages,
qasp_decode_step_quant): KIVI-style codes (2 bits, groups of 32; SCBench
notes, the method table) for the pages outside a bf16 residual region
(SparseEngine article, decode-hook paragraph).

Oracle: the token written into the bf16 pools, summaries from scratch,
oracle.scores / select (unchanged by quantisation), oracle.quantize over the
pages j < P - R, oracle.attend_quant.  Bar: bf16 pools, summaries, selections
and every quantised page-head (codes and binary16 pairs, decoded from the
packed layout below) bit-exact; outputs within 5e-3 max-abs."""
import numpy as np
import pytest
import torch

from query_aware_sparse_paged_amd import api, workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    from gpu_cases import DEV, OUT_TOL, olayout, opolicy


def _pairs(words):
    """Code words [..., 2] (uint32) -> codes [..., 16, 2]: pair p sits in word
    p // 8 rotated left by 2 (p % 8) from first code at bits 5-6, second at
    bits 21-22."""
    out = np.zeros(words.shape[:-1] + (16, 2), np.uint8)
    for p in range(16):
        w = words[..., p // 8].astype(np.uint64)
        a = 2 * (p % 8)
        r = ((w >> a) | (w << (32 - a))) & 0xffffffff if a else w
        out[..., p, 0] = (r >> 5) & 3
        out[..., p, 1] = (r >> 21) & 3
    return out


def unpack(qpool: np.ndarray):
    """Packed quantised pool [pool][Hkv][1536] -> the oracle's logical arrays
    (key codes [pool][Hkv][16][128], key pairs [pool][Hkv][16][4][2], value
    codes, value pairs), per the library header's layout: key words of token
    t, lane group kg at byte 32t + 8kg, pair 4i + k = channels 32i + 8kg + 2k
    and + 1; value words of channel n, lane group kg at byte 768 + 8(4n + kg),
    pair 2i + h = tokens 4kg + 2h and + 1 of channel 16i + n."""
    P, H = qpool.shape[:2]
    kw = qpool[..., :512].copy().view(np.uint32).reshape(P, H, 16, 4, 2)       # t, kg, word
    kc = _pairs(kw).reshape(P, H, 16, 4, 4, 4, 2)                              # t, kg, i, k, e
    kc = kc.transpose(0, 1, 2, 4, 3, 5, 6).reshape(P, H, 16, 128)
    km = qpool[..., 512:768].copy().view(np.uint16).reshape(P, H, 16, 4, 2)
    vw = qpool[..., 768:1280].copy().view(np.uint32).reshape(P, H, 16, 4, 2)   # n, kg, word
    vc = _pairs(vw).reshape(P, H, 16, 4, 8, 2, 2)                              # n, kg, i, h, e
    vc = vc.transpose(0, 1, 3, 5, 6, 4, 2).reshape(P, H, 16, 128)              # (kg, h, e) -> t, (i, n) -> dv
    vm = qpool[..., 1280:].copy().view(np.uint16).reshape(P, H, 16, 4, 2)
    return kc, km, vc, vm


@pytest.mark.parametrize("name,batch,R,kw", [
    ("llama8b_b32_32k", 3, 2, dict(seq_len=1500, seq_len_min=700)),              # kernel chain, split units
    ("llama8b_b32_32k", 32, 8, dict(seq_len=1300, seq_len_min=500)),              # many units: fused selection
    ("llama8b_b32_32k", 4, 1, dict(seq_len=900, seq_len_min=600, top_k=200)),     # every page selected
    ("ragged_b64_mixed", 6, 3, dict(seq_len=3000, seq_len_min=1200)),             # static heads
    ("ragged_b64_mixed", 32, 5, dict(seq_len=2600, seq_len_min=900))])            # static heads, many units
def test_quant_step_matches_oracle(name, batch, R, kw):
    print("quantised-page case", name, batch, R, kw, flush=True)
    w = workloads.make(name, device="cpu", seed=13, batch=batch, **kw)
    # some sequences whose token opens a new page (quantised inside the step)
    sl = w.seq_lens.clone()
    for b in range(0, batch, 2):
        sl[b] = 16 * ((int(sl[b]) - 1) // 16) + 1
    w.seq_lens = sl
    gen = torch.Generator().manual_seed(4)
    k_new = torch.randn(w.k_new.shape, generator=gen).to(torch.bfloat16)
    v_new = torch.randn(w.v_new.shape, generator=gen).to(torch.bfloat16)
    lay, pol = api.layout_of(w), api.policy_of(w)
    Hq = w.spec.num_q_heads
    bat = api.Batch(w.page_table.to(DEV), sl.to(DEV), Hq)
    bat_before = api.Batch(bat.page_table, (bat.seq_lens - 1).contiguous(), Hq)
    msel = api.max_sel(lay, pol, bat.max_pages)
    kp, vp = w.k_pool.to(DEV), w.v_pool.to(DEV)
    summ = torch.zeros((lay.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16, device=DEV)
    api.build_summaries(lay, bat_before, kp, summ)
    qpool = api.new_quant_pool(lay, DEV)
    api.quantize_pages(lay, bat_before, R, kp, vp, qpool)
    ws = api.new_workspace(lay, bat, pol, msel, DEV)
    sel = torch.full((batch, lay.num_kv_heads, msel), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((batch, lay.num_kv_heads), -7, dtype=torch.int32, device=DEV)
    out = api.decode_step_quant(lay, bat, pol, R, w.q.to(DEV), kp, vp, summ, qpool, w.scale, ws, msel,
                                k_new=k_new.to(DEV), v_new=v_new.to(DEV), sel=sel, sel_count=cnt)
    torch.cuda.synchronize()

    ps = lay.page_size
    for b in range(batch):
        L = int(sl[b])
        phys = int(w.page_table[b, (L - 1) // ps])
        w.k_pool[phys, :, (L - 1) % ps, :] = k_new[b]
        w.v_pool[phys, :, :, (L - 1) % ps] = v_new[b]
    assert torch.equal(kp.cpu().view(torch.int16), w.k_pool.view(torch.int16))
    assert torch.equal(vp.cpu().view(torch.int16), w.v_pool.view(torch.int16))
    olay, opol = olayout(lay), opolicy(pol)
    pt_np, sl_np = w.page_table.numpy(), sl.numpy()
    kbits, vbits = workloads.bits(w.k_pool), workloads.bits(w.v_pool)
    rs = oracle.summaries(olay, pt_np, sl_np, Hq, kbits)
    sc = oracle.scores(olay, pt_np, sl_np, workloads.bits(w.q), rs, opol)
    rsel, rcnt = oracle.select(olay, pt_np, sl_np, Hq, sc, opol, max_sel_n=msel)
    gsel, gcnt = sel.cpu().numpy(), cnt.cpu().numpy()
    assert np.array_equal(gcnt, rcnt)
    for b in range(batch):
        for g in range(lay.num_kv_heads):
            assert np.array_equal(gsel[b, g, :gcnt[b, g]], rsel[b, g, :rcnt[b, g]]), (b, g)
    qz = oracle.quantize(olay, pt_np, sl_np, Hq, R, kbits, vbits)
    kc, km, vc, vm = unpack(qpool.cpu().numpy())
    n_pages = 0
    for b in range(batch):
        P = (int(sl[b]) + ps - 1) // ps
        for j in range(P - R):
            ph = int(w.page_table[b, j])
            assert np.array_equal(kc[ph], qz.k_codes[ph]) and np.array_equal(km[ph], qz.k_meta[ph]), (b, j)
            assert np.array_equal(vc[ph], qz.v_codes[ph]) and np.array_equal(vm[ph], qz.v_meta[ph]), (b, j)
            n_pages += 1
    assert n_pages > 0
    ref = oracle.attend_quant(olay, pt_np, sl_np, workloads.bits(w.q), kbits, vbits, qz, rsel, rcnt, opol, w.scale)
    gout = out.cpu().numpy()
    assert np.isfinite(gout).all()
    err = np.abs(gout.astype(np.float64) - ref).max()
    assert err <= OUT_TOL, err
    # the quantised pages change the result (the test would not see a bf16 read)
    plain = oracle.attend(olay, pt_np, sl_np, workloads.bits(w.q), kbits, vbits, rsel, rcnt, opol, w.scale)
    assert np.abs(plain - ref).max() > 10 * OUT_TOL
