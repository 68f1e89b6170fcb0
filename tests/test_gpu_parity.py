"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: summaries and selected page ids bit-exact, every fp32 score within its
own error bound of the exact score, attention outputs within 5e-3 max-abs.
Small cases and the full-size workloads alike run the oracle on every
sequence (the full sizes in chunks of sequences re-packed into small pools).
"""
import numpy as np
import pytest
import torch

from query_aware_sparse_paged_amd import api, workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_cases import DEV, check_every_sequence, compare, run_gpu, run_oracle


def _small(name, **kw):
    return workloads.make(name, device="cpu", **kw)


# ----------------------------------------------------------------------------
# small cases: oracle on every sequence
# ----------------------------------------------------------------------------

def test_tiny_config_exact():
    w = _small("tiny_b1_4k")
    g = run_gpu(w)
    r = run_oracle(w, api.policy_of(w), g.max_sel)
    k_phys = w.page_table[0, :256].long()
    assert np.array_equal(workloads.bits(api.summary_rows(g.summ.cpu(), k_phys)), r.summ[k_phys.numpy()])
    compare(g, r, what="tiny_b1_4k")
    assert (g.cnt == 37).all()


@pytest.mark.parametrize("seed", [0, 1])
def test_llama_shape_ragged_small(seed):
    w = _small("llama8b_b32_32k", seed=seed, batch=3, seq_len=3001, seq_len_min=1500)
    g = run_gpu(w)
    r = run_oracle(w, api.policy_of(w), g.max_sel)
    compare(g, r, what="llama small")


def test_needles_small_all_found():
    w = _small("needle_b8_128k", batch=2, seq_len=12000)
    g = run_gpu(w)
    r = run_oracle(w, api.policy_of(w), g.max_sel)
    compare(g, r, what="needle small")
    for b in range(2):
        pages = set((w.needle_pos[b] // 16).tolist())
        for h in range(8):
            assert pages <= set(g.sel[b, h, :g.cnt[b, h]].tolist())


def test_ragged_mixed_static_small():
    w = _small("ragged_b64_mixed", batch=5, seq_len=4000, seq_len_min=1)
    g = run_gpu(w)
    r = run_oracle(w, api.policy_of(w), g.max_sel)
    compare(g, r, what="ragged small")


@pytest.mark.parametrize("lens,pol", [
    ([1, 16, 17, 33], api.Policy(1, 1, 2)),
    ([5, 40, 129, 300], api.Policy(0, 0, 3)),
    ([200, 201, 64, 95], api.Policy(3, 2, 0)),
    ([250, 7, 90, 1000], api.Policy(1, 4, 1000)),
    ([513, 700, 31, 48], api.Policy(2, 1, 5, 3, 40, [1, 0, 1, 0, 0, 0, 1, 1])),
])
def test_edges(lens, pol):
    w = _small("tiny_b1_4k", batch=len(lens), seq_len=max(lens))
    w.seq_lens[:] = torch.tensor(lens, dtype=torch.int32)
    # the new token of each sequence is the one at its (new) last position
    ps = 16
    for b, L in enumerate(lens):
        phys = int(w.page_table[b, (L - 1) // ps])
        w.k_new[b] = w.k_pool[phys, :, (L - 1) % ps, :]
        w.v_new[b] = w.v_pool[phys, :, :, (L - 1) % ps]
    g = run_gpu(w, pol=pol)
    r = run_oracle(w, pol, g.max_sel)
    compare(g, r, what="edge %s" % lens)


@pytest.mark.parametrize("sink,window", [(0, 40), (5, 0), (0, 0), (33, 31), (4000, 16), (16, 17)])
def test_static_heads_page_ranges(sink, window):
    """A static head's list is two page ranges computed from the length (in
    the one-kernel step, with no selection pass): pages that hold sink tokens,
    then pages that hold window tokens; cases at page boundaries, with an empty
    sink or window or both, and with the two ranges meeting or overlapping."""
    lens = [1, 15, 16, 17, 31, 32, 33, 100]
    w = _small("tiny_b1_4k", batch=len(lens), seq_len=max(lens))
    w.seq_lens[:] = torch.tensor(lens, dtype=torch.int32)
    for b, L in enumerate(lens):
        phys = int(w.page_table[b, (L - 1) // 16])
        w.k_new[b] = w.k_pool[phys, :, (L - 1) % 16, :]
        w.v_new[b] = w.v_pool[phys, :, :, (L - 1) % 16]
    pol = api.Policy(1, 2, 3, sink, window, [1, 1, 0, 1, 0, 1, 1, 0])
    lay = api.layout_of(w)
    bat = api.Batch(w.page_table, w.seq_lens, w.spec.num_q_heads)
    assert api.decode_step_path(lay, bat, pol, api.max_sel(lay, pol, bat.max_pages)) == api.PATH_ONE_KERNEL
    g = run_gpu(w, pol=pol)
    r = run_oracle(w, pol, g.max_sel)
    compare(g, r, what="static page ranges %d/%d" % (sink, window))


def test_all_static_heads_without_summaries():
    w = _small("ragged_b64_mixed", batch=3, seq_len=3000, seq_len_min=10)
    pol = api.Policy(0, 0, 0, 4, 100, [1] * 8)
    g = run_gpu(w, pol=pol, use_summ=False)
    r = run_oracle(w, pol, g.max_sel)
    compare(g, r, check_scores=False, what="all static")


def test_zero_query_ties_go_to_lowest_ids():
    w = _small("llama8b_b32_32k", batch=2, seq_len=3000)
    w.q.zero_()
    g = run_gpu(w)
    r = run_oracle(w, api.policy_of(w), g.max_sel)
    compare(g, r, what="zero query")
    P = 188
    want = list(range(0, 1 + 119)) + list(range(P - 8, P))
    assert g.sel[0, 0, :128].tolist() == want


def test_integer_keys_many_ties():
    w = _small("tiny_b1_4k", batch=2, seq_len=1500)
    gen = torch.Generator().manual_seed(3)
    w.k_pool.copy_(torch.randint(-2, 3, w.k_pool.shape, generator=gen).to(torch.bfloat16))
    w.q.copy_(torch.randint(-1, 2, w.q.shape, generator=gen).to(torch.bfloat16))
    for b in range(2):
        L = int(w.seq_lens[b])
        w.k_new[b] = w.k_pool[int(w.page_table[b, (L - 1) // 16]), :, (L - 1) % 16, :]
    g = run_gpu(w)
    r = run_oracle(w, api.policy_of(w), g.max_sel)
    compare(g, r, what="integer ties")


def test_exact_rescore_needs_tiny_terms():
    """Pages whose bounds differ only through a term 2^-80 below the others:
    the exact re-score must keep it (1 + 2^-53 + 2^-80 rounds up, 1 + 2^-53
    ties to even and rounds down)."""
    w = _small("tiny_b1_4k", batch=1, seq_len=16 * 12)
    w.q.zero_()
    w.k_pool.zero_()
    f = lambda x: torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)
    # q head 0 of KV head 0: channel 0 = 1, channel 1 = 2^-27, channel 2 = 2^-40
    w.q[0, 0, 0], w.q[0, 0, 1], w.q[0, 0, 2] = f(1.0), f(2.0 ** -27), f(2.0 ** -40)
    pt = w.page_table[0]
    # page 3: 1 + 2^-53 + 2^-80 -> 1 + 2^-52 ; page 5: 1 + 2^-53 -> 1 ;
    # page 7: 1 + 2^-52 exactly (2^-26 * 2^-26) -> ties with page 3, lower id wins
    for j, (c1, c2) in {3: (2.0 ** -26, 2.0 ** -40), 5: (2.0 ** -26, 0.0)}.items():
        w.k_pool[int(pt[j]), 0, :, 0] = f(1.0)
        w.k_pool[int(pt[j]), 0, :, 1] = f(c1)
        w.k_pool[int(pt[j]), 0, :, 2] = f(c2)
    w.k_pool[int(pt[7]), 0, :, 0] = f(1.0)
    w.k_pool[int(pt[7]), 0, :, 1] = f(2.0 ** -25)
    w.k_new.zero_()
    pol = api.Policy(1, 1, 1)
    g = run_gpu(w, pol=pol, append=False)
    r = run_oracle(w, pol, g.max_sel)
    compare(g, r, what="tiny terms")
    assert g.sel[0, 0, :3].tolist() == [0, 3, 11]


def test_append_updates_summaries_incrementally():
    """Append 16 tokens one at a time (at most one new page per sequence, the
    spare one the generator maps); summaries must equal a rebuild."""
    w = _small("llama8b_b32_32k", batch=3, seq_len=100, seq_len_min=40)
    lay, pol = api.layout_of(w), api.policy_of(w)
    kp, vp = w.k_pool.to(DEV), w.v_pool.to(DEV)
    pt = w.page_table.to(DEV)
    lens = w.seq_lens.clone()
    summ = torch.zeros((lay.num_pool_pages, 8, 2, 128), dtype=torch.bfloat16, device=DEV)
    api.build_summaries(lay, api.Batch(pt, lens.to(DEV), 32), kp, summ)
    gen = torch.Generator().manual_seed(9)
    for step in range(16):
        kn = torch.randn((3, 8, 128), generator=gen).to(torch.bfloat16)
        vn = torch.randn((3, 8, 128), generator=gen).to(torch.bfloat16)
        # the spare page covers a crossing into a new page
        api.append_kv(lay, api.Batch(pt, lens.to(DEV), 32), pol, kn.to(DEV), vn.to(DEV), kp, vp, summ)
        lens += 1
    torch.cuda.synchronize()
    rebuilt = torch.zeros_like(summ)
    api.build_summaries(lay, api.Batch(pt, lens.to(DEV), 32), kp, rebuilt)
    torch.cuda.synchronize()
    used = []
    for b in range(3):
        used += w.page_table[b, :(int(lens[b]) + 15) // 16].tolist()
    used = torch.tensor(used, device=DEV)
    assert torch.equal(summ[used].view(torch.int16), rebuilt[used].view(torch.int16))
    import oracle
    from gpu_cases import olayout
    osumm = oracle.summaries(olayout(lay), w.page_table.numpy(), lens.numpy(), 32, workloads.bits(kp))
    assert np.array_equal(workloads.bits(api.summary_rows(summ, used)), osumm[used.cpu().numpy()])


def test_split_entry_points_match_decode_step():
    w = _small("llama8b_b32_32k", batch=2, seq_len=2500)
    lay, pol = api.layout_of(w), api.policy_of(w)
    g = run_gpu(w)
    q, kp, vp = w.q.to(DEV), w.k_pool.to(DEV), w.v_pool.to(DEV)
    bat = api.Batch(w.page_table.to(DEV), w.seq_lens.to(DEV), 32)
    sc = api.score_pages(lay, bat, pol, q, g.summ)
    sel, cnt = api.select_topk(lay, bat, pol, q, g.summ, sc)
    ws = api.new_workspace(lay, bat, pol, sel.shape[2], DEV)
    out = api.sparse_paged_decode(lay, bat, pol, q, kp, vp, sel, cnt, w.scale, ws)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), g.sel)
    assert np.array_equal(out.cpu().numpy(), g.out)


@pytest.mark.parametrize("name,kw", [
    ("llama8b_b32_32k", dict(batch=32, seq_len=2500, seq_len_min=300)),      # 256 units: one-kernel step
    ("ragged_b64_mixed", dict(batch=26, seq_len=3000, seq_len_min=1)),       # 208 units, static heads
])
def test_single_kernel_step_matches_oracle_and_kernel_chain(name, kw):
    """Many units: qasp_decode_step runs the whole step as one kernel; it must
    match the oracle and the score -> select -> decode kernel chain."""
    w = _small(name, **kw)
    lay, pol = api.layout_of(w), api.policy_of(w)
    assert w.spec.batch * lay.num_kv_heads >= 200
    g = run_gpu(w)
    r = run_oracle(w, pol, g.max_sel)
    compare(g, r, what="one-kernel step " + name)
    q, kp, vp = w.q.to(DEV), w.k_pool.to(DEV), w.v_pool.to(DEV)
    bat = api.Batch(w.page_table.to(DEV), w.seq_lens.to(DEV), w.spec.num_q_heads)
    sc = api.score_pages(lay, bat, pol, q, g.summ)
    sel, cnt = api.select_topk(lay, bat, pol, q, g.summ, sc, max_sel_n=g.max_sel)
    ws = api.new_workspace(lay, bat, pol, g.max_sel, DEV)
    out = api.sparse_paged_decode(lay, bat, pol, q, kp, vp, sel, cnt, w.scale, ws)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), g.sel) and np.array_equal(cnt.cpu().numpy(), g.cnt)
    assert np.abs(out.cpu().numpy() - g.out).max() <= 1e-5


@pytest.mark.parametrize("batch,seq_len,top_k", [
    (32, 9000, 520),      # 529 pages per unit: more than 64 per wave of the one-kernel step
    (32, 8500, 100000),   # every page of every unit selected (about 530)
    (3, 9000, 520),       # the kernel chain
])
def test_large_selections(batch, seq_len, top_k):
    """Selections of more than 512 pages (64 per wave of an 8-wave block): each
    wave walks its list in chunks of 64 pages."""
    print("large selections", batch, seq_len, top_k, flush=True)
    w = workloads.make("llama8b_b32_32k", device=DEV, batch=batch, seq_len=seq_len, seq_len_min=seq_len - 300)
    pol = api.Policy(1, 8, top_k)
    g = run_gpu(w, pol=pol)
    P = (w.seq_lens.cpu().numpy() + 15) // 16
    assert (g.cnt == np.minimum(P, 1 + 8 + top_k)[:, None]).all() and g.cnt.min() > 512
    check_every_sequence(w, g, pol=pol, what="large selections")
    del w, g
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("batch", [32, 3])   # one-kernel step; kernel chain
@pytest.mark.parametrize("local,boost", [(None, 1.0), (0, 6.0)])
def test_step_appends(batch, local, boost):
    """The decode step writes the token at L-1 and updates its summary (the
    one-kernel step in its last wave, the chain in its scoring kernel, or in a
    kernel of its own when the page is a candidate).  With no local window the
    last page is a candidate, and a large new key makes it the best page: it
    must be scored with the new token."""
    w = _small("llama8b_b32_32k", batch=batch, seq_len=700, seq_len_min=600)
    lay, pol = api.layout_of(w), api.policy_of(w)
    if local is not None:
        pol = api.Policy(pol.n_sink_pages, local, pol.top_k)
    gen = torch.Generator().manual_seed(5)
    new_k = (torch.randn(w.k_new.shape, generator=gen) * boost).to(torch.bfloat16)
    new_v = torch.randn(w.v_new.shape, generator=gen).to(torch.bfloat16)
    kp, vp = w.k_pool.to(DEV), w.v_pool.to(DEV)
    bat = api.Batch(w.page_table.to(DEV), w.seq_lens.to(DEV), 32)
    summ = torch.zeros((lay.num_pool_pages, 8, 2, 128), dtype=torch.bfloat16, device=DEV)
    # summaries of the cache before the new token: lengths L-1
    api.build_summaries(lay, api.Batch(bat.page_table, (bat.seq_lens - 1).contiguous(), 32), kp, summ)
    msel = api.max_sel(lay, pol, bat.max_pages)
    ws = api.new_workspace(lay, bat, pol, msel, DEV)
    sel = torch.full((batch, lay.num_kv_heads, msel), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((batch, lay.num_kv_heads), -7, dtype=torch.int32, device=DEV)
    out = api.decode_step(lay, bat, pol, w.q.to(DEV), kp, vp, summ, w.scale, ws, msel,
                          k_new=new_k.to(DEV), v_new=new_v.to(DEV), sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    # the oracle sees the pool with the token written and summaries from scratch
    for b in range(batch):
        L = int(w.seq_lens[b])
        phys = int(w.page_table[b, (L - 1) // 16])
        w.k_pool[phys, :, (L - 1) % 16, :] = new_k[b]
        w.v_pool[phys, :, :, (L - 1) % 16] = new_v[b]
    assert torch.equal(kp.cpu().view(torch.int16), w.k_pool.view(torch.int16))
    assert torch.equal(vp.cpu().view(torch.int16), w.v_pool.view(torch.int16))
    r = run_oracle(w, pol, msel)
    used = w.page_table[:, :44].reshape(-1).long()
    used = used[used >= 0]
    assert np.array_equal(workloads.bits(api.summary_rows(summ.cpu(), used)), r.summ[used.numpy()])
    assert np.array_equal(cnt.cpu().numpy(), r.cnt) and np.array_equal(sel.cpu().numpy(), r.sel)
    assert np.abs(out.cpu().numpy().astype(np.float64) - r.out).max() <= 5e-3
    if local == 0:  # the test is only sensitive if the boosted last pages are chosen
        last = (w.seq_lens.numpy() - 1) // 16
        chosen = (r.sel == last[:, None, None]).any(-1)
        assert chosen.mean() > 0.5


@pytest.mark.parametrize("batch", [3, 32])   # kernel chain; one-kernel step
def test_stale_non_finite_tail_is_not_read(batch):
    """Pool slots past each length hold NaN keys and values: the output must
    not see them."""
    w = _small("llama8b_b32_32k", batch=batch, seq_len=900, seq_len_min=400)
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
    for b in range(batch):
        L = int(w.seq_lens[b])
        if L % 16:
            phys = int(w.page_table[b, (L - 1) // 16])
            w.k_pool[phys, :, L % 16:, :] = nan
            w.v_pool[phys, :, :, L % 16:] = nan
    g = run_gpu(w)
    assert np.isfinite(g.out).all()
    r = run_oracle(w, api.policy_of(w), g.max_sel)
    compare(g, r, what="NaN tail")


@pytest.mark.parametrize("batch", [4, 32])   # kernel chain; one-kernel step
def test_repeated_calls_are_deterministic(batch):
    w = _small("llama8b_b32_32k", batch=batch, seq_len=4000, seq_len_min=3000)
    a = run_gpu(w)
    b = run_gpu(w)
    assert np.array_equal(a.sel, b.sel) and np.array_equal(a.out, b.out)


# ----------------------------------------------------------------------------
# full-size workloads: the oracle on every sequence (chunks re-packed into
# small pools), in the launch configuration the benchmark times
# ----------------------------------------------------------------------------

def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_full_llama8b_b32_32k():
    print("full llama8b_b32_32k", flush=True)
    w = workloads.make("llama8b_b32_32k", device=DEV)
    g = run_gpu(w)
    assert (g.cnt == 128).all()
    assert (np.diff(g.sel, axis=2) > 0).all()
    check_every_sequence(w, g, what="llama8b_b32_32k")
    del w, g
    _free()


def test_full_needle_b8_128k():
    print("full needle_b8_128k", flush=True)
    w = workloads.make("needle_b8_128k", device=DEV)
    g = run_gpu(w)
    assert (g.cnt == 256).all()
    for b in range(8):
        pages = set((w.needle_pos[b] // 16).tolist())
        for h in range(8):
            assert pages <= set(g.sel[b, h].tolist())
    check_every_sequence(w, g, chunk=1, what="needle_b8_128k")
    del w, g
    _free()


def test_full_ragged_b64_mixed():
    print("full ragged_b64_mixed", flush=True)
    w = workloads.make("ragged_b64_mixed", device=DEV)
    g = run_gpu(w)
    assert (g.cnt[:, 4:] == 64).all()
    assert ((g.cnt[:, :4] >= 65) & (g.cnt[:, :4] <= 66)).all()
    check_every_sequence(w, g, what="ragged_b64_mixed")
    del w, g
    _free()
