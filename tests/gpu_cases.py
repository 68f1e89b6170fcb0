"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and run the oracle on the same inputs (or on a sampled sequence of them)."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import oracle
from query_aware_sparse_paged_amd import api, workloads

DEV = torch.device("cuda:0")
OUT_TOL = 5e-3   # max-abs error bound on the attention output


def olayout(lay: api.Layout) -> oracle.Layout:
    return oracle.Layout(lay.num_pool_pages, lay.page_size, lay.num_kv_heads, lay.head_dim_k,
                         lay.head_dim_v, lay.v_from_k)


def opolicy(pol: api.Policy) -> oracle.Policy:
    return oracle.Policy(pol.n_sink_pages, pol.n_local_pages, pol.top_k, pol.sink_tokens,
                         pol.window_tokens, pol.static_heads)


@dataclass
class GpuRun:
    out: np.ndarray       # fp32 [B][Hq][Dv]
    sel: np.ndarray       # int32 [B][Hkv][max_sel]
    cnt: np.ndarray       # int32 [B][Hkv]
    scores: np.ndarray    # fp32 [B][Hkv][max_pages][4] (qasp_score records) or None
    summ: torch.Tensor    # device summary pool
    max_sel: int


def run_gpu(w, lay=None, pol=None, with_scores=True, append=True, use_summ=True) -> GpuRun:
    """Builds summaries, then one decode step through qasp_decode_step (with
    the append of the token at L-1, which rewrites the same values)."""
    lay = lay or api.layout_of(w)
    pol = pol or api.policy_of(w)
    t = lambda x: None if x is None else x.to(DEV)
    q, kp, vp = t(w.q), t(w.k_pool), t(w.v_pool)
    bat = api.Batch(t(w.page_table), t(w.seq_lens), w.spec.num_q_heads)
    msel = api.max_sel(lay, pol, bat.max_pages)
    summ = None
    if use_summ:
        summ = torch.zeros((lay.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16,
                           device=DEV)
        api.build_summaries(lay, bat, kp, summ)
    scores = None
    if with_scores and use_summ:
        scores = api.score_pages(lay, bat, pol, q, summ).cpu().numpy()
    ws = api.new_workspace(lay, bat, pol, msel, DEV)
    sel = torch.full((w.spec.batch, lay.num_kv_heads, msel), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((w.spec.batch, lay.num_kv_heads), -7, dtype=torch.int32, device=DEV)
    out = api.decode_step(lay, bat, pol, q, kp, vp, summ, w.scale, ws, msel,
                          k_new=t(w.k_new) if append else None, v_new=t(w.v_new) if append else None,
                          sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    return GpuRun(out.cpu().numpy(), sel.cpu().numpy(), cnt.cpu().numpy(), scores, summ, msel)


@dataclass
class OracleRun:
    out: np.ndarray
    sel: np.ndarray
    cnt: np.ndarray
    scores: np.ndarray
    summ: np.ndarray
    page_table: np.ndarray


def run_oracle(w, pol: api.Policy, max_sel_n: int, seqs=None) -> OracleRun:
    """Oracle on the whole workload (seqs None) or on a sub-batch of sequences
    re-packed into a small pool (logical page ids are unchanged)."""
    spec = w.spec
    lay = api.layout_of(w)
    if seqs is None:
        pt = w.page_table.cpu().numpy()
        sl = w.seq_lens.cpu().numpy()
        q = workloads.bits(w.q)
        k = workloads.bits(w.k_pool)
        v = None if w.v_pool is None else workloads.bits(w.v_pool)
        olay = olayout(lay)
    else:
        seqs = list(seqs)
        pt_full = w.page_table[seqs]                                   # [n][stride]
        stride = pt_full.shape[1]
        valid = pt_full >= 0
        phys = pt_full[valid].long()
        k = workloads.bits(w.k_pool[phys])
        v = None if w.v_pool is None else workloads.bits(w.v_pool[phys])
        pt = np.full((len(seqs), stride), -1, np.int32)
        pt[valid.cpu().numpy()] = np.arange(phys.numel(), dtype=np.int32)
        sl = w.seq_lens[seqs].cpu().numpy()
        q = workloads.bits(w.q[seqs])
        olay = oracle.Layout(int(phys.numel()), lay.page_size, lay.num_kv_heads, lay.head_dim_k,
                             lay.head_dim_v, lay.v_from_k)
    opol = opolicy(pol)
    summ = oracle.summaries(olay, pt, sl, spec.num_q_heads, k)
    scores = oracle.scores(olay, pt, sl, q, summ, opol)
    out, sel, cnt = oracle.decode(olay, pt, sl, q, k, v, summ, opol, w.scale, num_threads=8,
                                  max_sel_n=max_sel_n)
    return OracleRun(out, sel, cnt, scores, summ, pt)


def gpu_summaries_of(g: GpuRun, w, seqs, ref: OracleRun):
    """GPU summaries of the sampled sequences' pages, in the sub-pool order."""
    pt_full = w.page_table[list(seqs)]
    phys = pt_full[pt_full >= 0].long().to(DEV)
    s = workloads.bits(g.summ[phys])
    return s


def compare(g: GpuRun, r: OracleRun, seqs=None, check_scores=True, what=""):
    """Selections exact, outputs within OUT_TOL, scores inside their bounds."""
    idx = slice(None) if seqs is None else list(seqs)
    gsel, gcnt, gout = g.sel[idx], g.cnt[idx], g.out[idx]
    assert np.array_equal(gcnt, r.cnt), "%s: selection counts differ" % what
    assert np.array_equal(gsel, r.sel), "%s: selected pages differ (first diff at %s)" % (
        what, np.argwhere(gsel != r.sel)[:3].tolist())
    err = np.abs(gout.astype(np.float64) - r.out)
    assert np.isfinite(gout).all(), "%s: non-finite output" % what
    assert err.max() <= OUT_TOL, "%s: max abs error %.3g" % (what, err.max())
    if check_scores and g.scores is not None:
        gs = g.scores[idx]
        val, bound = gs[..., 0].astype(np.float64), gs[..., 1].astype(np.float64)
        mp = min(val.shape[-1], r.scores.shape[-1])
        ref = r.scores[..., :mp]
        val, bound = val[..., :mp], bound[..., :mp]
        cand = np.isfinite(ref)
        assert np.array_equal(np.isfinite(val), cand), "%s: candidate sets differ" % what
        assert np.all(np.abs(val[cand] - ref[cand]) <= bound[cand]), "%s: score outside its bound" % what
    return float(err.max())
