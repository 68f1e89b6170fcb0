"""Pins of the oracle's multi-query step (several draft tokens per sequence).

Readings (stated beside orc_scores_multi in the oracle's header): the draft
tokens sit at positions L - nq ... L - 1 of a sequence of length L; they share
one selection per (sequence, KV head), scored with the maximum bound over every
draft query's heads of the group; query i attends causally, to the tokens at
positions <= L - nq + i of the shared pages; a static head reads the union of
the queries' sink + window token sets.

Each test checks the oracle against something it does not compute itself:
exact rational bounds, dense softmax attention under an explicit token mask,
the A-shape masks written out, and the one-token step it reduces to.
"""
import math

import numpy as np
import pytest

import oracle
from brute import (ashape_mask, bf16_bits_to_f64, dense_attention, f32_to_bf16_bits, page_bound,
                   page_token_mask, rank_select, summary)
from paged_case import make_case


def _layout(c):
    return oracle.Layout(**c.layout_args())


def _drafts(c, nq, seed):
    """Queries for nq draft tokens: [B][nq][Hq][Dk] bf16 bits."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((c.batch, nq, c.num_q_heads, c.head_dim_k)).astype(np.float32))


def _pages(c, b, g):
    L, ps = int(c.seq_lens[b]), c.page_size
    return [[list(c.K[b][t, g]) for t in range(j * ps, min((j + 1) * ps, L))]
            for j in range((L + ps - 1) // ps)]


def test_one_draft_is_the_one_token_step():
    c = make_case(41, B=3, Hq=6, Hkv=2, Dk=16, Dv=8, ps=4, lens=[45, 13, 30])
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=3, sink_tokens=2, window_tokens=7,
                        static_heads=[0, 1])
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 6, c.k_pool)
    q1 = c.q_bits[:, None]
    sc = oracle.scores(lay, c.page_table, c.seq_lens, c.q_bits, summ, pol)
    scm = oracle.scores_multi(lay, c.page_table, c.seq_lens, q1, summ, pol)
    assert np.array_equal(sc, scm)
    sel, cnt = oracle.select(lay, c.page_table, c.seq_lens, 6, sc, pol)
    selm, cntm = oracle.select_multi(lay, c.page_table, c.seq_lens, 6, 1, scm, pol)
    assert np.array_equal(sel, selm) and np.array_equal(cnt, cntm)
    out = oracle.attend(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool, c.v_pool, sel, cnt, pol, 0.4)
    outm = oracle.attend_multi(lay, c.page_table, c.seq_lens, q1, c.k_pool, c.v_pool, sel, cnt, pol, 0.4)
    assert np.array_equal(out, outm[:, 0])


@pytest.mark.parametrize("nq", [2, 3])
def test_scores_are_the_max_over_draft_queries(nq):
    c = make_case(42, B=2, Hq=4, Hkv=2, Dk=8, Dv=8, ps=4, lens=[27, 19])
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=2)
    q = _drafts(c, nq, 5)
    qf = bf16_bits_to_f64(q)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 4, c.k_pool)
    sc = oracle.scores_multi(lay, c.page_table, c.seq_lens, q, summ, pol)
    G = 2
    for b in range(2):
        for g in range(2):
            pages = _pages(c, b, g)
            P = len(pages)
            for j, toks in enumerate(pages):
                if not 1 <= j < P - 1:
                    assert sc[b, g, j] == -math.inf
                    continue
                lo, hi = summary(toks)
                want = max(page_bound(qf[b, i, h], lo, hi) for i in range(nq) for h in range(g * G, (g + 1) * G))
                assert sc[b, g, j] == want
            # the selection is the rank-counting top-k of those scores
            keys = {j: sc[b, g, j] for j in range(1, P - 1)}
            want_sel = sorted(set([0, P - 1]) | set(rank_select(keys, 2)))
            sel, cnt = oracle.select_multi(lay, c.page_table, c.seq_lens, 4, nq, sc, pol)
            assert list(sel[b, g, :cnt[b, g]]) == want_sel


@pytest.mark.parametrize("v_from_k", [False, True])
def test_all_pages_selected_is_causal_dense_attention(v_from_k):
    nq = 3
    c = make_case(43, B=2, Hq=4, Hkv=2, Dk=16, Dv=8, ps=4, lens=[33, 10], v_from_k=v_from_k)
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=1000)
    q = _drafts(c, nq, 6)
    qf = bf16_bits_to_f64(q)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 4, c.k_pool)
    sc = oracle.scores_multi(lay, c.page_table, c.seq_lens, q, summ, pol)
    sel, cnt = oracle.select_multi(lay, c.page_table, c.seq_lens, 4, nq, sc, pol)
    out = oracle.attend_multi(lay, c.page_table, c.seq_lens, q, c.k_pool, c.v_pool, sel, cnt, pol, 0.3)
    for b in range(2):
        L = int(c.seq_lens[b])
        for i in range(nq):
            causal = np.arange(L) <= L - nq + i
            for h in range(4):
                g = h // 2
                want = dense_attention(qf[b, i, h], c.K[b][:, g], c.V[b][:, g], causal, 0.3)
                np.testing.assert_allclose(out[b, i, h], want, rtol=0, atol=1e-12)
    # the last draft query sees the whole sequence; the first does not see the later drafts
    assert not np.allclose(out[:, 0], out[:, nq - 1])


def test_selected_pages_attention_is_causal_and_shared():
    nq = 4
    c = make_case(44, B=2, Hq=8, Hkv=2, Dk=8, Dv=6, ps=4, lens=[61, 26])
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=3)
    q = _drafts(c, nq, 7)
    qf = bf16_bits_to_f64(q)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 8, c.k_pool)
    sc = oracle.scores_multi(lay, c.page_table, c.seq_lens, q, summ, pol)
    sel, cnt = oracle.select_multi(lay, c.page_table, c.seq_lens, 8, nq, sc, pol)
    out = oracle.attend_multi(lay, c.page_table, c.seq_lens, q, c.k_pool, c.v_pool, sel, cnt, pol, 0.5)
    for b in range(2):
        L = int(c.seq_lens[b])
        for h in range(8):
            g = h // 4
            m = page_token_mask(L, 4, sel[b, g, :cnt[b, g]])
            for i in range(nq):
                want = dense_attention(qf[b, i, h], c.K[b][:, g], c.V[b][:, g], m & (np.arange(L) <= L - nq + i), 0.5)
                np.testing.assert_allclose(out[b, i, h], want, rtol=0, atol=1e-12)


def test_static_heads_read_the_union_of_the_queries_windows():
    nq = 3
    c = make_case(45, B=3, Hq=4, Hkv=2, Dk=8, Dv=8, ps=4, lens=[70, 9, 33])
    lay = _layout(c)
    q = _drafts(c, nq, 8)
    qf = bf16_bits_to_f64(q)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 4, c.k_pool)
    for sink, win in [(3, 10), (0, 5), (6, 0), (2, 1000), (1, 3)]:
        pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=2, sink_tokens=sink, window_tokens=win,
                            static_heads=[1, 0])
        sc = oracle.scores_multi(lay, c.page_table, c.seq_lens, q, summ, pol)
        assert np.all(sc[:, 0] == -math.inf)
        sel, cnt = oracle.select_multi(lay, c.page_table, c.seq_lens, 4, nq, sc, pol)
        out = oracle.attend_multi(lay, c.page_table, c.seq_lens, q, c.k_pool, c.v_pool, sel, cnt, pol, 0.25)
        for b in range(3):
            L = int(c.seq_lens[b])
            masks = []
            for i in range(nq):
                Li = L - nq + 1 + i
                m = np.zeros(L, bool)
                m[:Li] = ashape_mask(Li, sink, win)
                masks.append(m)
            union = np.logical_or.reduce(masks)
            pages = sorted({t // 4 for t in np.nonzero(union)[0]})
            assert list(sel[b, 0, :cnt[b, 0]]) == pages
            for i in range(nq):
                for h in range(2):
                    want = dense_attention(qf[b, i, h], c.K[b][:, 0], c.V[b][:, 0], masks[i], 0.25)
                    np.testing.assert_allclose(out[b, i, h], want, rtol=0, atol=1e-12)


def test_sequences_shorter_than_the_drafts():
    nq = 4
    c = make_case(46, B=3, Hq=2, Hkv=1, Dk=8, Dv=8, ps=4, lens=[2, 0, 4])
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=2)
    q = _drafts(c, nq, 9)
    qf = bf16_bits_to_f64(q)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 2, c.k_pool)
    sc = oracle.scores_multi(lay, c.page_table, c.seq_lens, q, summ, pol)
    sel, cnt = oracle.select_multi(lay, c.page_table, c.seq_lens, 2, nq, sc, pol)
    out = oracle.attend_multi(lay, c.page_table, c.seq_lens, q, c.k_pool, c.v_pool, sel, cnt, pol, 1.0)
    # length 2: queries 0 and 1 have no position (output 0), query 2 sees token 0, query 3 tokens 0..1
    assert np.all(out[0, :2] == 0.0)
    for h in range(2):
        assert np.array_equal(out[0, 2, h], c.V[0][0, 0])
        want = dense_attention(qf[0, 3, h], c.K[0][:, 0], c.V[0][:, 0], np.ones(2, bool), 1.0)
        np.testing.assert_allclose(out[0, 3, h], want, rtol=0, atol=1e-12)
    assert np.all(out[1] == 0.0) and cnt[1, 0] == 0
    # length 4 = nq: query 0 sees only token 0
    for h in range(2):
        assert np.array_equal(out[2, 0, h], c.V[2][0, 0])


def test_max_sel_multi_covers_the_widened_window():
    lay = oracle.Layout(num_pool_pages=64, page_size=16, num_kv_heads=2, head_dim_k=8, head_dim_v=8)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=0, sink_tokens=4, window_tokens=32,
                        static_heads=[1, 1])
    # a window of 32 tokens spans at most 3 pages of 16; 32 + 3 tokens span up to 4
    assert oracle.max_sel(lay, pol, 64) == 1 + 2 + 1
    assert oracle.max_sel_multi(lay, pol, 4, 64) == 1 + 3 + 1
