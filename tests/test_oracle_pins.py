"""Pins of the CPU oracle against things other than itself: exact rational
arithmetic, a library routine (math.fsum), closed forms, hand-worked
selections, invariants of the bound, and dense attention computed from the
logical token arrays.

The set is chosen so that a plausible slip anywhere in the oracle (a dropped
term, a swapped min/max, a wrong sign, an off-by-one page range, the tie going
to the wrong page, a transposed value layout, a leaked token past the end of a
sequence) fails at least one test; test_oracle_mutants.py checks exactly that.
"""
import math
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
from brute import (ashape_mask, bf16_bits_to_f64, dense_attention, exact_dot,
                   f32_to_bf16_bits, page_bound, page_token_mask, rank_select, summary)
from paged_case import make_case


def _layout(c):
    return oracle.Layout(**c.layout_args())


def _logical_pages(c, b, g):
    """Per logical page: the list of valid token keys of KV head g."""
    L, ps = int(c.seq_lens[b]), c.page_size
    return [[list(c.K[b][t, g]) for t in range(j * ps, min((j + 1) * ps, L))]
            for j in range((L + ps - 1) // ps)]


# ----------------------------------------------------------------------------
# exact summation
# ----------------------------------------------------------------------------

def test_exact_sum_closed_forms():
    # half-way cases round to even; anything beyond half-way rounds up
    assert oracle.exact_sum([1.0, 2.0 ** -53]) == 1.0
    assert oracle.exact_sum([1.0, 2.0 ** -53, 2.0 ** -200]) == 1.0 + 2.0 ** -52
    assert oracle.exact_sum([1.0 + 2.0 ** -52, 2.0 ** -53]) == 1.0 + 2.0 ** -51
    assert oracle.exact_sum([-1.0, -(2.0 ** -53)]) == -1.0
    # cancellation
    assert oracle.exact_sum([1e16, 1.0, -1e16]) == 1.0
    assert oracle.exact_sum([2.0 ** 900, -(2.0 ** 900), 3.0]) == 3.0
    assert oracle.exact_sum([]) == 0.0
    assert oracle.exact_sum([0.1] * 10) == math.fsum([0.1] * 10)


def test_exact_sum_matches_rationals_and_fsum():
    rnd = random.Random(11)
    for _ in range(1500):
        n = rnd.randint(1, 64)
        xs = [rnd.choice((-1, 1)) * rnd.random() * 2.0 ** rnd.randint(-300, 300) for _ in range(n)]
        if rnd.random() < 0.4:
            xs += [-x * (1 + 2.0 ** -40) for x in xs[: n // 2]]
        rnd.shuffle(xs)
        want = float(sum((Fraction(x) for x in xs), Fraction(0)))
        got = oracle.exact_sum(xs)
        assert got == want
        assert got == math.fsum(xs)


def test_exact_sum_of_bf16_products_order_free():
    rng = np.random.default_rng(5)
    a = bf16_bits_to_f64(f32_to_bf16_bits(rng.standard_normal(4096).astype(np.float32)))
    b = bf16_bits_to_f64(f32_to_bf16_bits(rng.standard_normal(4096).astype(np.float32)))
    p = a * b
    assert np.array_equal(p, np.asarray([float(Fraction(x) * Fraction(y)) for x, y in zip(a, b)]))
    ref = oracle.exact_sum(p)
    for s in range(5):
        assert oracle.exact_sum(np.random.default_rng(s).permutation(p)) == ref
    assert ref == float(sum((Fraction(x) for x in p), Fraction(0)))


# ----------------------------------------------------------------------------
# summaries and scores
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_summaries_and_scores_match_exact_rationals(seed):
    c = make_case(seed, B=2, Hq=4, Hkv=2, Dk=8, Dv=8, ps=4, lens=[23, 18])
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=2)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, c.num_q_heads, c.k_pool)
    sc = oracle.scores(lay, c.page_table, c.seq_lens, c.q_bits, summ, pol)
    G = c.num_q_heads // c.num_kv_heads
    for b in range(c.batch):
        for g in range(c.num_kv_heads):
            pages = _logical_pages(c, b, g)
            P = len(pages)
            for j, toks in enumerate(pages):
                lo, hi = summary(toks)
                phys = c.page_table[b, j]
                assert list(bf16_bits_to_f64(summ[phys, g, 0])) == lo
                assert list(bf16_bits_to_f64(summ[phys, g, 1])) == hi
                cand = 1 <= j < P - 1
                if not cand:
                    assert sc[b, g, j] == -math.inf
                    continue
                want = max(page_bound(c.q[b, h], lo, hi) for h in range(g * G, (g + 1) * G))
                assert sc[b, g, j] == want
            assert np.all(sc[b, g, P:] == -math.inf)


def test_summary_orders_signed_zero():
    c = make_case(3, B=1, Hq=1, Hkv=1, Dk=2, Dv=2, ps=2, lens=[2], values="zero", garbage=False)
    phys = c.page_table[0, 0]
    c.k_pool[phys, 0, 0] = [0x8000, 0x0000]   # (-0, +0)
    c.k_pool[phys, 0, 1] = [0x0000, 0x8000]   # (+0, -0)
    summ = oracle.summaries(_layout(c), c.page_table, c.seq_lens, 1, c.k_pool)
    assert list(summ[phys, 0, 0]) == [0x8000, 0x8000]
    assert list(summ[phys, 0, 1]) == [0x0000, 0x0000]


def test_bound_dominates_every_key_and_split_form_identity():
    c = make_case(4, B=1, Hq=8, Hkv=2, Dk=16, Dv=4, ps=8, lens=[77], key_scale=3.0)
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=0, n_local_pages=0, top_k=3)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, c.num_q_heads, c.k_pool)
    sc = oracle.scores(lay, c.page_table, c.seq_lens, c.q_bits, summ, pol)
    G = 4
    for g in range(2):
        for j, toks in enumerate(_logical_pages(c, 0, g)):
            phys = c.page_table[0, j]
            lo = bf16_bits_to_f64(summ[phys, g, 0])
            hi = bf16_bits_to_f64(summ[phys, g, 1])
            split = []
            for h in range(g * G, (g + 1) * G):
                qh = c.q[0, h]
                for k in toks:  # bound >= every true q.k in the page (exactly)
                    assert Fraction(sc[0, g, j]) >= exact_dot(qh, k) or sc[0, g, j] == float(exact_dot(qh, k))
                qp, qn = np.maximum(qh, 0.0), np.minimum(qh, 0.0)
                split.append(math.fsum(list(qp * hi) + list(qn * lo)))
            assert sc[0, g, j] == max(split)


def test_constant_page_bound_is_tight():
    c = make_case(5, B=1, Hq=3, Hkv=1, Dk=8, Dv=4, ps=4, lens=[16])
    for j in range(4):
        phys = c.page_table[0, j]
        c.k_pool[phys, 0, :, :] = c.k_pool[phys, 0, 0, :][None, :]
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=0, n_local_pages=0, top_k=1)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 3, c.k_pool)
    sc = oracle.scores(lay, c.page_table, c.seq_lens, c.q_bits, summ, pol)
    for j in range(4):
        k = bf16_bits_to_f64(c.k_pool[c.page_table[0, j], 0, 0])
        assert sc[0, 0, j] == max(float(exact_dot(c.q[0, h], k)) for h in range(3))


# ----------------------------------------------------------------------------
# selection
# ----------------------------------------------------------------------------

def _worked_case(p4_second_key):
    """G=1, d=2, page 2, q=(1,-2), 7 pages of 2 tokens each."""
    pages = [[(0, 0), (1, 1)], [(2, 1), (-1, 3)], [(3, -1), (0, 0)], [(1, -1), (1, -1)],
             [(-1, -1), p4_second_key], [(0, 1), (0, 1)], [(0, 0), (0, 0)]]
    c = make_case(0, B=1, Hq=1, Hkv=1, Dk=2, Dv=2, ps=2, lens=[14], values="zero", garbage=False)
    for j, toks in enumerate(pages):
        for t, k in enumerate(toks):
            c.k_pool[c.page_table[0, j], 0, t] = f32_to_bf16_bits(np.asarray(k, np.float32))
    c.q_bits[0, 0] = f32_to_bf16_bits(np.asarray([1, -2], np.float32))
    return c


def test_hand_worked_selection():
    # bounds: p0 1, p1 0, p2 5, p3 3, p4 4, p5 -2; p0 sink, p6 local
    c = _worked_case((2, 0))
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=2)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 1, c.k_pool)
    sc = oracle.scores(lay, c.page_table, c.seq_lens, c.q_bits, summ, pol)
    assert list(sc[0, 0, :7]) == [-math.inf, 0, 5, 3, 4, -2, -math.inf]
    sel, cnt = oracle.select(lay, c.page_table, c.seq_lens, 1, sc, pol)
    assert cnt[0, 0] == 4 and list(sel[0, 0, :4]) == [0, 2, 4, 6]
    # p4's second key (3,0) lifts its bound to 5: tie with p2, lowest id wins
    c = _worked_case((3, 0))
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=1)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 1, c.k_pool)
    sc = oracle.scores(lay, c.page_table, c.seq_lens, c.q_bits, summ, pol)
    assert sc[0, 0, 2] == sc[0, 0, 4] == 5
    sel, cnt = oracle.select(lay, c.page_table, c.seq_lens, 1, sc, pol)
    assert cnt[0, 0] == 3 and list(sel[0, 0, :3]) == [0, 2, 6]


@pytest.mark.parametrize("seed,values", [(0, "int"), (1, "int"), (2, "normal"), (3, "int")])
def test_selection_matches_rank_counting(seed, values):
    c = make_case(seed, B=3, Hq=4, Hkv=2, Dk=4, Dv=4, ps=3, lens=[40, 7, 29], values=values)
    lay = _layout(c)
    for ns, nl, k in [(1, 2, 3), (0, 0, 5), (2, 1, 0), (1, 1, 100), (3, 3, 1)]:
        pol = oracle.Policy(n_sink_pages=ns, n_local_pages=nl, top_k=k)
        summ = oracle.summaries(lay, c.page_table, c.seq_lens, 4, c.k_pool)
        sc = oracle.scores(lay, c.page_table, c.seq_lens, c.q_bits, summ, pol)
        sel, cnt = oracle.select(lay, c.page_table, c.seq_lens, 4, sc, pol, max_sel_n=40)
        for b in range(3):
            P = (int(c.seq_lens[b]) + 2) // 3
            for g in range(2):
                fixed = set(range(min(ns, P))) | set(range(max(0, P - nl), P))
                keys = {j: sc[b, g, j] for j in range(P) if j not in fixed}
                want = sorted(fixed | set(rank_select(keys, k)))
                assert list(sel[b, g, :cnt[b, g]]) == want
                assert np.all(sel[b, g, cnt[b, g]:] == -1)


def test_zero_query_selects_lowest_ids_and_averages_values():
    c = make_case(6, B=1, Hq=2, Hkv=1, Dk=8, Dv=8, ps=4, lens=[50], q_values="zero")
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=2, top_k=3)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 2, c.k_pool)
    out, sel, cnt = oracle.decode(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool, c.v_pool,
                                  summ, pol, 0.125)
    # 13 pages: sink 0, local 11 12, lowest candidates 1 2 3
    assert list(sel[0, 0, :cnt[0, 0]]) == [0, 1, 2, 3, 11, 12]
    toks = page_token_mask(50, 4, [0, 1, 2, 3, 11, 12])
    mean = c.V[0][toks, 0].mean(0)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], mean, rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("v_from_k", [False, True])
def test_all_pages_selected_equals_dense_attention(v_from_k):
    c = make_case(7, B=2, Hq=6, Hkv=3, Dk=16, Dv=8, ps=4, lens=[37, 12], v_from_k=v_from_k)
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=1000)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 6, c.k_pool)
    out, sel, cnt = oracle.decode(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool, c.v_pool,
                                  summ, pol, 0.3)
    for b in range(2):
        L = int(c.seq_lens[b])
        for h in range(6):
            g = h // 2
            want = dense_attention(c.q[b, h], c.K[b][:, g], c.V[b][:, g], np.ones(L, bool), 0.3)
            np.testing.assert_allclose(out[b, h], want, rtol=0, atol=1e-12)


def test_selected_pages_attention_matches_masked_dense():
    c = make_case(8, B=2, Hq=4, Hkv=2, Dk=8, Dv=6, ps=4, lens=[61, 30])
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=3)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 4, c.k_pool)
    out, sel, cnt = oracle.decode(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool, c.v_pool,
                                  summ, pol, 0.5)
    for b in range(2):
        L = int(c.seq_lens[b])
        for h in range(4):
            g = h // 2
            m = page_token_mask(L, 4, sel[b, g, :cnt[b, g]])
            want = dense_attention(c.q[b, h], c.K[b][:, g], c.V[b][:, g], m, 0.5)
            np.testing.assert_allclose(out[b, h], want, rtol=0, atol=1e-12)


def test_static_ashape_heads():
    c = make_case(9, B=3, Hq=4, Hkv=2, Dk=8, Dv=8, ps=4, lens=[70, 9, 33])
    lay = _layout(c)
    for sink, win in [(3, 10), (0, 5), (6, 0), (2, 1000)]:
        pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=2, sink_tokens=sink,
                            window_tokens=win, static_heads=[1, 0])
        summ = oracle.summaries(lay, c.page_table, c.seq_lens, 4, c.k_pool)
        sc = oracle.scores(lay, c.page_table, c.seq_lens, c.q_bits, summ, pol)
        assert np.all(sc[:, 0] == -math.inf)
        out, sel, cnt = oracle.decode(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool,
                                      c.v_pool, summ, pol, 0.25)
        for b in range(3):
            L = int(c.seq_lens[b])
            m = ashape_mask(L, sink, win)
            pages = sorted({t // 4 for t in np.nonzero(m)[0]})
            assert list(sel[b, 0, :cnt[b, 0]]) == pages
            for h in range(2):
                want = dense_attention(c.q[b, h], c.K[b][:, 0], c.V[b][:, 0], m, 0.25)
                np.testing.assert_allclose(out[b, h], want, rtol=0, atol=1e-12)


def test_single_token_returns_its_value():
    c = make_case(10, B=2, Hq=2, Hkv=1, Dk=8, Dv=8, ps=4, lens=[1, 1])
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=0, n_local_pages=0, top_k=1)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 2, c.k_pool)
    out, sel, cnt = oracle.decode(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool, c.v_pool,
                                  summ, pol, 1.0)
    for b in range(2):
        for h in range(2):
            assert np.array_equal(out[b, h], c.V[b][0, 0])


def test_empty_sequences_and_empty_batch():
    c = make_case(11, B=2, Hq=2, Hkv=1, Dk=4, Dv=4, ps=4, lens=[0, 5])
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=1)
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 2, c.k_pool)
    out, sel, cnt = oracle.decode(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool, c.v_pool,
                                  summ, pol, 1.0)
    assert cnt[0, 0] == 0 and np.all(out[0] == 0)
    assert cnt[1, 0] == 2
    e = oracle.decode(lay, c.page_table[:0], c.seq_lens[:0], c.q_bits[:0], c.k_pool, c.v_pool,
                      summ, pol, 1.0)
    assert e[0].shape[0] == 0


def test_physical_placement_does_not_matter():
    a = make_case(12, B=2, Hq=4, Hkv=2, Dk=8, Dv=8, ps=4, lens=[45, 26], perm_seed=1)
    b = make_case(12, B=2, Hq=4, Hkv=2, Dk=8, Dv=8, ps=4, lens=[45, 26], perm_seed=2)
    assert not np.array_equal(a.page_table, b.page_table)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=3)
    res = []
    for c in (a, b):
        lay = _layout(c)
        summ = oracle.summaries(lay, c.page_table, c.seq_lens, 4, c.k_pool)
        res.append(oracle.decode(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool, c.v_pool,
                                 summ, pol, 0.35))
    for x, y in zip(res[0], res[1]):
        assert np.array_equal(x, y)


def test_tokens_past_the_end_are_ignored():
    a = make_case(13, B=1, Hq=2, Hkv=1, Dk=8, Dv=8, ps=8, lens=[29])
    lay = _layout(a)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=1)
    outs = []
    for fill in (0x4780, 0xC780):   # +65536, -65536 in the 3 slots past L
        phys = a.page_table[0, 3]
        a.k_pool[phys, 0, 5:] = fill
        a.v_pool[phys, 0, :, 5:] = fill
        summ = oracle.summaries(lay, a.page_table, a.seq_lens, 2, a.k_pool)
        outs.append(oracle.decode(lay, a.page_table, a.seq_lens, a.q_bits, a.k_pool, a.v_pool,
                                  summ, pol, 0.4)[0])
    assert np.array_equal(outs[0], outs[1])


def test_append_then_summaries_match_recomputation():
    c = make_case(14, B=3, Hq=2, Hkv=2, Dk=8, Dv=4, ps=4, lens=[8, 13, 3])
    lay = _layout(c)
    rng = np.random.default_rng(0)
    kn = f32_to_bf16_bits(rng.standard_normal((3, 2, 8)).astype(np.float32))
    vn = f32_to_bf16_bits(rng.standard_normal((3, 2, 4)).astype(np.float32))
    k2, v2 = oracle.append(lay, c.page_table, c.seq_lens, 2, kn, vn, c.k_pool, c.v_pool)
    new_lens = c.seq_lens + 1
    for b in range(3):
        L = int(c.seq_lens[b])
        phys, t = c.page_table[b, L // 4], L % 4
        assert np.array_equal(k2[phys, :, t, :], kn[b])
        assert np.array_equal(v2[phys, :, :, t], vn[b])
    summ = oracle.summaries(lay, c.page_table, new_lens, 2, k2)
    for b in range(3):
        L = int(new_lens[b])
        j = (L - 1) // 4
        for g in range(2):
            toks = [list(c.K[b][t, g]) for t in range(j * 4, L - 1)] + [list(bf16_bits_to_f64(kn[b, g]))]
            lo, hi = summary(toks)
            phys = c.page_table[b, j]
            assert list(bf16_bits_to_f64(summ[phys, g, 0])) == lo
            assert list(bf16_bits_to_f64(summ[phys, g, 1])) == hi


def test_max_sel_bounds():
    lay = oracle.Layout(64, 16, 8, 128, 128)
    assert oracle.max_sel(lay, oracle.Policy(1, 8, 119), 2049) == 128
    assert oracle.max_sel(lay, oracle.Policy(1, 8, 55, 4, 1024, [1] * 4 + [0] * 4), 4097) == 66
    assert oracle.max_sel(lay, oracle.Policy(1, 8, 119), 50) == 50
