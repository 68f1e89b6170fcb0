"""Pins of the oracle's 2-bit quantised pages (KIVI-style: 2 bits, groups of
32, a full-precision residual region; SCBench notes' method table and the
SparseEngine article's decode-hook paragraph).

Readings (stated beside orc_quantize in the oracle's header): a group is 32
consecutive channels of one token; zero point = the group minimum and step =
(max - min) / 3, both stored as binary16; code = round-half-even((x - m) / s)
clamped to 0..3 in binary32; read back as m + code * s; the last
residual_pages logical pages stay bf16.

Checks against things the oracle does not compute itself: numpy's binary16
rounding, the round-to-nearest error bound, data placed exactly on the grid
(codes and values recovered exactly), and dense attention over values read
back by numpy."""
import numpy as np
import pytest

import oracle
from brute import bf16_bits_to_f64, dense_attention, f32_to_bf16_bits, page_token_mask
from paged_case import make_case


def _layout(c):
    return oracle.Layout(**c.layout_args())


def test_half_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-9, 5, 2000),
                         [0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e-8, 2.0 ** -24, 2.0 ** -25,
                          3 * 2.0 ** -26, 2.0 ** -14, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2047.5, 2048.5]])
    for x in xs:
        x = float(np.float32(x))  # the oracle converts binary32 values
        with np.errstate(over="ignore"):
            want = int(np.array(x, np.float64).astype(np.float16).view(np.uint16))
        assert oracle.half_bits(x) == want, x


def _fill_on_grid(c, rng):
    """Rewrites every token's keys and values so that each group of 32 holds
    m + code * s with exactly representable m, s (codes 0 and 3 present), and
    returns the codes [per sequence][L][Hkv][D] for keys and values."""
    kcodes, vcodes = [], []
    for b in range(c.batch):
        L = int(c.seq_lens[b])
        ks = np.zeros((L, c.num_kv_heads, c.head_dim_k))
        vs = np.zeros((L, c.num_kv_heads, c.head_dim_v))
        kc = rng.integers(0, 4, (L, c.num_kv_heads, c.head_dim_k))
        vc = rng.integers(0, 4, (L, c.num_kv_heads, c.head_dim_v))
        for arr, codes in ((ks, kc), (vs, vc)):
            codes[..., 0::32] = 0
            codes[..., 1::32] = 3
            m = rng.integers(-16, 16, arr.shape[:-1] + (arr.shape[-1] // 32,)) / 8.0
            s = rng.integers(1, 9, m.shape) / 8.0
            arr[:] = np.repeat(m, 32, -1) + codes * np.repeat(s, 32, -1)
        kcodes.append(kc)
        vcodes.append(vc)
        kb, vb = f32_to_bf16_bits(ks.astype(np.float32)), f32_to_bf16_bits(vs.astype(np.float32))
        assert np.array_equal(bf16_bits_to_f64(kb), ks) and np.array_equal(bf16_bits_to_f64(vb), vs)
        for t in range(L):
            phys = c.page_table[b, t // c.page_size]
            c.k_pool[phys, :, t % c.page_size, :] = kb[t]
            c.v_pool[phys, :, :, t % c.page_size] = vb[t]
        c.K[b], c.V[b] = ks, vs
    return kcodes, vcodes


def _read_back(codes, meta):
    m = meta[..., 0].view(np.float16).astype(np.float64)
    s = meta[..., 1].view(np.float16).astype(np.float64)
    return np.repeat(m, 32, -1) + codes.astype(np.float64) * np.repeat(s, 32, -1)


def test_codes_on_grid_are_recovered_exactly():
    rng = np.random.default_rng(1)
    c = make_case(51, B=3, Hq=4, Hkv=2, Dk=64, Dv=32, ps=4, lens=[37, 9, 24])
    kcodes, vcodes = _fill_on_grid(c, rng)
    lay = _layout(c)
    for R in (1, 3):
        qz = oracle.quantize(lay, c.page_table, c.seq_lens, 4, R, c.k_pool, c.v_pool)
        for b in range(c.batch):
            L = int(c.seq_lens[b])
            P = (L + 3) // 4
            for j in range(P):
                phys = c.page_table[b, j]
                if j >= P - R:   # residual pages are not written
                    assert not qz.k_codes[phys].any() and not qz.k_meta[phys].any()
                    continue
                toks = slice(4 * j, 4 * j + 4)
                assert np.array_equal(qz.k_codes[phys].transpose(1, 0, 2), kcodes[b][toks])
                assert np.array_equal(qz.v_codes[phys].transpose(1, 0, 2), vcodes[b][toks])
                assert np.array_equal(_read_back(qz.k_codes[phys], qz.k_meta[phys]).transpose(1, 0, 2),
                                      c.K[b][toks])
                assert np.array_equal(_read_back(qz.v_codes[phys], qz.v_meta[phys]).transpose(1, 0, 2),
                                      c.V[b][toks])


@pytest.mark.parametrize("scale", [1.0, 1e-3, 300.0])
def test_quantisation_error_and_order_properties(scale):
    c = make_case(52, B=2, Hq=2, Hkv=2, Dk=64, Dv=64, ps=4, lens=[33, 21], key_scale=scale)
    lay = _layout(c)
    qz = oracle.quantize(lay, c.page_table, c.seq_lens, 2, 1, c.k_pool, c.v_pool)
    for b in range(c.batch):
        L = int(c.seq_lens[b])
        P = (L + 3) // 4
        for j in range(P - 1):
            phys = c.page_table[b, j]
            for codes, meta, X in ((qz.k_codes, qz.k_meta, c.K[b]), (qz.v_codes, qz.v_meta, c.V[b])):
                x = X[4 * j:4 * j + 4].transpose(1, 0, 2).reshape(-1, 32)     # groups of 32
                cd = codes[phys].reshape(-1, 32)
                m = meta[phys][..., 0].reshape(-1).view(np.float16).astype(np.float64)
                s = meta[phys][..., 1].reshape(-1).view(np.float16).astype(np.float64)
                xh = m[:, None] + cd * s[:, None]
                assert cd.max() <= 3
                # zero point: the group minimum as binary16; the minimum gets code 0
                assert np.array_equal(m, x.min(1).astype(np.float16).astype(np.float64))
                assert np.all(cd[np.arange(len(x)), x.argmin(1)] == 0)
                # the step spans the range: within 1% of (max - min) / 3
                np.testing.assert_allclose(3 * s, x.max(1) - x.min(1), rtol=1e-2)
                # read-back error of a nearest code: half a step (+ the binary16 roundings)
                err = np.abs(xh - x)
                assert np.all(err <= 0.5 * s[:, None] * 1.01 + np.abs(m - x.min(1))[:, None] + 1e-30)
                # codes follow the order of the values
                o = np.argsort(x, 1, kind="stable")
                assert np.all(np.diff(np.take_along_axis(cd, o, 1).astype(int), axis=1) >= 0)


def test_constant_group_has_zero_step():
    c = make_case(53, B=1, Hq=2, Hkv=1, Dk=32, Dv=32, ps=4, lens=[12], values="zero")
    c.k_pool[:] = f32_to_bf16_bits(np.float32(0.375))
    c.v_pool[:] = f32_to_bf16_bits(np.float32(-2.5))
    lay = _layout(c)
    qz = oracle.quantize(lay, c.page_table, c.seq_lens, 2, 1, c.k_pool, c.v_pool)
    for j in range(2):
        phys = c.page_table[0, j]
        assert not qz.k_codes[phys].any() and not qz.v_codes[phys].any()
        assert np.all(qz.k_meta[phys][..., 1] == 0) and np.all(qz.v_meta[phys][..., 1] == 0)
        assert np.all(qz.k_meta[phys][..., 0].view(np.float16) == 0.375)
        assert np.all(qz.v_meta[phys][..., 0].view(np.float16) == -2.5)


def test_quantised_attention_is_dense_attention_over_read_back_values():
    c = make_case(54, B=3, Hq=4, Hkv=2, Dk=64, Dv=32, ps=4, lens=[45, 14, 30])
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=2, top_k=3)
    R = 2
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 4, c.k_pool)
    sc = oracle.scores(lay, c.page_table, c.seq_lens, c.q_bits, summ, pol)
    sel, cnt = oracle.select(lay, c.page_table, c.seq_lens, 4, sc, pol)
    qz = oracle.quantize(lay, c.page_table, c.seq_lens, 4, R, c.k_pool, c.v_pool)
    out = oracle.attend_quant(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool, c.v_pool, qz, sel, cnt, pol, 0.3)
    for b in range(3):
        L = int(c.seq_lens[b])
        P = (L + 3) // 4
        Kh, Vh = c.K[b].copy(), c.V[b].copy()
        for j in range(P - R):
            phys = c.page_table[b, j]
            Kh[4 * j:4 * j + 4] = _read_back(qz.k_codes[phys], qz.k_meta[phys]).transpose(1, 0, 2)
            Vh[4 * j:4 * j + 4] = _read_back(qz.v_codes[phys], qz.v_meta[phys]).transpose(1, 0, 2)
        for h in range(4):
            g = h // 2
            m = page_token_mask(L, 4, sel[b, g, :cnt[b, g]])
            want = dense_attention(c.q[b, h], Kh[:, g], Vh[:, g], m, 0.3)
            np.testing.assert_allclose(out[b, h], want, rtol=0, atol=1e-12)
    # every page in the residual region: the plain attention exactly
    big = oracle.quantize(lay, c.page_table, c.seq_lens, 4, 100, c.k_pool, c.v_pool)
    out_all = oracle.attend_quant(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool, c.v_pool, big, sel, cnt, pol,
                                  0.3)
    plain = oracle.attend(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool, c.v_pool, sel, cnt, pol, 0.3)
    assert np.array_equal(out_all, plain)


def test_on_grid_data_attends_as_unquantised():
    rng = np.random.default_rng(2)
    c = make_case(55, B=2, Hq=4, Hkv=2, Dk=64, Dv=64, ps=4, lens=[29, 18])
    _fill_on_grid(c, rng)
    lay = _layout(c)
    pol = oracle.Policy(n_sink_pages=1, n_local_pages=1, top_k=2, sink_tokens=3, window_tokens=6,
                        static_heads=[0, 1])
    summ = oracle.summaries(lay, c.page_table, c.seq_lens, 4, c.k_pool)
    sc = oracle.scores(lay, c.page_table, c.seq_lens, c.q_bits, summ, pol)
    sel, cnt = oracle.select(lay, c.page_table, c.seq_lens, 4, sc, pol)
    qz = oracle.quantize(lay, c.page_table, c.seq_lens, 4, 1, c.k_pool, c.v_pool)
    out = oracle.attend_quant(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool, c.v_pool, qz, sel, cnt, pol, 0.7)
    plain = oracle.attend(lay, c.page_table, c.seq_lens, c.q_bits, c.k_pool, c.v_pool, sel, cnt, pol, 0.7)
    assert np.array_equal(out, plain)
