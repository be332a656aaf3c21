"""Pins of the fp64 oracle against facts it does not compute itself.

Each test ties the oracle to something outside it: a value the pages state
(tests/golden/page_cases.json), a closed form, an invariant of softmax
attention, or a library routine (torch's scaled_dot_product_attention in
float64 on the CPU). Together they are chosen so that a plausible slip in
oracle.c (a dropped scale, a wrong sign, h % Hkv instead of h / hpk, j < i
instead of j <= i, a window off by one, a transposed stride) fails at least
one of them; test_oracle_mutants.py plants such slips and checks that.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth

RTOL = 1e-12  # fp64 closed forms and library cross-checks


def _rng(seed):
    return np.random.default_rng(seed)


def _prefill_case(seed, m, hq, hpk, d, q_pad=0, kv_pad=0, sigma=1.0):
    w = synth.PrefillWorkload("t", m=m, num_q_heads=hq, heads_per_kv=hpk,
                              head_dim=d, q_stride=hq * d + q_pad,
                              kv_stride=(hq // hpk) * d + kv_pad, sigma=sigma,
                              seed=seed)
    return w, synth.prefill_inputs(w)


def _run_prefill(orc, w, q, k, v, **kw):
    return orc.prefill_causal(q, k, v, w.m, w.q_stride, w.kv_stride,
                              w.num_q_heads, w.heads_per_kv, w.head_dim, **kw)


def _decode_case(seed, b, hq, hkv, d, max_seq, t, window=0, sigma=1.0,
                 spike_frac=0.0, spike_scale=1.0):
    w = synth.DecodeWorkload("t", batch=b, num_heads=hq, kv_heads=hkv,
                             head_dim=d, max_seq=max_seq, total_seq=t,
                             window=window, sigma=sigma, spike_frac=spike_frac,
                             spike_scale=spike_scale, seed=seed)
    return w, synth.decode_inputs(w)


def _run_decode(orc, w, q, k, v, **kw):
    return orc.decode(q, k, v, w.batch, w.num_heads, w.kv_heads, w.head_dim,
                      w.max_seq, w.total_seq, w.window, w.scale, **kw)


# ---------------------------------------------------------------- page facts

def test_decode_total_seq_one_is_v_row0(orc, golden):
    """Bypass kernel of the decode page: total_seq = 1 returns V[g, 0]."""
    for i, shp in enumerate(golden["decode_bypass"]["shapes"]):
        w, (q, k, v) = _decode_case(10 + i, shp["batch"], shp["num_heads"],
                                    shp["kv_heads"], shp["head_dim"],
                                    shp["max_seq"], 1)
        out = _run_decode(orc, w, q, k, v)
        rep = w.num_heads // w.kv_heads
        for b in range(w.batch):
            for h in range(w.num_heads):
                assert np.array_equal(out[b, h], v[b, h // rep, 0].astype(np.float64))


def test_prefill_row0_is_v_row0(orc):
    """Causal range j <= i: row 0 attends only key 0, so O[0] = V[0]."""
    w, (q, k, v) = _prefill_case(20, 9, 6, 3, 64, q_pad=32, kv_pad=64)
    out = _run_prefill(orc, w, q, k, v)
    d = w.head_dim
    for h in range(w.num_q_heads):
        g = h // w.heads_per_kv
        assert np.array_equal(out[0, h], v[0, g * d:(g + 1) * d].astype(np.float64))


def test_prefill_scale_is_f32_inverse_sqrt(orc):
    """The prefill scale is 1/sqrt(head_dim) evaluated in f32 (IEEE-rounded
    sqrt and divide, here done by numpy's float32 ops)."""
    for d in (32, 64, 96, 128, 256):
        want = np.float32(1.0) / np.sqrt(np.float32(d))
        assert orc.prefill_scale(d) == float(want)


# -------------------------------------------------------------- closed forms

def test_decode_closed_form_scores_0_1_2(orc):
    """q = 2 e0, k_j = j e0, scale 0.5 gives scores exactly 0, 1, 2, so the
    weights are 1, e, e^2 over their sum."""
    d = 32
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 2.0
    k = np.zeros((1, 1, 3, d), np.float32)
    for j in range(3):
        k[0, 0, j, 0] = j
    v = _rng(1).standard_normal((1, 1, 3, d), dtype=np.float32)
    out = orc.decode(q, k, v, 1, 1, 1, d, 3, 3, 0, 0.5)
    wts = np.array([1.0, math.e, math.e ** 2])
    want = (wts[:, None] * v[0, 0].astype(np.float64)).sum(0) / wts.sum()
    np.testing.assert_allclose(out[0, 0], want, rtol=RTOL, atol=1e-15)


def test_prefill_closed_form_scale(orc):
    """Prefill with q = a e0 and k_j = b_j e0 has scores scale*a*b_j with the
    f32 scale 1/sqrt(d): checks that the scale is applied, once, with the
    right sign."""
    d, m = 32, 4
    q = np.zeros((m, d), np.float32)
    k = np.zeros((m, d), np.float32)
    q[:, 0] = 3.0
    k[:, 0] = [0.0, 1.0, -2.0, 4.0]
    v = _rng(2).standard_normal((m, d), dtype=np.float32)
    out = orc.prefill_causal(q, k, v, m, d, d, 1, 1, d)
    s = float(np.float32(1.0) / np.sqrt(np.float32(d)))
    for i in range(m):
        sc = np.array([s * 3.0 * float(k[j, 0]) for j in range(i + 1)])
        wts = np.exp(sc - sc.max())
        want = (wts[:, None] * v[: i + 1].astype(np.float64)).sum(0) / wts.sum()
        np.testing.assert_allclose(out[i, 0], want, rtol=RTOL, atol=1e-15)


def test_extreme_scores_stay_finite(orc):
    """Scores 0, 800, -800 (beyond exp's range when shifted the wrong way):
    the softmax must put all weight on the 800 row, exactly (e^-800 is 0)."""
    d = 32
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    k = np.zeros((1, 1, 3, d), np.float32)
    k[0, 0, :, 0] = [0.0, 800.0, -800.0]
    v = _rng(3).standard_normal((1, 1, 3, d), dtype=np.float32)
    out = orc.decode(q, k, v, 1, 1, 1, d, 3, 3, 0, 1.0)
    assert np.array_equal(out[0, 0], v[0, 0, 1].astype(np.float64))


def test_prefill_zero_q_is_cumulative_mean(orc):
    """Q = 0 makes every score 0: row i is the mean of V rows 0..i."""
    w, (q, k, v) = _prefill_case(30, 37, 4, 2, 32)
    q[:] = 0.0
    out = _run_prefill(orc, w, q, k, v)
    d = w.head_dim
    for h in range(w.num_q_heads):
        g = h // w.heads_per_kv
        vg = v[:, g * d:(g + 1) * d].astype(np.float64)
        want = np.cumsum(vg, axis=0) / np.arange(1, w.m + 1)[:, None]
        np.testing.assert_allclose(out[:, h], want, rtol=RTOL, atol=1e-13)


def test_identical_keys_give_mean_of_v(orc):
    """All keys equal: uniform weights, output = mean of the attended V rows."""
    w, (q, k, v) = _decode_case(40, 2, 4, 2, 64, 50, 41, window=17)
    k[:] = k[:, :, :1, :]
    out = _run_decode(orc, w, q, k, v)
    w0 = w.total_seq - w.window
    for b in range(w.batch):
        for h in range(w.num_heads):
            g = h // 2
            want = v[b, g, w0:w.total_seq].astype(np.float64).mean(0)
            np.testing.assert_allclose(out[b, h], want, rtol=RTOL, atol=1e-13)


# ---------------------------------------------------------------- invariants

def test_prefill_future_independence(orc):
    """Changing K/V rows j > i leaves row i bit-for-bit unchanged."""
    w, (q, k, v) = _prefill_case(50, 40, 4, 4, 32)
    out0 = _run_prefill(orc, w, q, k, v)
    cut = 23
    k2, v2 = k.copy(), v.copy()
    k2[cut + 1:] = _rng(51).standard_normal(k2[cut + 1:].shape, dtype=np.float32)
    v2[cut + 1:] *= -3.0
    out1 = _run_prefill(orc, w, q, k2, v2)
    assert np.array_equal(out0[: cut + 1], out1[: cut + 1])
    assert not np.allclose(out0[cut + 1:], out1[cut + 1:])


def test_prefill_gqa_is_mha_with_consecutive_repeat(orc):
    """GQA with heads_per_kv = r equals MHA over K/V heads repeated r times
    consecutively (h / r), and differs from the interleaved h % Hkv map."""
    w, (q, k, v) = _prefill_case(60, 21, 6, 3, 32)
    d, hkv, r = w.head_dim, w.kv_heads, w.heads_per_kv
    out = _run_prefill(orc, w, q, k, v)
    kh = k.reshape(w.m, hkv, d)
    vh = v.reshape(w.m, hkv, d)
    k_rep = np.ascontiguousarray(np.repeat(kh, r, axis=1).reshape(w.m, -1))
    v_rep = np.ascontiguousarray(np.repeat(vh, r, axis=1).reshape(w.m, -1))
    mha = orc.prefill_causal(q, k_rep, v_rep, w.m, w.q_stride, w.num_q_heads * d,
                             w.num_q_heads, 1, d)
    assert np.array_equal(out, mha)
    k_til = np.ascontiguousarray(np.tile(kh, (1, r, 1)).reshape(w.m, -1))
    v_til = np.ascontiguousarray(np.tile(vh, (1, r, 1)).reshape(w.m, -1))
    wrong = orc.prefill_causal(q, k_til, v_til, w.m, w.q_stride,
                               w.num_q_heads * d, w.num_q_heads, 1, d)
    assert not np.allclose(out, wrong)


def test_decode_gqa_is_mha_with_consecutive_repeat(orc):
    w, (q, k, v) = _decode_case(61, 2, 8, 2, 32, 30, 30)
    out = _run_decode(orc, w, q, k, v)
    r = w.heads_per_kv
    k_rep = np.ascontiguousarray(np.repeat(k, r, axis=1))
    v_rep = np.ascontiguousarray(np.repeat(v, r, axis=1))
    mha = orc.decode(q, k_rep, v_rep, w.batch, w.num_heads, w.num_heads,
                     w.head_dim, w.max_seq, w.total_seq, 0, w.scale)
    assert np.array_equal(out, mha)


def test_window_equals_truncated_cache(orc):
    """window = w equals window = 0 over a cache holding only rows [T-w, T);
    out-of-window spikes (x8 K rows) have no effect."""
    w, (q, k, v) = _decode_case(70, 2, 4, 2, 32, 64, 57, window=13, sigma=0.5,
                                spike_frac=0.2, spike_scale=8.0)
    out = _run_decode(orc, w, q, k, v)
    lo = w.total_seq - w.window
    kt = np.ascontiguousarray(k[:, :, lo:w.total_seq])
    vt = np.ascontiguousarray(v[:, :, lo:w.total_seq])
    trunc = orc.decode(q, kt, vt, w.batch, w.num_heads, w.kv_heads, w.head_dim,
                       w.window, w.window, 0, w.scale)
    assert np.array_equal(out, trunc)
    # rows before the window may hold anything
    k2 = k.copy()
    k2[:, :, :lo] = 1e3
    assert np.array_equal(_run_decode(orc, w, q, k2, v), out)


def test_window_edge_values(orc):
    w, (q, k, v) = _decode_case(71, 3, 6, 3, 64, 40, 33)
    base = _run_decode(orc, w, q, k, v)
    for big in (33, 34, 1000):  # window >= total_seq keeps every row
        assert np.array_equal(_run_decode(orc, w.with_(window=big), q, k, v), base)
    one = _run_decode(orc, w.with_(window=1), q, k, v)  # last row only
    for b in range(w.batch):
        for h in range(w.num_heads):
            assert np.array_equal(one[b, h], v[b, h // 2, 32].astype(np.float64))
    # window = T - 1 drops exactly row 0
    w32 = _run_decode(orc, w.with_(window=32), q, k, v)
    kt = np.ascontiguousarray(k[:, :, 1:33])
    vt = np.ascontiguousarray(v[:, :, 1:33])
    assert np.array_equal(w32, orc.decode(q, kt, vt, 3, 6, 3, 64, 32, 32, 0, w.scale))


def test_cross_mode_decode_equals_prefill_row(orc):
    """Decode with total_seq = i+1 over a cache of prefill's K/V rows, at the
    prefill scale, equals prefill row i (same definition, both modes)."""
    w, (q, k, v) = _prefill_case(80, 19, 4, 2, 32, q_pad=4, kv_pad=8)
    out = _run_prefill(orc, w, q, k, v)
    d, hkv = w.head_dim, w.kv_heads
    kc = np.ascontiguousarray(k[:, : hkv * d].reshape(w.m, hkv, d).transpose(1, 0, 2))[None]
    vc = np.ascontiguousarray(v[:, : hkv * d].reshape(w.m, hkv, d).transpose(1, 0, 2))[None]
    s = orc.prefill_scale(d)
    for i in (0, 1, 7, 18):
        qi = np.ascontiguousarray(q[i, : w.num_q_heads * d].reshape(1, w.num_q_heads, d))
        dec = orc.decode(qi, np.ascontiguousarray(kc), np.ascontiguousarray(vc), 1,
                         w.num_q_heads, hkv, d, w.m, i + 1, 0, s)
        assert np.array_equal(dec[0], out[i])


def test_outputs_are_convex_combinations(orc):
    w, (q, k, v) = _prefill_case(90, 33, 4, 2, 32, sigma=2.0)
    out = _run_prefill(orc, w, q, k, v)
    d = w.head_dim
    for h in range(w.num_q_heads):
        g = h // 2
        vg = v[:, g * d:(g + 1) * d].astype(np.float64)
        lo = np.minimum.accumulate(vg, axis=0)
        hi = np.maximum.accumulate(vg, axis=0)
        assert np.all(out[:, h] >= lo - 1e-12) and np.all(out[:, h] <= hi + 1e-12)


def test_linear_in_v(orc):
    w, (q, k, v) = _decode_case(91, 2, 4, 1, 32, 20, 20)
    # values on a 2^-10 grid, so v + 2*v2 is exact in float32
    v = np.round(v * 1024) / np.float32(1024)
    v2 = np.round(_rng(92).standard_normal(v.shape, dtype=np.float32) * 1024) / np.float32(1024)
    a = _run_decode(orc, w, q, k, v)
    b = _run_decode(orc, w, q, k, v2)
    c = _run_decode(orc, w, q, k, np.ascontiguousarray(v + 2 * v2))
    np.testing.assert_allclose(c, a + 2 * b, rtol=1e-9, atol=1e-9)


def test_selected_pairs_match_full(orc):
    w, (q, k, v) = _prefill_case(93, 29, 6, 2, 64)
    full = _run_prefill(orc, w, q, k, v)
    rows = np.array([0, 28, 5, 17, 17])
    heads = np.array([5, 0, 3, 1, 4])
    sel = _run_prefill(orc, w, q, k, v, rows=rows, heads=heads)
    assert np.array_equal(sel, full[rows, heads])
    wd, (qd, kd, vd) = _decode_case(94, 3, 6, 2, 32, 12, 10, window=4)
    fulld = _run_decode(orc, wd, qd, kd, vd)
    bs, hs = np.array([2, 0, 1]), np.array([5, 0, 3])
    assert np.array_equal(_run_decode(orc, wd, qd, kd, vd, bs=bs, hs=hs), fulld[bs, hs])


# ---------------------------------------------------- library cross-checks

def _sdpa(q, k, v, causal, scale):
    return F.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)


@pytest.mark.parametrize("m,hq,hpk,d,qp,kp", [
    (16, 4, 2, 32, 0, 0),      # the tiny prefill workload's shape
    (33, 6, 3, 64, 32, 64),    # fused-QKV-style row padding
    (7, 8, 8, 32, 0, 0),       # one KV head
    (12, 5, 1, 128, 128, 0),   # MHA
])
def test_prefill_matches_torch_sdpa_fp64(orc, m, hq, hpk, d, qp, kp):
    w, (q, k, v) = _prefill_case(100 + m, m, hq, hpk, d, q_pad=qp, kv_pad=kp)
    out = _run_prefill(orc, w, q, k, v)
    hkv = hq // hpk
    qt = torch.from_numpy(q[:, : hq * d].astype(np.float64)).reshape(m, hq, d).transpose(0, 1)
    kt = torch.from_numpy(k[:, : hkv * d].astype(np.float64)).reshape(m, hkv, d).transpose(0, 1)
    vt = torch.from_numpy(v[:, : hkv * d].astype(np.float64)).reshape(m, hkv, d).transpose(0, 1)
    kt = kt.repeat_interleave(hpk, dim=0).contiguous()
    vt = vt.repeat_interleave(hpk, dim=0).contiguous()
    ref = _sdpa(qt.contiguous(), kt, vt, True, orc.prefill_scale(d))
    np.testing.assert_allclose(out, ref.transpose(0, 1).numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("b,hq,hkv,d,ms,t,win", [
    (2, 12, 2, 128, 70, 64, 0),
    (3, 4, 4, 32, 50, 50, 9),
    (1, 8, 2, 64, 20, 11, 3),
])
def test_decode_matches_torch_sdpa_fp64(orc, b, hq, hkv, d, ms, t, win):
    w, (q, k, v) = _decode_case(200 + t, b, hq, hkv, d, ms, t, window=win)
    out = _run_decode(orc, w, q, k, v)
    lo = t - win if (win and t > win) else 0
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    kt = torch.from_numpy(k[:, :, lo:t].astype(np.float64))
    vt = torch.from_numpy(v[:, :, lo:t].astype(np.float64))
    # torch's own GQA head map (enable_gqa) must agree too
    ref_gqa = F.scaled_dot_product_attention(qt, kt, vt, scale=w.scale, enable_gqa=True)
    kt = kt.repeat_interleave(hq // hkv, dim=1)
    vt = vt.repeat_interleave(hq // hkv, dim=1)
    ref = _sdpa(qt, kt, vt, False, w.scale)
    np.testing.assert_allclose(out, ref[:, :, 0].numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out, ref_gqa[:, :, 0].numpy(), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- kv append

def test_kv_append_writes_only_position(orc):
    b, hkv, d, ms, pos = 3, 2, 64, 9, 4
    k_src, v_src = synth.append_inputs(b, hkv, d, seed=300)
    kc = np.full((b, hkv, ms, d), -7.25, np.float32)
    vc = np.full((b, hkv, ms, d), 3.5, np.float32)
    orc.kv_append(k_src, v_src, kc, vc, b, hkv, d, ms, pos)
    assert np.array_equal(kc[:, :, pos], k_src)
    assert np.array_equal(vc[:, :, pos], v_src)
    mask = np.ones(ms, bool)
    mask[pos] = False
    assert np.all(kc[:, :, mask] == -7.25) and np.all(vc[:, :, mask] == 3.5)
    with pytest.raises(ValueError):
        orc.kv_append(k_src, v_src, kc, vc, b, hkv, d, ms, ms)


# ------------------------------------------------------------- generator

def test_generator_is_seeded_and_shaped():
    w = synth.WORKLOADS["prefill_hq4_hkv2_d32_m16"]
    a = synth.prefill_inputs(w)
    b = synth.prefill_inputs(w)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert a[0].shape == (16, 128) and a[1].shape == (16, 64) and a[0].dtype == np.float32
    wd = synth.DecodeWorkload("t", batch=2, num_heads=4, kv_heads=2, head_dim=32,
                              max_seq=1000, total_seq=1000, window=100, sigma=0.5,
                              spike_frac=0.01, spike_scale=8.0, seed=5)
    q, k, v = synth.decode_inputs(wd)
    assert k.shape == (2, 2, 1000, 32)
    norms = np.abs(k).max(axis=-1).reshape(-1)
    # exactly floor(1% of 4000) = 40 spiky rows (x8 of sigma 0.5)
    assert (norms > 3.0).sum() >= 30
    assert abs(float(v.std()) - 0.5) < 0.01
