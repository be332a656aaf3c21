"""Pins of the oracle's serving-side operations: the bulk append of a
prefill pass's K/V rows into a sequence's caches (the page's KV-append
kernels taken over M rows of the packed prefill layout), and decode of a
batch whose sequences have their own lengths (the Params struct's
total_seq, one per sequence).

Routes independent of the oracle's loops: numpy reshape/transpose for the
cache layout, torch's scaled_dot_product_attention in float64 per sequence,
and the already-pinned prefill and single-length decode.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth


def _packed_kv(seed, m, hkv, d, pad):
    rng = np.random.default_rng(seed)
    stride = hkv * d + pad
    k = rng.standard_normal((m, stride), dtype=np.float32)
    v = rng.standard_normal((m, stride), dtype=np.float32)
    k[:, hkv * d:] = 1e6   # padding columns must never reach a cache
    v[:, hkv * d:] = -1e6
    return k, v, stride


def test_kv_append_rows_is_a_slice_copy(orc):
    m, hkv, d, ms, pos = 7, 3, 32, 20, 9
    k, v, stride = _packed_kv(1, m, hkv, d, pad=8)
    kc = np.full((hkv, ms, d), -5.0, np.float32)
    vc = np.full((hkv, ms, d), 6.0, np.float32)
    orc.kv_append_rows(k, v, kc, vc, m, stride, hkv, d, ms, pos)
    ek = np.full_like(kc, -5.0)
    ev = np.full_like(vc, 6.0)
    ek[:, pos:pos + m] = k[:, :hkv * d].reshape(m, hkv, d).transpose(1, 0, 2)
    ev[:, pos:pos + m] = v[:, :hkv * d].reshape(m, hkv, d).transpose(1, 0, 2)
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)


def test_kv_append_rows_bounds(orc):
    m, hkv, d, ms = 5, 2, 32, 8
    k, v, stride = _packed_kv(2, m, hkv, d, pad=0)
    kc = np.zeros((hkv, ms, d), np.float32)
    vc = np.zeros((hkv, ms, d), np.float32)
    orc.kv_append_rows(k, v, kc, vc, m, stride, hkv, d, ms, ms - m)   # fills to the end
    assert np.array_equal(kc[:, ms - m:], k.reshape(m, hkv, d).transpose(1, 0, 2))
    with pytest.raises(ValueError):
        orc.kv_append_rows(k, v, kc, vc, m, stride, hkv, d, ms, ms - m + 1)
    with pytest.raises(ValueError):
        orc.kv_append_rows(k, v, kc, vc, m, hkv * d - 4, hkv, d, ms, 0)
    before = kc.copy()
    orc.kv_append_rows(k, v, kc, vc, 0, stride, hkv, d, ms, ms)       # no rows: no change
    assert np.array_equal(kc, before)


def test_prefill_then_bulk_append_then_decode(orc):
    """Prefill row i equals a decode of Q row i over the first i+1 cache rows
    after the prefill's K/V rows were appended from position 0."""
    m, hq, hpk, d = 23, 6, 3, 32
    w = synth.PrefillWorkload("t", m=m, num_q_heads=hq, heads_per_kv=hpk, head_dim=d,
                              q_stride=hq * d + 4, kv_stride=(hq // hpk) * d + 12, seed=9)
    q, k, v = synth.prefill_inputs(w)
    out = orc.prefill_causal(q, k, v, m, w.q_stride, w.kv_stride, hq, hpk, d)
    hkv, ms = hq // hpk, 30
    kc = np.full((hkv, ms, d), np.nan, np.float32)   # rows past m stay unread
    vc = np.full((hkv, ms, d), np.nan, np.float32)
    orc.kv_append_rows(k, v, kc, vc, m, w.kv_stride, hkv, d, ms, 0)
    s = orc.prefill_scale(d)
    for i in (0, 5, m - 1):
        qi = np.ascontiguousarray(q[i, :hq * d].reshape(1, hq, d))
        dec = orc.decode(qi, kc, vc, 1, hq, hkv, d, ms, i + 1, 0, s)
        assert np.array_equal(dec[0], out[i])


@pytest.mark.parametrize("window", [0, 6])
def test_decode_varlen_matches_sdpa_per_sequence(orc, window):
    b, hq, hkv, d, ms = 6, 8, 2, 32, 20
    lens = np.array([0, 1, 7, 20, 13, 6], np.uint32)
    w = synth.DecodeWorkload("t", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=ms, total_seq=ms, seed=4)
    q, k, v = synth.decode_inputs(w)
    out = orc.decode_varlen(q, k, v, lens, b, hq, hkv, d, ms, window, w.scale)
    assert np.all(out[0] == 0.0)                      # idle slot
    for i in range(1, b):
        t = int(lens[i])
        lo = t - window if (window and t > window) else 0
        qt = torch.from_numpy(q[i].astype(np.float64))[None, :, None, :]
        kt = torch.from_numpy(k[i, :, lo:t].astype(np.float64))[None]
        vt = torch.from_numpy(v[i, :, lo:t].astype(np.float64))[None]
        ref = F.scaled_dot_product_attention(qt, kt, vt, scale=w.scale, enable_gqa=True)
        np.testing.assert_allclose(out[i], ref[0, :, 0].numpy(), rtol=1e-10, atol=1e-12)


def test_decode_varlen_equal_lengths_is_decode(orc):
    b, hq, hkv, d, ms, t = 3, 12, 2, 64, 40, 33
    w = synth.DecodeWorkload("t", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=ms, total_seq=t, window=10, seed=5)
    q, k, v = synth.decode_inputs(w)
    ref = orc.decode(q, k, v, b, hq, hkv, d, ms, t, 10, w.scale)
    got = orc.decode_varlen(q, k, v, np.full(b, t, np.uint32), b, hq, hkv, d, ms, 10, w.scale)
    assert np.array_equal(got, ref)


def test_decode_varlen_sequences_are_independent(orc):
    """Changing one sequence's length or cache changes only its outputs."""
    b, hq, hkv, d, ms = 4, 4, 4, 32, 16
    w = synth.DecodeWorkload("t", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=ms, total_seq=ms, seed=6)
    q, k, v = synth.decode_inputs(w)
    lens = np.array([16, 3, 9, 1], np.uint32)
    a = orc.decode_varlen(q, k, v, lens, b, hq, hkv, d, ms, 0, w.scale)
    lens2 = lens.copy()
    lens2[2] = 12
    k2 = k.copy()
    k2[1, :, 5:] = 99.0            # past sequence 1's length: never read
    bb = orc.decode_varlen(q, k2, v, lens2, b, hq, hkv, d, ms, 0, w.scale)
    assert np.array_equal(a[[0, 1, 3]], bb[[0, 1, 3]])
    assert not np.array_equal(a[2], bb[2])


def test_decode_varlen_rejects_lengths_past_the_cache(orc):
    b, hq, hkv, d, ms = 2, 2, 1, 32, 8
    q = np.zeros((b, hq, d), np.float32)
    kc = np.zeros((b, hkv, ms, d), np.float32)
    with pytest.raises(ValueError):
        orc.decode_varlen(q, kc, kc, np.array([8, 9], np.uint32), b, hq, hkv, d, ms, 0, 0.1)


def test_seq_lengths_generator():
    lens = synth.seq_lengths(32, 4096, seed=3, idle=2)
    assert lens.dtype == np.uint32 and lens.shape == (32,)
    assert lens.max() == 4096 and int((lens == 0).sum()) == 2
    assert np.array_equal(lens, synth.seq_lengths(32, 4096, seed=3, idle=2))
