"""Pins of the oracle's rotary embedding and fused decode step.

Rotate-half rotary embedding (glia honeycrisp "attention.rs" page, fused
RoPE + KV-append + decode kernel) turns each pair (x[i], x[i + d/2]) by an
angle given by its cosine and sine. The pins use a route the oracle does
not: complex multiplication (x[i] + i x[i+d/2]) * (cos + i sin), plus exact
special angles, norm preservation, composition of angles and the
relative-position property that motivates the construction.
"""
import numpy as np
import pytest

import synth


def _angles(d, pos, base=10000.0):
    i = np.arange(d // 2, dtype=np.float64)
    return pos * base ** (-2.0 * i / d)


def _tables(d, pos):
    th = _angles(d, pos)
    return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)


def test_rope_is_complex_rotation(orc):
    rng = np.random.default_rng(1)
    d = 128
    x = rng.standard_normal((5, d), dtype=np.float32)
    c, s = _tables(d, 37)
    got = orc.rope(x, c, s)
    z = (x[:, : d // 2].astype(np.float64) + 1j * x[:, d // 2:].astype(np.float64)) * \
        (c.astype(np.float64) + 1j * s.astype(np.float64))
    want = np.concatenate([z.real, z.imag], axis=1)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)


def test_rope_special_angles(orc):
    rng = np.random.default_rng(2)
    d = 64
    x = rng.standard_normal((3, d), dtype=np.float32)
    one, zero = np.ones(d // 2, np.float32), np.zeros(d // 2, np.float32)
    assert np.array_equal(orc.rope(x, one, zero), x.astype(np.float64))  # angle 0
    q = orc.rope(x, zero, one)                                           # angle 90 deg
    assert np.array_equal(q[:, : d // 2], -x[:, d // 2:].astype(np.float64))
    assert np.array_equal(q[:, d // 2:], x[:, : d // 2].astype(np.float64))
    h = orc.rope(x, -one, zero)                                          # angle 180 deg
    assert np.array_equal(h, -x.astype(np.float64))


def test_rope_preserves_pair_norms_and_composes(orc):
    rng = np.random.default_rng(3)
    d = 128
    x = rng.standard_normal((4, d), dtype=np.float32)
    c1, s1 = _tables(d, 11)
    y = orc.rope(x, c1, s1)
    n0 = x[:, : d // 2].astype(np.float64) ** 2 + x[:, d // 2:].astype(np.float64) ** 2
    n1 = y[:, : d // 2] ** 2 + y[:, d // 2:] ** 2
    scale = c1.astype(np.float64) ** 2 + s1.astype(np.float64) ** 2
    np.testing.assert_allclose(n1, n0 * scale, rtol=1e-13)
    # R(11) then R(29) = R(40), up to the float32 rounding of the tables
    c2, s2 = _tables(d, 29)
    c3, s3 = _tables(d, 40)
    twice = orc.rope(y.astype(np.float32), c2, s2)
    once = orc.rope(x, c3, s3)
    np.testing.assert_allclose(twice, once, rtol=0, atol=5e-6)


def test_rope_relative_position(orc):
    """<R(p) q, R(p') k> depends only on p - p' (the point of rotary codes)."""
    rng = np.random.default_rng(4)
    d = 128
    q = rng.standard_normal((1, d), dtype=np.float32)
    k = rng.standard_normal((1, d), dtype=np.float32)
    vals = []
    for p, pk in ((50, 20), (130, 100), (31, 1)):
        qp = orc.rope(q, *_tables(d, p))
        kp = orc.rope(k, *_tables(d, pk))
        vals.append(float((qp * kp).sum()))
    np.testing.assert_allclose(vals, vals[0], rtol=0, atol=2e-4)


def test_decode_rope_append_is_rotate_append_decode(orc):
    """The fused step equals: rotate q and the new K rows, append rotated K
    and raw V, decode at total_seq = position + 1 (up to the fp32 rounding
    of the rotated q handed to plain decode)."""
    b, hq, hkv, d, ms, pos, win = 2, 12, 2, 128, 300, 257, 100
    w = synth.DecodeWorkload("t", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=ms, total_seq=pos + 1, window=win, seed=5)
    q, k, v = synth.decode_inputs(w)
    kn, vn = synth.append_inputs(b, hkv, d, seed=6)
    c, s = _tables(d, pos)
    k1, v1 = k.copy(), v.copy()
    fused = orc.decode_rope_append(q, kn, vn, c, s, k1, v1, b, hq, hkv, d, ms, pos, win, w.scale)
    # cache rows: rotated K (fp32), raw V; nothing else changed
    krot = orc.rope(kn, c, s).astype(np.float32)
    assert np.array_equal(k1[:, :, pos], krot) and np.array_equal(v1[:, :, pos], vn)
    mask = np.ones(ms, bool)
    mask[pos] = False
    assert np.array_equal(k1[:, :, mask], k[:, :, mask])
    qrot = np.ascontiguousarray(orc.rope(q, c, s).astype(np.float32))
    plain = orc.decode(qrot, k1, v1, b, hq, hkv, d, ms, pos + 1, win, w.scale)
    np.testing.assert_allclose(fused, plain, rtol=0, atol=2e-6)
    # angle 0 reduces the step to the plain append + decode
    one, zero = np.ones(d // 2, np.float32), np.zeros(d // 2, np.float32)
    k2, v2 = k.copy(), v.copy()
    f0 = orc.decode_rope_append(q, kn, vn, one, zero, k2, v2, b, hq, hkv, d, ms, pos, win,
                                w.scale)
    k3, v3 = k.copy(), v.copy()
    orc.kv_append(kn, vn, k3, v3, b, hkv, d, ms, pos)
    assert np.array_equal(k2, k3) and np.array_equal(v2, v3)
    np.testing.assert_allclose(f0, orc.decode(q, k3, v3, b, hq, hkv, d, ms, pos + 1, win,
                                              w.scale), rtol=1e-13, atol=1e-14)
