"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bar: max |GPU - oracle| <= 2e-5 * max|V|, with max|V| over the V elements the
call may attend (all of V's head columns for prefill; rows [w0, T) of every
cache for decode). kv_append is bit-exact. Inputs come from synth (seeded).
Full workload sizes are checked element by element where the oracle is fast
(decode, the two smaller prefills) and on a stated sample of (row, head)
outputs for the long prefill.
"""
import sys

import numpy as np
import pytest
import torch

import attention_gqa_online_amd as A
import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 2e-5


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    A.library()
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", file=sys.stderr, flush=True)


def _err(got, ref):
    return float(np.abs(got.astype(np.float64) - ref).max()) if ref.size else 0.0


def _assert_close(got, ref, vmax, what):
    err = _err(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= TOL * vmax, f"{what}: max|err| {err:.3e} > {TOL * vmax:.3e} (max|V| {vmax:.3f})"
    return err


def _poisoned_ws(nbytes, batch, num_heads, dev):
    """A decode workspace of every byte 0xFF (NaN floats: a partial state read
    before this call wrote it shows as NaN), except the arrival counters,
    which must be zero before the first use: the first 65536 bytes, or
    4 * batch * num_heads rounded up to 256 where that is more."""
    ws = torch.full((max(1, nbytes),), 0xFF, dtype=torch.uint8, device=dev)
    ws[: max(65536, (4 * batch * num_heads + 255) // 256 * 256)] = 0
    return ws


# ------------------------------------------------------------------ decode

def _gpu_decode(dev, w, q, k, v, ws=None, out=None):
    qd = torch.from_numpy(q).to(dev)
    kd = torch.from_numpy(k).to(dev)
    vd = torch.from_numpy(v).to(dev)
    if out is None:
        out = torch.full((w.batch, w.num_heads, w.head_dim), float("nan"), device=dev)
    if ws is None:
        ws = A.decode_workspace(w.batch, w.num_heads, w.kv_heads, w.head_dim,
                                w.total_seq, w.window, device=dev)
    A.attn_decode(qd, kd, vd, out, w.batch, w.num_heads, w.kv_heads, w.head_dim,
                  w.max_seq, w.total_seq, w.window, w.scale, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ref_decode(w, q, k, v):
    return oracle.decode(q, k, v, w.batch, w.num_heads, w.kv_heads, w.head_dim,
                         w.max_seq, w.total_seq, w.window, w.scale)


def _vmax_decode(w, v):
    return float(np.abs(v[:, :, w.window_start:w.total_seq]).max())


def _decode_case(b, hq, hkv, d, max_seq, t, window=0, sigma=1.0, seed=0, **kw):
    w = synth.DecodeWorkload("case", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=max_seq, total_seq=t, window=window, sigma=sigma,
                             seed=seed, **kw)
    return w, synth.decode_inputs(w)


@pytest.mark.parametrize("name", ["decode_b32_hq12_hkv2_d128_t4096",
                                  "decode_b16_hq32_hkv8_d128_t32768_w4096"])
def test_decode_full_workloads(dev, name):
    w = synth.WORKLOADS[name]
    q, k, v = synth.decode_inputs(w)
    got = _gpu_decode(dev, w, q, k, v)
    _assert_close(got, _ref_decode(w, q, k, v), _vmax_decode(w, v), name)


DECODE_SWEEP = [
    # (batch, hq, hkv, d, max_seq, total_seq, window)
    (1, 1, 1, 32, 8, 1, 0),
    (2, 4, 2, 32, 70, 65, 0),
    (3, 8, 8, 64, 130, 129, 0),
    (2, 6, 2, 64, 300, 257, 31),
    (1, 12, 2, 128, 1, 1, 0),
    (2, 12, 2, 128, 5, 3, 0),
    (2, 12, 2, 128, 64, 63, 0),
    (2, 12, 2, 128, 600, 511, 0),
    (2, 12, 2, 128, 600, 513, 0),
    (1, 12, 2, 128, 5000, 4097, 0),
    (2, 12, 2, 128, 2000, 1000, 1),
    (2, 12, 2, 128, 2000, 1000, 999),
    (2, 12, 2, 128, 2000, 1000, 1000),
    (2, 12, 2, 128, 2000, 1000, 1005),
    (2, 12, 2, 128, 2000, 1000, 129),
    (1, 3, 1, 128, 100, 77, 0),
    (1, 5, 1, 128, 100, 77, 13),
    (2, 7, 1, 128, 400, 333, 0),
    (2, 16, 2, 128, 300, 300, 0),     # 8 Q heads per KV head
    (1, 9, 1, 128, 200, 150, 0),      # 9 -> two chunks of 5 and 4 heads
    (1, 24, 2, 128, 200, 190, 0),     # 12 per KV head -> two chunks of 6
    (1, 16, 1, 64, 300, 299, 0),      # 16 per KV head -> two chunks of 8
    (2, 4, 4, 256, 300, 200, 0),
    (1, 8, 1, 256, 500, 480, 100),
    (1, 2, 1, 32, 20000, 20000, 0),   # many splits
    (64, 8, 4, 128, 300, 300, 0),     # 256 units: one split, output written directly
    (80, 12, 4, 64, 200, 170, 50),    # 320 units, one split, windowed
    (1, 32, 8, 128, 9000, 9000, 4096),
    # head sizes held in 8 lanes per row, and capped head chunks
    (2, 12, 2, 96, 300, 257, 0),
    (1, 8, 1, 160, 500, 480, 100),    # 8 heads per KV head -> chunks of 4 (cap 6)
    (3, 4, 4, 160, 200, 130, 7),
    (2, 6, 2, 192, 300, 299, 0),
    (1, 10, 2, 224, 600, 513, 0),     # 5 per KV head -> chunks of 3 and 2 (cap 4)
    (64, 4, 4, 224, 100, 77, 0),      # 256 units, one split
]


@pytest.mark.parametrize("case", DECODE_SWEEP, ids=lambda c: "b{}_hq{}_hkv{}_d{}_ms{}_t{}_w{}".format(*c))
def test_decode_sweep(dev, case):
    w, (q, k, v) = _decode_case(*case, seed=hash(case) % 1000)
    got = _gpu_decode(dev, w, q, k, v)
    _assert_close(got, _ref_decode(w, q, k, v), _vmax_decode(w, v), str(case))


def _random_decode_shapes(n, seed):
    """Seeded decode shapes: head sizes, GQA ratios (including ones that take
    two head chunks), batch, cache lengths, attended lengths and windows."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([32, 64, 96, 128, 160, 192, 224, 256]))
        hkv = int(rng.integers(1, 5))
        hpk = int(rng.choice([1, 2, 3, 4, 6, 8, 9, 12, 16]))
        b = int(rng.integers(1, 7))
        max_seq = int(rng.integers(1, 3000))
        t = int(rng.integers(1, max_seq + 1))
        window = 0 if rng.random() < 0.5 else int(rng.integers(1, t + 10))
        out.append((b, hkv * hpk, hkv, d, max_seq, t, window))
    return out


DECODE_RANDOM = _random_decode_shapes(24, 4048)


@pytest.mark.parametrize("case", DECODE_RANDOM, ids=lambda c: "b{}_hq{}_hkv{}_d{}_ms{}_t{}_w{}".format(*c))
def test_decode_random_shapes(dev, case):
    w, (q, k, v) = _decode_case(*case, seed=sum(case) % 997)
    got = _gpu_decode(dev, w, q, k, v)
    _assert_close(got, _ref_decode(w, q, k, v), _vmax_decode(w, v), str(case))


def test_decode_spiky_window(dev):
    """N(0, 0.5) values with 1% of K rows x8 over all positions: the
    out-of-window spikes must not leak in, in-window ones stress the max."""
    w, (q, k, v) = _decode_case(4, 32, 8, 128, 6000, 6000, window=2048, sigma=0.5,
                                spike_frac=0.01, spike_scale=8.0, seed=44)
    got = _gpu_decode(dev, w, q, k, v)
    _assert_close(got, _ref_decode(w, q, k, v), _vmax_decode(w, v), "spiky")


def test_decode_total_seq_one_returns_v_row0(dev):
    w, (q, k, v) = _decode_case(3, 12, 2, 128, 9, 1, seed=5)
    got = _gpu_decode(dev, w, q, k, v)
    rep = w.num_heads // w.kv_heads
    for b in range(w.batch):
        for h in range(w.num_heads):
            assert np.array_equal(got[b, h], v[b, h // rep, 0])


def test_decode_large_scores_stay_finite(dev):
    """Scores far apart (x100 scale): one row dominates, nothing overflows."""
    w, (q, k, v) = _decode_case(2, 12, 2, 128, 700, 650, seed=6)
    w = w.with_(scale=float(np.float32(w.scale * 100)))
    got = _gpu_decode(dev, w, q, k, v)
    _assert_close(got, _ref_decode(w, q, k, v), _vmax_decode(w, v), "large scores")


def test_decode_deterministic_and_workspace_reused(dev):
    """Two identical calls give identical bits; one workspace, cleared only
    where the counters are (the rest NaN bytes up front), serves calls of
    different shapes."""
    big = A.attn_decode_workspace_bytes(32, 12, 2, 128, 4096, 0)
    ws = _poisoned_ws(big, 32, 12, dev)
    w, (q, k, v) = _decode_case(8, 12, 2, 128, 3000, 2900, seed=9)
    a = _gpu_decode(dev, w, q, k, v, ws=ws)
    b = _gpu_decode(dev, w, q, k, v, ws=ws)
    assert np.array_equal(a, b)
    w2, (q2, k2, v2) = _decode_case(3, 8, 4, 64, 1500, 1400, window=700, seed=10)
    _assert_close(_gpu_decode(dev, w2, q2, k2, v2, ws=ws), _ref_decode(w2, q2, k2, v2),
                  _vmax_decode(w2, v2), "reused workspace")
    _assert_close(_gpu_decode(dev, w, q, k, v, ws=ws), _ref_decode(w, q, k, v),
                  _vmax_decode(w, v), "reused workspace, first shape again")


FUSED_MERGE_CASES = [
    # (batch, hq, hkv, d, max_seq, position, window)
    (3, 12, 2, 128, 3000, 2999, 0),    # 6 units: a unit's splits on several XCDs
    (1, 8, 1, 128, 20000, 19999, 0),   # one unit, many splits (several merge rounds)
    (5, 12, 2, 224, 2000, 1999, 300),  # two head chunks per KV head, window
    (3, 16, 2, 256, 900, 700, 0),      # 8 heads x 64 float4 items: two per thread in the merge
]


@pytest.mark.parametrize("case", FUSED_MERGE_CASES,
                         ids=lambda c: "b{}_hq{}_hkv{}_d{}_ms{}_pos{}_w{}".format(*c))
def test_decode_fused_merge_alternating_inputs(dev, case):
    """The last workgroup of each unit merges the partial states the other
    workgroups of the same launch wrote. Two input sets alternate over one
    workspace (NaN bytes apart from its counters), four decode steps and four
    plain decodes: a state left over from the previous call, or one not yet
    visible to the merging workgroup, would give a wrong or NaN output, and
    counters not returned to zero would leave the next call's output unwritten
    (NaN)."""
    b, hq, hkv, d, ms, pos, win = case
    ws = _poisoned_ws(A.attn_decode_workspace_bytes(b, hq, hkv, d, pos + 1, win), b, hq, dev)
    sets = []
    for i in range(2):
        seed = 700 + 11 * i + sum(case) % 89
        w, (q, k, v) = _decode_case(b, hq, hkv, d, ms, pos + 1, window=win, seed=seed)
        kn, vn = synth.append_inputs(b, hkv, d, seed=seed + 1)
        kf, vf = k.copy(), v.copy()
        oracle.kv_append(kn, vn, kf, vf, b, hkv, d, ms, pos)
        sets.append((w, q, k, v, kn, vn, kf, vf, _ref_decode(w, q, kf, vf), _vmax_decode(w, vf)))
    for call in range(4):
        w, q, k, v, kn, vn, kf, vf, ref, vmax = sets[call % 2]
        kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
        out = torch.full((b, hq, d), float("nan"), device=dev)
        A.attn_decode_append(torch.from_numpy(q).to(dev), torch.from_numpy(kn).to(dev),
                             torch.from_numpy(vn).to(dev), kd, vd, out, b, hq, hkv, d, ms, pos,
                             win, w.scale, ws)
        got_plain = _gpu_decode(dev, w, q, kf, vf, ws=ws)
        torch.cuda.synchronize()
        _assert_close(out.cpu().numpy(), ref, vmax, f"decode step, call {call}")
        _assert_close(got_plain, ref, vmax, f"decode, call {call}")
        assert np.array_equal(kd.cpu().numpy(), kf) and np.array_equal(vd.cpu().numpy(), vf)


def test_decode_workspace_shared_by_unit_counts(dev):
    """One workspace (zeroed once) serves calls whose unit counts differ: a
    4-unit call writes its partial states, then a 64-unit call must still find
    its counters at zero, then the 4-unit call again."""
    ws = torch.zeros(max(A.attn_decode_workspace_bytes(32, 12, 2, 128, 2048, 0),
                         A.attn_decode_workspace_bytes(2, 12, 2, 128, 6000, 0)),
                     dtype=torch.uint8, device=dev)
    small = _decode_case(2, 12, 2, 128, 6000, 6000, seed=31)
    large = _decode_case(32, 12, 2, 128, 2048, 2048, seed=32)
    for w, (q, k, v) in (small, large, small, large):
        _assert_close(_gpu_decode(dev, w, q, k, v, ws=ws), _ref_decode(w, q, k, v),
                      _vmax_decode(w, v), f"shared workspace, batch {w.batch}")


def test_decode_on_a_side_stream(dev):
    w, (q, k, v) = _decode_case(2, 12, 2, 128, 500, 500, seed=11)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
        out = torch.empty(w.batch, w.num_heads, w.head_dim, device=dev)
        ws = A.decode_workspace(w.batch, w.num_heads, w.kv_heads, w.head_dim,
                                w.total_seq, w.window, device=dev)
        A.attn_decode(qd, kd, vd, out, w.batch, w.num_heads, w.kv_heads, w.head_dim,
                      w.max_seq, w.total_seq, w.window, w.scale, ws, stream=s)
    s.synchronize()
    _assert_close(out.cpu().numpy(), _ref_decode(w, q, k, v), _vmax_decode(w, v), "stream")


# ------------------------------------------------------- decode + append

DECODE_APPEND_CASES = [
    # (batch, hq, hkv, d, max_seq, position, window)
    (2, 12, 2, 128, 8, 0, 0),          # first token: nothing cached yet
    (2, 12, 2, 128, 40, 1, 0),
    (3, 4, 2, 32, 90, 64, 0),
    (2, 6, 2, 64, 300, 256, 31),
    (2, 12, 2, 128, 2000, 999, 1),     # window 1: the new row only
    (2, 12, 2, 128, 2000, 999, 2),
    (2, 12, 2, 128, 2000, 999, 5000),  # window past the start: no window
    (1, 9, 1, 128, 300, 250, 0),       # two head chunks
    (64, 8, 4, 128, 300, 299, 0),      # 256 units
    (2, 8, 1, 256, 600, 512, 100),
    (1, 32, 8, 128, 9000, 8999, 4096),
    (2, 8, 2, 96, 300, 250, 0),
    (1, 12, 2, 224, 400, 399, 31),
]


def _random_step_shapes(n, seed):
    """Seeded (batch, hq, hkv, d, max_seq, position or length bound, window)
    cases for the fused decode steps."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([32, 64, 96, 128, 160, 192, 224, 256]))
        hkv = int(rng.integers(1, 5))
        hpk = int(rng.choice([1, 2, 3, 4, 6, 8, 9, 12]))
        b = int(rng.integers(1, 9))
        ms = int(rng.integers(1, 2500))
        pos = int(rng.integers(0, ms))
        win = 0 if rng.random() < 0.5 else int(rng.integers(1, pos + 12))
        out.append((b, hkv * hpk, hkv, d, ms, pos, win))
    return out


# seeded random cases beside the hand-picked ones
DECODE_APPEND_CASES = DECODE_APPEND_CASES + _random_step_shapes(16, 8096)


def _decode_append_case(dev, case, seed):
    b, hq, hkv, d, ms, pos, win = case
    w, (q, k, v) = _decode_case(b, hq, hkv, d, ms, pos + 1, window=win, seed=seed)
    kn, vn = synth.append_inputs(b, hkv, d, seed=seed + 1)
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    out = torch.full((b, hq, d), float("nan"), device=dev)
    ws = _poisoned_ws(A.attn_decode_workspace_bytes(b, hq, hkv, d, pos + 1, win), b, hq, dev)
    A.attn_decode_append(torch.from_numpy(q).to(dev), torch.from_numpy(kn).to(dev),
                         torch.from_numpy(vn).to(dev), kd, vd, out, b, hq, hkv, d, ms, pos,
                         win, w.scale, ws)
    torch.cuda.synchronize()
    oracle.kv_append(kn, vn, k, v, b, hkv, d, ms, pos)   # the reference step
    return w, (q, k, v), out.cpu().numpy(), kd.cpu().numpy(), vd.cpu().numpy()


@pytest.mark.parametrize("case", DECODE_APPEND_CASES,
                         ids=lambda c: "b{}_hq{}_hkv{}_d{}_ms{}_pos{}_w{}".format(*c))
def test_decode_append_matches_append_then_decode(dev, case):
    w, (q, k, v), got, kc, vc = _decode_append_case(dev, case, seed=sum(case) % 997)
    assert np.array_equal(kc, k) and np.array_equal(vc, v)  # only row `position` changed
    _assert_close(got, _ref_decode(w, q, k, v), _vmax_decode(w, v), str(case))


def test_decode_append_no_heads_only_appends(dev):
    """num_heads == 0: the step reduces to kv_append (bit-exact)."""
    b, hkv, d, ms, pos = 2, 3, 128, 12, 5
    ks, vs = synth.append_inputs(b, hkv, d, seed=31)
    kc = torch.full((b, hkv, ms, d), 2.0, device=dev)
    vc = torch.full((b, hkv, ms, d), -3.0, device=dev)
    A.attn_decode_append(0, torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev), kc, vc,
                         0, b, 0, hkv, d, ms, pos, 0, 0.1, None)
    torch.cuda.synchronize()
    kr, vr = np.full((b, hkv, ms, d), 2.0, np.float32), np.full((b, hkv, ms, d), -3.0, np.float32)
    oracle.kv_append(ks, vs, kr, vr, b, hkv, d, ms, pos)
    assert np.array_equal(kc.cpu().numpy(), kr) and np.array_equal(vc.cpu().numpy(), vr)


def test_decode_append_full_decode_workload(dev):
    """The decode workload's shape (32 x 12 heads, 4096 positions) as a decode
    step: append at position 4095, attend all 4096 rows."""
    w0 = synth.WORKLOADS["decode_b32_hq12_hkv2_d128_t4096"]
    case = (w0.batch, w0.num_heads, w0.kv_heads, w0.head_dim, w0.max_seq, 4095, 0)
    w, (q, k, v), got, kc, vc = _decode_append_case(dev, case, seed=w0.seed)
    assert np.array_equal(kc, k) and np.array_equal(vc, v)
    _assert_close(got, _ref_decode(w, q, k, v), _vmax_decode(w, v), "decode step")


# --------------------------------------------------- decode step with RoPE

def _rope_row_bound(x):
    """Per-element bound for a rotated fp32 row against the fp64 rotation
    rounded to fp32: each output is x c - x' s (or x' s + x c) with |c|,|s| <= 1;
    a product rounding, the sum's rounding and the final cast each cost at
    most 2^-24 of |x| + |x'|, so 3 * 2^-24 * (|x| + |x'|) < 2^-22 (|x| + |x'|)."""
    d = x.shape[-1]
    h = d // 2
    partner = np.concatenate([x[..., h:], x[..., :h]], axis=-1)
    return 2.0 ** -22 * (np.abs(x).astype(np.float64) + np.abs(partner))


def _decode_rope_case(dev, case, seed, scale_angles=1.0):
    b, hq, hkv, d, ms, pos, win = case
    w, (q, k, v) = _decode_case(b, hq, hkv, d, ms, pos + 1, window=win, seed=seed)
    kn, vn = synth.append_inputs(b, hkv, d, seed=seed + 1)
    cos_t, sin_t = synth.rope_tables(d, pos * scale_angles)
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    out = torch.full((b, hq, d), float("nan"), device=dev)
    ws = _poisoned_ws(A.attn_decode_workspace_bytes(b, hq, hkv, d, pos + 1, win), b, hq, dev)
    A.attn_decode_rope_append(torch.from_numpy(q).to(dev), torch.from_numpy(kn).to(dev),
                              torch.from_numpy(vn).to(dev), torch.from_numpy(cos_t).to(dev),
                              torch.from_numpy(sin_t).to(dev), kd, vd, out, b, hq, hkv, d, ms,
                              pos, win, w.scale, ws)
    torch.cuda.synchronize()
    ref = oracle.decode_rope_append(q, kn, vn, cos_t, sin_t, k, v, b, hq, hkv, d, ms, pos,
                                    win, w.scale)   # updates k, v like the step
    return w, (q, k, v, kn), ref, out.cpu().numpy(), kd.cpu().numpy(), vd.cpu().numpy()


def _check_rope_step(w, pos, q, k, v, kn, ref, got, kc, vc, label):
    # every cache row but `position` untouched, V row copied exactly
    keep = np.ones(w.max_seq, dtype=bool)
    keep[pos] = False
    assert np.array_equal(kc[:, :, keep], k[:, :, keep]), label
    assert np.array_equal(vc, v), label
    # the rotated K row within the rounding bound of the fp64 rotation
    err = np.abs(kc[:, :, pos].astype(np.float64) - k[:, :, pos])
    assert np.all(err <= _rope_row_bound(kn)), (label, float(err.max()))
    _assert_close(got, ref, _vmax_decode(w, v), label)


@pytest.mark.parametrize("case", DECODE_APPEND_CASES,
                         ids=lambda c: "b{}_hq{}_hkv{}_d{}_ms{}_pos{}_w{}".format(*c))
def test_decode_rope_append_matches_oracle(dev, case):
    w, (q, k, v, kn), ref, got, kc, vc = _decode_rope_case(dev, case, seed=sum(case) % 991)
    _check_rope_step(w, case[5], q, k, v, kn, ref, got, kc, vc, str(case))


def test_decode_rope_append_large_angles(dev):
    """Angles far from zero for every pair (positions scaled by 1e3): the
    rotation is then far from the identity in every dimension."""
    case = (3, 12, 2, 128, 700, 613, 0)
    w, (q, k, v, kn), ref, got, kc, vc = _decode_rope_case(dev, case, seed=5,
                                                           scale_angles=1000.0)
    _check_rope_step(w, case[5], q, k, v, kn, ref, got, kc, vc, "large angles")


def test_decode_rope_append_angle_zero_is_plain_step(dev):
    """cos = 1, sin = 0 turns nothing: outputs and caches equal the plain
    decode step's bit for bit."""
    b, hq, hkv, d, ms, pos, win = 2, 12, 2, 128, 500, 411, 0
    w, (q, k, v) = _decode_case(b, hq, hkv, d, ms, pos + 1, window=win, seed=77)
    kn, vn = synth.append_inputs(b, hkv, d, seed=78)
    ones = torch.ones(d // 2, device=dev)
    zeros = torch.zeros(d // 2, device=dev)
    ws = A.decode_workspace(b, hq, hkv, d, pos + 1, win)
    res = []
    for rope in (False, True):
        kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
        out = torch.full((b, hq, d), float("nan"), device=dev)
        args = (torch.from_numpy(q).to(dev), torch.from_numpy(kn).to(dev),
                torch.from_numpy(vn).to(dev))
        if rope:
            A.attn_decode_rope_append(*args, ones, zeros, kd, vd, out, b, hq, hkv, d, ms,
                                      pos, win, w.scale, ws)
        else:
            A.attn_decode_append(*args, kd, vd, out, b, hq, hkv, d, ms, pos, win, w.scale, ws)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), kd.cpu().numpy(), vd.cpu().numpy()))
    for a, r in zip(res[0], res[1]):
        assert np.array_equal(a, r)


def test_decode_rope_append_no_heads_appends_rotated_rows(dev):
    """num_heads == 0: nothing to attend, the rotated K row and the V row are
    still appended."""
    b, hkv, d, ms, pos = 3, 4, 64, 20, 17
    ks, vs = synth.append_inputs(b, hkv, d, seed=3)
    cos_t, sin_t = synth.rope_tables(d, 123.0)
    kc = torch.full((b, hkv, ms, d), -1.5, device=dev)
    vc = torch.full((b, hkv, ms, d), 0.75, device=dev)
    A.attn_decode_rope_append(0, torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev),
                              torch.from_numpy(cos_t).to(dev), torch.from_numpy(sin_t).to(dev),
                              kc, vc, 0, b, 0, hkv, d, ms, pos, 0, 0.125, None)
    torch.cuda.synchronize()
    kn, vn = kc.cpu().numpy(), vc.cpu().numpy()
    assert np.array_equal(vn[:, :, pos], vs)
    err = np.abs(kn[:, :, pos].astype(np.float64) - oracle.rope(ks, cos_t, sin_t))
    assert np.all(err <= _rope_row_bound(ks)), float(err.max())
    keep = np.arange(ms) != pos
    assert np.all(kn[:, :, keep] == -1.5) and np.all(vn[:, :, keep] == 0.75)


def test_decode_rope_append_full_decode_workload(dev):
    """The decode workload's shape (32 x 12 heads, 4096 positions) as a
    rotary decode step at position 4095."""
    w0 = synth.WORKLOADS["decode_b32_hq12_hkv2_d128_t4096"]
    case = (w0.batch, w0.num_heads, w0.kv_heads, w0.head_dim, w0.max_seq, 4095, 0)
    w, (q, k, v, kn), ref, got, kc, vc = _decode_rope_case(dev, case, seed=w0.seed)
    _check_rope_step(w, 4095, q, k, v, kn, ref, got, kc, vc, "rotary decode step")


# --------------------------------------------------------------- kv append

@pytest.mark.parametrize("b,hkv,d,ms,pos", [(1, 1, 32, 1, 0), (2, 2, 128, 16, 15),
                                            (3, 4, 64, 9, 4), (32, 2, 128, 4096, 4095),
                                            (2, 8, 256, 40, 0)])
def test_kv_append_bit_exact(dev, b, hkv, d, ms, pos):
    ks, vs = synth.append_inputs(b, hkv, d, seed=pos + d)
    kc = torch.full((b, hkv, ms, d), -7.25, device=dev)
    vc = torch.full((b, hkv, ms, d), 3.5, device=dev)
    A.kv_append(torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev), kc, vc,
                b, hkv, d, ms, pos)
    torch.cuda.synchronize()
    kn, vn = kc.cpu().numpy(), vc.cpu().numpy()
    kr = np.full_like(kn, -7.25)
    vr = np.full_like(vn, 3.5)
    oracle.kv_append(ks, vs, kr, vr, b, hkv, d, ms, pos)
    assert np.array_equal(kn, kr) and np.array_equal(vn, vr)


def test_kv_append_full_size_window_workload(dev):
    """Cache shape of the sliding-window workload (2 GiB per cache): the
    written row is exact and nothing else changed (checked on the GPU)."""
    b, hkv, d, ms, pos = 16, 8, 128, 32768, 32767
    ks, vs = synth.append_inputs(b, hkv, d, seed=12)
    kc = torch.full((b, hkv, ms, d), 1.25, device=dev)
    vc = torch.full((b, hkv, ms, d), -2.5, device=dev)
    A.kv_append(torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev), kc, vc,
                b, hkv, d, ms, pos)
    torch.cuda.synchronize()
    assert np.array_equal(kc[:, :, pos].cpu().numpy(), ks)
    assert np.array_equal(vc[:, :, pos].cpu().numpy(), vs)
    assert int((kc[:, :, :pos] != 1.25).sum()) == 0
    assert int((vc[:, :, :pos] != -2.5).sum()) == 0
    del kc, vc
    torch.cuda.empty_cache()


# ------------------------------------------------- bulk append (prefill rows)

ROWS_CASES = [
    # (m, kv_heads, head_dim, pad, max_seq, position)
    (1, 1, 32, 0, 1, 0),
    (17, 2, 32, 4, 40, 3),
    (65, 4, 64, 0, 65, 0),
    (300, 3, 128, 8, 512, 211),
    (129, 1, 256, 4, 130, 1),
    (2048, 4, 128, 0, 4096, 0),          # the Qwen-shaped prefill's K/V
    (33, 2, 96, 4, 40, 3),
    (70, 3, 224, 8, 80, 9),
]


@pytest.mark.parametrize("case", ROWS_CASES, ids=lambda c: "m{}_hkv{}_d{}_pad{}_ms{}_p{}".format(*c))
def test_kv_append_rows_bit_exact(dev, case):
    m, hkv, d, pad, ms, pos = case
    rng = np.random.default_rng(m + d)
    stride = hkv * d + pad
    k = rng.standard_normal((m, stride), dtype=np.float32)
    v = rng.standard_normal((m, stride), dtype=np.float32)
    kc = torch.full((hkv, ms, d), -7.5, device=dev)
    vc = torch.full((hkv, ms, d), 8.25, device=dev)
    A.kv_append_rows(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), kc, vc, m,
                     stride, hkv, d, ms, pos)
    torch.cuda.synchronize()
    kr = np.full((hkv, ms, d), -7.5, np.float32)
    vr = np.full((hkv, ms, d), 8.25, np.float32)
    oracle.kv_append_rows(k, v, kr, vr, m, stride, hkv, d, ms, pos)
    assert np.array_equal(kc.cpu().numpy(), kr) and np.array_equal(vc.cpu().numpy(), vr)


def test_kv_append_rows_long_prefill_shape(dev):
    """The long prefill's K/V (16384 rows, 8 KV heads of 128) into caches
    sized for 20000 rows; checked on the GPU against a gather of the source."""
    m, hkv, d, ms = 16384, 8, 128, 20000
    g = torch.Generator(device=dev).manual_seed(5)
    k = torch.randn((m, hkv * d), generator=g, device=dev)
    v = torch.randn((m, hkv * d), generator=g, device=dev)
    kc = torch.full((hkv, ms, d), 3.0, device=dev)
    vc = torch.full((hkv, ms, d), 4.0, device=dev)
    A.kv_append_rows(k, v, kc, vc, m, hkv * d, hkv, d, ms, 7)
    torch.cuda.synchronize()
    assert torch.equal(kc[:, 7:7 + m], k.view(m, hkv, d).permute(1, 0, 2))
    assert torch.equal(vc[:, 7:7 + m], v.view(m, hkv, d).permute(1, 0, 2))
    assert bool((kc[:, :7] == 3.0).all()) and bool((kc[:, 7 + m:] == 3.0).all())
    assert bool((vc[:, :7] == 4.0).all()) and bool((vc[:, 7 + m:] == 4.0).all())


def test_prefill_then_append_rows_then_decode(dev):
    """GPU prefill over a fused QKV buffer, its K/V rows appended to a cache,
    then GPU decode of Q row i over the first i+1 rows equals prefill row i."""
    m, hq, hpk, d = 300, 12, 6, 128
    hkv = hq // hpk
    stride = (hq + 2 * hkv) * d
    rng = np.random.default_rng(11)
    qkv = rng.standard_normal((m, stride), dtype=np.float32)
    buf = torch.from_numpy(qkv).to(dev)
    q, k, v = buf[:, :hq * d], buf[:, hq * d:(hq + hkv) * d], buf[:, (hq + hkv) * d:]
    o = torch.full((m, stride), float("nan"), device=dev)
    A.attn_prefill_causal(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), m, stride,
                          stride, hq, hpk, d)
    ms = 320
    kc = torch.full((1, hkv, ms, d), float("nan"), device=dev)
    vc = torch.full((1, hkv, ms, d), float("nan"), device=dev)
    A.kv_append_rows(k.data_ptr(), v.data_ptr(), kc, vc, m, stride, hkv, d, ms, 0)
    scale = 1.0 / np.sqrt(np.float32(d))
    for i in (0, 63, 64, m - 1):
        qi = q[i].reshape(1, hq, d).contiguous()
        out = torch.full((1, hq, d), float("nan"), device=dev)
        ws = A.decode_workspace(1, hq, hkv, d, i + 1, 0)
        A.attn_decode(qi, kc, vc, out, 1, hq, hkv, d, ms, i + 1, 0, float(scale), ws)
        torch.cuda.synchronize()
        ref = oracle.prefill_causal(qkv[:, :hq * d].copy(), qkv[:, hq * d:(hq + hkv) * d].copy(),
                                    qkv[:, (hq + hkv) * d:].copy(), m, hq * d, hkv * d, hq, hpk,
                                    d, rows=np.full(hq, i, np.uint32),
                                    heads=np.arange(hq, dtype=np.uint32))
        vmax = float(np.abs(qkv[:i + 1, (hq + hkv) * d:]).max())
        got_p = o[i, :hq * d].cpu().numpy().reshape(hq, d)
        got_d = out[0].cpu().numpy()
        _assert_close(got_p, ref.reshape(hq, d), vmax, f"prefill row {i}")
        _assert_close(got_d, ref.reshape(hq, d), vmax, f"decode row {i}")


# -------------------------------------------------------------- varlen decode

VARLEN_CASES = [
    # (batch, hq, hkv, d, max_seq, bound, window, idle)
    (6, 12, 2, 128, 300, 300, 0, 1),
    (5, 8, 8, 64, 100, 77, 9, 1),        # MHA, window below most lengths
    (7, 4, 2, 32, 50, 50, 0, 2),
    (3, 16, 2, 256, 700, 650, 100, 0),
    (64, 8, 4, 128, 200, 200, 0, 3),     # many units: single-split plan (direct)
    (2, 9, 1, 128, 3000, 3000, 0, 0),    # two head chunks
    (32, 12, 2, 128, 4096, 4096, 0, 2),  # the decode workload's shape, mixed lengths
    (4, 8, 2, 160, 300, 300, 0, 1),
]


def _varlen_inputs(case, seed):
    b, hq, hkv, d, ms, bound, win, idle = case
    w = synth.DecodeWorkload("varlen", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=ms, total_seq=bound, window=win, seed=seed)
    q, k, v = synth.decode_inputs(w)
    lens = synth.seq_lengths(b, bound, seed=seed + 7, idle=idle)
    return w, q, k, v, lens


def _vmax_varlen(w, v, lens, plus=0):
    vm = 0.0
    for i, t in enumerate(lens):
        t = int(t) + plus
        if t:
            lo = t - w.window if (w.window and t > w.window) else 0
            vm = max(vm, float(np.abs(v[i, :, lo:t]).max()))
    return vm


@pytest.mark.parametrize("case", VARLEN_CASES,
                         ids=lambda c: "b{}_hq{}_hkv{}_d{}_ms{}_bd{}_w{}_idle{}".format(*c))
def test_decode_varlen_matches_oracle(dev, case):
    w, q, k, v, lens = _varlen_inputs(case, seed=sum(case) % 883)
    b, hq, hkv, d, ms, bound, win, _ = case
    out = torch.full((b, hq, d), float("nan"), device=dev)
    ws = _poisoned_ws(A.attn_decode_workspace_bytes(b, hq, hkv, d, bound, win), b, hq, dev)
    A.attn_decode_varlen(torch.from_numpy(q).to(dev), torch.from_numpy(k).to(dev),
                         torch.from_numpy(v).to(dev), out,
                         torch.from_numpy(lens.astype(np.int32)).to(dev), b, hq, hkv, d, ms,
                         bound, win, w.scale, ws)
    torch.cuda.synchronize()
    ref = oracle.decode_varlen(q, k, v, lens, b, hq, hkv, d, ms, win, w.scale)
    got = out.cpu().numpy()
    assert np.all(got[lens == 0] == 0.0)
    _assert_close(got, ref, _vmax_varlen(w, v, lens), str(case))


def test_decode_varlen_invalid_length_gives_nan_rows(dev):
    """A length past seq_bound yields NaN for that sequence only."""
    b, hq, hkv, d, ms, bound = 4, 12, 2, 128, 64, 40
    w = synth.DecodeWorkload("varlen", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=ms, total_seq=bound, seed=21)
    q, k, v = synth.decode_inputs(w)
    lens = np.array([40, 41, 0, 17], np.uint32)
    out = torch.zeros((b, hq, d), device=dev)
    ws = A.decode_workspace(b, hq, hkv, d, bound, 0)
    A.attn_decode_varlen(torch.from_numpy(q).to(dev), torch.from_numpy(k).to(dev),
                         torch.from_numpy(v).to(dev), out,
                         torch.from_numpy(lens.astype(np.int32)).to(dev), b, hq, hkv, d, ms,
                         bound, 0, w.scale, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isnan(got[1])) and np.all(got[2] == 0.0)
    ok = lens.copy()
    ok[1] = 0
    ref = oracle.decode_varlen(q, k, v, ok, b, hq, hkv, d, ms, 0, w.scale)
    _assert_close(got[[0, 3]], ref[[0, 3]], _vmax_varlen(w, v, ok), "valid rows")


VARLEN_APPEND_CASES = [
    # (batch, hq, hkv, d, max_seq, bound, window)
    (6, 12, 2, 128, 300, 300, 0),
    (5, 4, 2, 64, 90, 90, 17),
    (4, 8, 8, 32, 40, 1, 0),             # bound 1: every sequence at position 0
    (64, 8, 4, 128, 200, 160, 0),
    (32, 12, 2, 128, 4096, 4096, 0),
    (20, 4, 2, 32, 64, 64, 0),           # 40 units: more than one 32-lane merge wave's table
] + [(b, hq, hkv, d, ms, pos + 1, win) for (b, hq, hkv, d, ms, pos, win) in _random_step_shapes(12, 16192)]


@pytest.mark.parametrize("case", VARLEN_APPEND_CASES,
                         ids=lambda c: "b{}_hq{}_hkv{}_d{}_ms{}_bd{}_w{}".format(*c))
def test_decode_append_varlen_matches_oracle(dev, case):
    b, hq, hkv, d, ms, bound, win = case
    seed = sum(case) % 877
    w = synth.DecodeWorkload("varlen", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=ms, total_seq=bound, window=win, seed=seed)
    q, k, v = synth.decode_inputs(w)
    kn, vn = synth.append_inputs(b, hkv, d, seed=seed + 1)
    pos = synth.seq_lengths(b, bound, seed=seed + 2) - 1        # positions in [0, bound)
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    out = torch.full((b, hq, d), float("nan"), device=dev)
    nws = A.attn_decode_workspace_bytes(b, hq, hkv, d, bound, win)
    ws = _poisoned_ws(nws, b, hq, dev)
    A.attn_decode_append_varlen(torch.from_numpy(q).to(dev), torch.from_numpy(kn).to(dev),
                                torch.from_numpy(vn).to(dev), kd, vd, out,
                                torch.from_numpy(pos.astype(np.int32)).to(dev), b, hq, hkv, d,
                                ms, bound, win, w.scale, ws)
    torch.cuda.synchronize()
    for i in range(b):   # the reference step: each sequence appends at its position
        oracle.kv_append(kn[i:i + 1], vn[i:i + 1], k[i:i + 1], v[i:i + 1], 1, hkv, d, ms,
                         int(pos[i]))
    assert np.array_equal(kd.cpu().numpy(), k) and np.array_equal(vd.cpu().numpy(), v)
    ref = oracle.decode_varlen(q, k, v, pos + 1, b, hq, hkv, d, ms, win, w.scale)
    _assert_close(out.cpu().numpy(), ref, _vmax_varlen(w, v, pos, plus=1), str(case))


def test_decode_append_varlen_invalid_position_and_no_heads(dev):
    """positions[b] + 1 > seq_bound: NaN output, no write for that sequence;
    num_heads == 0: the per-sequence appends alone."""
    b, hq, hkv, d, ms, bound = 3, 6, 2, 64, 32, 20
    w = synth.DecodeWorkload("varlen", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=ms, total_seq=bound, seed=23)
    q, k, v = synth.decode_inputs(w)
    kn, vn = synth.append_inputs(b, hkv, d, seed=24)
    pos = np.array([19, 20, 4], np.uint32)
    for heads in (hq, 0):
        kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
        out = torch.zeros((b, max(heads, 1), d), device=dev)
        ws = A.decode_workspace(b, hq, hkv, d, bound, 0)
        A.attn_decode_append_varlen(torch.from_numpy(q).to(dev) if heads else 0,
                                    torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev),
                                    kd, vd, out if heads else 0,
                                    torch.from_numpy(pos.astype(np.int32)).to(dev), b, heads,
                                    hkv, d, ms, bound, 0, w.scale, ws if heads else None)
        torch.cuda.synchronize()
        kr, vr = k.copy(), v.copy()
        for i in (0, 2):
            oracle.kv_append(kn[i:i + 1], vn[i:i + 1], kr[i:i + 1], vr[i:i + 1], 1, hkv, d, ms,
                             int(pos[i]))
        assert np.array_equal(kd.cpu().numpy(), kr) and np.array_equal(vd.cpu().numpy(), vr)
        if heads:
            got = out.cpu().numpy()
            assert np.all(np.isnan(got[1]))
            ref = oracle.decode_varlen(q, kr, vr, np.where(pos < bound, pos + 1, 0), b, hq, hkv,
                                       d, ms, 0, w.scale)
            _assert_close(got[[0, 2]], ref[[0, 2]], _vmax_varlen(w, vr, pos[[0, 2]], plus=1),
                          "valid rows")


@pytest.mark.parametrize("rope", [False, True], ids=["plain", "rope"])
def test_decode_append_varlen_units_without_rows(dev, rope):
    """More than 64 units (the table is scanned in 64-lane chunks), some with
    no row before the new one (position 0: the output is the new V row) and
    one with an invalid position (NaN, no cache write): those units get the
    grid's spare workgroups, which merge over an empty range."""
    b, hq, hkv, d, ms, bound, win = 40, 8, 2, 64, 500, 500, 0   # 80 units
    w = synth.DecodeWorkload("varlen", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=ms, total_seq=bound, window=win, seed=41)
    q, k, v = synth.decode_inputs(w)
    kn, vn = synth.append_inputs(b, hkv, d, seed=42)
    pos = (synth.seq_lengths(b, bound, seed=43) - 1).astype(np.uint32)
    pos[[3, 17, 30, 39]] = 0
    pos[5] = bound                                              # invalid: T_b > seq_bound
    valid = np.flatnonzero(pos < bound)
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    out = torch.full((b, hq, d), float("nan"), device=dev)
    ws = _poisoned_ws(A.attn_decode_workspace_bytes(b, hq, hkv, d, bound, win), b, hq, dev)
    posd = torch.from_numpy(pos.astype(np.int32)).to(dev)
    kr, vr = k.copy(), v.copy()
    vmax_pos = np.where(pos < bound, pos.astype(np.int64), -1)    # the invalid one skipped
    if rope:
        tabs = [synth.rope_tables(d, int(p) % bound) for p in pos]
        cos_t = np.ascontiguousarray(np.stack([t[0] for t in tabs]))
        sin_t = np.ascontiguousarray(np.stack([t[1] for t in tabs]))
        A.attn_decode_rope_append_varlen(
            torch.from_numpy(q).to(dev), torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev),
            torch.from_numpy(cos_t).to(dev), torch.from_numpy(sin_t).to(dev), kd, vd, out, posd,
            b, hq, hkv, d, ms, bound, win, w.scale, ws)
        torch.cuda.synchronize()
        ref = np.zeros((b, hq, d))
        for i in valid:   # the oracle's fused step, sequence by sequence (updates kr, vr)
            ref[i] = oracle.decode_rope_append(q[i:i + 1], kn[i:i + 1], vn[i:i + 1], cos_t[i],
                                               sin_t[i], kr[i:i + 1], vr[i:i + 1], 1, hq, hkv,
                                               d, ms, int(pos[i]), win, w.scale)[0]
        kc, vc = kd.cpu().numpy(), vd.cpu().numpy()
        assert np.array_equal(vc, vr)
        for i in range(b):
            keep = np.arange(ms) != pos[i] if i in valid else np.ones(ms, bool)
            assert np.array_equal(kc[i][:, keep], k[i][:, keep])
            if i in valid:
                err = np.abs(kc[i, :, pos[i]].astype(np.float64) - kr[i, :, pos[i]])
                assert np.all(err <= _rope_row_bound(kn[i])), (i, float(err.max()))
        _assert_close(out.cpu().numpy()[valid], ref[valid], _vmax_varlen(w, vr, vmax_pos, plus=1),
                      "valid sequences")
    else:
        A.attn_decode_append_varlen(torch.from_numpy(q).to(dev), torch.from_numpy(kn).to(dev),
                                    torch.from_numpy(vn).to(dev), kd, vd, out, posd, b, hq, hkv,
                                    d, ms, bound, win, w.scale, ws)
        torch.cuda.synchronize()
        for i in valid:
            oracle.kv_append(kn[i:i + 1], vn[i:i + 1], kr[i:i + 1], vr[i:i + 1], 1, hkv, d, ms,
                             int(pos[i]))
        assert np.array_equal(kd.cpu().numpy(), kr) and np.array_equal(vd.cpu().numpy(), vr)
        ref = oracle.decode_varlen(q, kr, vr, np.where(pos < bound, pos + 1, 0), b, hq, hkv,
                                   d, ms, win, w.scale)
        _assert_close(out.cpu().numpy()[valid], ref[valid], _vmax_varlen(w, vr, vmax_pos, plus=1),
                      "valid sequences")
        for i in (3, 17, 30, 39):   # only the new row: its V row, exactly
            want = np.repeat(vn[i], hq // hkv, axis=0)
            assert np.array_equal(out.cpu().numpy()[i], want), f"sequence {i}"
    assert np.all(np.isnan(out.cpu().numpy()[5]))


def test_decode_steps_deterministic_whichever_workgroup_merges(dev):
    """The last workgroup of a unit to finish merges it, and which one that is
    changes from call to call; the fold runs in split order all the same, so
    repeated calls give the same bits: the decode step (many splits per unit)
    and the varlen step, eight calls each on one workspace."""
    b, hq, hkv, d, ms = 3, 12, 2, 128, 3000           # 6 units, 43 splits each
    w, (q, k, v) = _decode_case(b, hq, hkv, d, ms, ms, seed=51)
    kn, vn = synth.append_inputs(b, hkv, d, seed=52)
    qd, knd, vnd = (torch.from_numpy(x).to(dev) for x in (q, kn, vn))
    ws = A.decode_workspace(b, hq, hkv, d, ms, 0, device=dev)
    pos = torch.from_numpy((synth.seq_lengths(b, ms, seed=53) - 1).astype(np.int32)).to(dev)
    for varlen in (False, True):
        outs = []
        for _ in range(8):
            kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
            out = torch.empty(b, hq, d, device=dev)
            if varlen:
                A.attn_decode_append_varlen(qd, knd, vnd, kd, vd, out, pos, b, hq, hkv, d, ms, ms,
                                            0, w.scale, ws)
            else:
                A.attn_decode_append(qd, knd, vnd, kd, vd, out, b, hq, hkv, d, ms, ms - 1, 0,
                                     w.scale, ws)
            outs.append(out)
        torch.cuda.synchronize()
        for o in outs[1:]:
            assert torch.equal(o, outs[0]), "varlen" if varlen else "uniform"


# ----------------------------------------------------------------- prefill

def _gpu_prefill(dev, w, q, k, v, fill=float("nan")):
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o = torch.full((w.m, w.q_stride), fill, device=dev)
    A.attn_prefill_causal(qd, kd, vd, o, w.m, w.q_stride, w.kv_stride, w.num_q_heads,
                          w.heads_per_kv, w.head_dim)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def _heads(w, o):
    return o[:, : w.num_q_heads * w.head_dim].reshape(w.m, w.num_q_heads, w.head_dim)


def _ref_prefill(w, q, k, v, **kw):
    return oracle.prefill_causal(q, k, v, w.m, w.q_stride, w.kv_stride, w.num_q_heads,
                                 w.heads_per_kv, w.head_dim, **kw)


def _vmax_prefill(w, v):
    return float(np.abs(v[:, : w.kv_heads * w.head_dim]).max())


@pytest.mark.parametrize("name", ["prefill_hq4_hkv2_d32_m16", "prefill_hq28_hkv4_d128_m2048"])
def test_prefill_full_workloads(dev, name):
    w = synth.WORKLOADS[name]
    q, k, v = synth.prefill_inputs(w)
    o = _gpu_prefill(dev, w, q, k, v)
    _assert_close(_heads(w, o), _ref_prefill(w, q, k, v), _vmax_prefill(w, v), name)


def test_prefill_long_workload_sampled(dev):
    """Long prefill (M=16384, 64 Q / 8 KV heads, d=128) at full size. Sample:
    every row of head 0 and head 63 (first and last KV group), the last 64
    rows of every head, and 1024 seeded random (row, head) pairs."""
    w = synth.WORKLOADS["prefill_hq64_hkv8_d128_m16384"]
    q, k, v = synth.prefill_inputs(w)
    o = _heads(w, _gpu_prefill(dev, w, q, k, v))
    rng = np.random.default_rng(2024)
    rows = [np.arange(w.m), np.arange(w.m)]
    heads = [np.zeros(w.m, np.int64), np.full(w.m, 63)]
    last = np.arange(w.m - 64, w.m)
    for h in range(w.num_q_heads):
        rows.append(last)
        heads.append(np.full(64, h))
    rows.append(rng.integers(0, w.m, 1024))
    heads.append(rng.integers(0, w.num_q_heads, 1024))
    rows = np.concatenate(rows)
    heads = np.concatenate(heads)
    ref = _ref_prefill(w, q, k, v, rows=rows, heads=heads)
    _assert_close(o[rows, heads], ref, _vmax_prefill(w, v), "long prefill sample")


def test_prefill_row_block_major_path_ragged(dev):
    """A grid of two or more workgroups per CU (here 1032) takes the
    row-block-major work map; m = 4100 leaves a ragged last row block.
    Sample: the last 40 rows of every head plus 1500 seeded random pairs."""
    w = synth.PrefillWorkload("case", m=4100, num_q_heads=64, heads_per_kv=8, head_dim=128,
                              q_stride=64 * 128, kv_stride=8 * 128, seed=4100)
    q, k, v = synth.prefill_inputs(w)
    o = _heads(w, _gpu_prefill(dev, w, q, k, v))
    rng = np.random.default_rng(4101)
    rows = [np.repeat(np.arange(w.m - 40, w.m), 64), rng.integers(0, w.m, 1500)]
    heads = [np.tile(np.arange(64), 40), rng.integers(0, 64, 1500)]
    rows, heads = np.concatenate(rows), np.concatenate(heads)
    ref = _ref_prefill(w, q, k, v, rows=rows, heads=heads)
    _assert_close(o[rows, heads], ref, _vmax_prefill(w, v), "row-block-major ragged")


@pytest.mark.parametrize("d,m", [(192, 2040), (256, 2048)])
def test_prefill_large_head_dim_four_wave_path(dev, d, m):
    """head_dim >= 192 on a grid that fills the chip twice runs 4-wave
    workgroups (one wave per SIMD); ragged last row block for d = 192.
    Sample: the last 24 rows of every head plus 600 seeded random pairs."""
    w = synth.PrefillWorkload("case", m=m, num_q_heads=32, heads_per_kv=4, head_dim=d,
                              q_stride=32 * d, kv_stride=8 * d, seed=d + m)
    q, k, v = synth.prefill_inputs(w)
    o = _heads(w, _gpu_prefill(dev, w, q, k, v))
    rng = np.random.default_rng(d)
    rows = [np.repeat(np.arange(w.m - 24, w.m), 32), rng.integers(0, w.m, 600)]
    heads = [np.tile(np.arange(32), 24), rng.integers(0, 32, 600)]
    rows, heads = np.concatenate(rows), np.concatenate(heads)
    ref = _ref_prefill(w, q, k, v, rows=rows, heads=heads)
    _assert_close(o[rows, heads], ref, _vmax_prefill(w, v), f"d {d} m {m}")


PREFILL_SWEEP = [
    # (m, hq, hpk, d)
    (1, 1, 1, 32), (2, 2, 1, 64), (15, 4, 2, 32), (16, 4, 2, 32), (17, 4, 2, 32),
    (31, 6, 6, 128), (32, 6, 6, 128), (33, 6, 6, 128), (63, 8, 8, 128),
    (64, 8, 8, 128), (65, 8, 8, 128), (127, 7, 7, 128), (128, 12, 6, 64),
    (129, 12, 3, 64), (300, 5, 5, 128), (257, 6, 2, 128), (1000, 8, 4, 128),
    (200, 3, 1, 256), (100, 16, 8, 256), (450, 10, 5, 32), (97, 9, 9, 64),
    (1000, 28, 7, 128),
    (200, 6, 3, 96), (64, 2, 1, 96), (129, 4, 2, 160), (300, 8, 4, 192), (97, 6, 6, 224),
    # 16-row blocks at head_dim 192 / 256: an odd count of 16-row blocks (the
    # middle one alone), ragged ends, workgroups whose tasks span two pairs
    (33, 2, 2, 256), (17, 3, 3, 192), (1000, 8, 4, 192), (1024, 16, 2, 256), (495, 14, 7, 192),
    # up to 16 rows: one wave per Q head, every built head size, head counts
    # that leave the last 4-wave workgroup part empty
    (16, 8, 4, 128), (5, 3, 3, 256), (1, 2, 2, 96), (16, 16, 8, 160), (9, 7, 7, 224),
    (12, 6, 2, 192), (3, 64, 8, 64), (16, 28, 7, 128), (7, 5, 1, 32),
]


@pytest.mark.parametrize("case", PREFILL_SWEEP, ids=lambda c: "m{}_hq{}_hpk{}_d{}".format(*c))
def test_prefill_sweep(dev, case):
    m, hq, hpk, d = case
    w = synth.PrefillWorkload("case", m=m, num_q_heads=hq, heads_per_kv=hpk, head_dim=d,
                              q_stride=hq * d, kv_stride=(hq // hpk) * d, seed=m + d)
    q, k, v = synth.prefill_inputs(w)
    o = _gpu_prefill(dev, w, q, k, v)
    _assert_close(_heads(w, o), _ref_prefill(w, q, k, v), _vmax_prefill(w, v), str(case))


def _random_prefill_shapes(n, seed):
    """Seeded shapes across the built head sizes, GQA ratios, prompt lengths on
    both sides of the small-prompt limit, and row strides with padding."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([32, 64, 96, 128, 160, 192, 224, 256]))
        hkv = int(rng.integers(1, 4))
        hpk = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8]))
        m = int(rng.integers(1, 17)) if rng.random() < 0.3 else int(rng.integers(17, 300))
        out.append((m, hkv * hpk, hpk, d, 4 * int(rng.integers(0, 3)), 4 * int(rng.integers(0, 3))))
    return out


PREFILL_RANDOM = _random_prefill_shapes(24, 2024)


@pytest.mark.parametrize("case", PREFILL_RANDOM,
                         ids=lambda c: "m{}_hq{}_hpk{}_d{}_qpad{}_kvpad{}".format(*c))
def test_prefill_random_shapes(dev, case):
    m, hq, hpk, d, qpad, kvpad = case
    w = synth.PrefillWorkload("rand", m=m, num_q_heads=hq, heads_per_kv=hpk, head_dim=d,
                              q_stride=hq * d + qpad, kv_stride=(hq // hpk) * d + kvpad,
                              seed=m * 31 + hq * 7 + d)
    q, k, v = synth.prefill_inputs(w)
    o = _gpu_prefill(dev, w, q, k, v)
    _assert_close(_heads(w, o), _ref_prefill(w, q, k, v), _vmax_prefill(w, v), str(case))
    assert np.isnan(o[:, hq * d:]).all(), "padding columns of O were written"


def test_prefill_fused_qkv_buffer(dev):
    """Q, K, V as column slices of one [m, (Hq + 2 Hkv) d] projection output,
    O written into its own buffer with the same stride; columns outside the
    Q heads of O stay untouched."""
    m, hq, hkv, d = 333, 12, 2, 128
    stride = (hq + 2 * hkv) * d
    x = synth.normal(np.random.default_rng(77), (m, stride), 1.0)
    xd = torch.from_numpy(x).to(dev)
    o = torch.full((m, stride), 9.0, device=dev)
    base = xd.data_ptr()
    A.attn_prefill_causal(base, base + 4 * hq * d, base + 4 * (hq + hkv) * d, o, m,
                          stride, stride, hq, hq // hkv, d)
    torch.cuda.synchronize()
    on = o.cpu().numpy()
    flat = x.reshape(-1)
    ref = oracle.prefill_causal(x, flat[hq * d:], flat[(hq + hkv) * d:], m, stride, stride,
                                hq, hq // hkv, d)
    vmax = float(np.abs(x[:, (hq + hkv) * d:]).max())
    _assert_close(on[:, : hq * d].reshape(m, hq, d), ref, vmax, "fused qkv")
    assert np.all(on[:, hq * d:] == 9.0)


def test_prefill_row0_and_determinism(dev):
    w = synth.PrefillWorkload("case", m=200, num_q_heads=8, heads_per_kv=4, head_dim=128,
                              q_stride=8 * 128 + 64, kv_stride=2 * 128 + 32, seed=3)
    q, k, v = synth.prefill_inputs(w)
    a = _gpu_prefill(dev, w, q, k, v)
    b = _gpu_prefill(dev, w, q, k, v)
    assert np.array_equal(a[:, : 8 * 128], b[:, : 8 * 128])
    ha = _heads(w, a)
    for h in range(8):
        g = h // 4
        np.testing.assert_allclose(ha[0, h], v[0, g * 128:(g + 1) * 128], rtol=0, atol=1e-6)
    assert np.all(np.isnan(a[:, 8 * 128:]))  # padding columns of O untouched


def test_prefill_zero_rows_is_a_no_op(dev):
    o = torch.full((4, 128), 5.0, device=dev)
    z = torch.empty(0, device=dev)
    A.attn_prefill_causal(z, z, z, z, 0, 128, 64, 4, 2, 32)
    torch.cuda.synchronize()
    assert torch.all(o == 5.0)


def test_cross_mode_prefill_rows_equal_decode(dev):
    """Append prefill's K/V rows one by one with kv_append, decode with
    total_seq = i + 1 at prefill's scale: equals prefill row i (both on GPU,
    both against the oracle's prefill)."""
    m, hq, hpk, d = 150, 12, 6, 128
    hkv = hq // hpk
    w = synth.PrefillWorkload("case", m=m, num_q_heads=hq, heads_per_kv=hpk, head_dim=d,
                              q_stride=hq * d, kv_stride=hkv * d, seed=21)
    q, k, v = synth.prefill_inputs(w)
    o = _heads(w, _gpu_prefill(dev, w, q, k, v))
    ref = _ref_prefill(w, q, k, v)
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    kc = torch.zeros(1, hkv, m, d, device=dev)
    vc = torch.zeros(1, hkv, m, d, device=dev)
    for i in range(m):
        A.kv_append(kd[i], vd[i], kc, vc, 1, hkv, d, m, i)
    scale = oracle.prefill_scale(d)
    ws = A.decode_workspace(1, hq, hkv, d, m, 0, device=dev)
    vmax = _vmax_prefill(w, v)
    for i in (0, 1, 63, 64, 149):
        out = torch.empty(1, hq, d, device=dev)
        qi = torch.from_numpy(np.ascontiguousarray(q[i].reshape(1, hq, d))).to(dev)
        A.attn_decode(qi, kc, vc, out, 1, hq, hkv, d, m, i + 1, 0, scale, ws)
        torch.cuda.synchronize()
        _assert_close(out.cpu().numpy()[0], ref[i], vmax, f"decode row {i}")
        _assert_close(o[i], ref[i], vmax, f"prefill row {i}")


def test_decode_calls_replay_correctly_from_a_hip_graph(dev):
    """attn_decode_append and attn_decode captured in a HIP graph: every
    replay, with eager work and synchronisations between replays, gives the
    same bits as the eager call (the kernels are deterministic)."""
    b, hq, hkv, d, ms, pos = 4, 12, 2, 128, 1500, 1300
    w, (q, k, v) = _decode_case(b, hq, hkv, d, ms, pos + 1, seed=31)
    kn, vn = synth.append_inputs(b, hkv, d, seed=32)
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    knd, vnd = torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev)
    ws = A.decode_workspace(b, hq, hkv, d, pos + 1, 0, device=dev)
    out_e = torch.empty(b, hq, d, device=dev)
    out_g = torch.empty(b, hq, d, device=dev)
    out2_e = torch.empty(b, hq, d, device=dev)
    out2_g = torch.empty(b, hq, d, device=dev)
    A.attn_decode_append(qd, knd, vnd, kd, vd, out_e, b, hq, hkv, d, ms, pos, 0, w.scale, ws)
    A.attn_decode(qd, kd, vd, out2_e, b, hq, hkv, d, ms, pos + 1, 0, w.scale, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.attn_decode_append(qd, knd, vnd, kd, vd, out_g, b, hq, hkv, d, ms, pos, 0, w.scale, ws)
        A.attn_decode(qd, kd, vd, out2_g, b, hq, hkv, d, ms, pos + 1, 0, w.scale, ws)
    for rep in range(4):
        out_g.fill_(float("nan"))
        out2_g.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=dev).sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}: attn_decode_append differs"
        assert torch.equal(out2_g, out2_e), f"replay {rep}: attn_decode differs"
        assert bool(torch.isfinite(junk))
    oracle.kv_append(kn, vn, k, v, b, hkv, d, ms, pos)
    _assert_close(out_e.cpu().numpy(), _ref_decode(w.with_(total_seq=pos + 1), q, k, v),
                  _vmax_decode(w, v), "graph case eager")


def test_varlen_decode_step_graph_follows_device_positions(dev):
    """A decode step of a mixed-length batch captured once in a HIP graph
    serves new positions and new rows on every replay: the positions live in
    device memory and are rewritten between replays (with other eager work),
    and each replay matches the oracle's append + decode at those positions."""
    b, hq, hkv, d, ms = 3, 12, 2, 128, 600
    w, (q, k, v) = _decode_case(b, hq, hkv, d, ms, ms, seed=41)
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    knd = torch.empty(b, hkv, d, device=dev)
    vnd = torch.empty(b, hkv, d, device=dev)
    pos_d = torch.zeros(b, dtype=torch.int32, device=dev)
    out = torch.empty(b, hq, d, device=dev)
    ws = A.decode_workspace(b, hq, hkv, d, ms, 0, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.attn_decode_append_varlen(qd, knd, vnd, kd, vd, out, pos_d, b, hq, hkv, d, ms, ms, 0,
                                    w.scale, ws)
    kr, vr = k.copy(), v.copy()   # host mirror of the caches
    for rep, pos in enumerate([[100, 5, 599], [101, 0, 300], [37, 6, 598]]):
        pos = np.array(pos, np.uint32)
        kn, vn = synth.append_inputs(b, hkv, d, seed=50 + rep)
        knd.copy_(torch.from_numpy(kn))
        vnd.copy_(torch.from_numpy(vn))
        pos_d.copy_(torch.from_numpy(pos.astype(np.int32)))
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=dev).sum()
        g.replay()
        torch.cuda.synchronize()
        for i in range(b):
            oracle.kv_append(kn[i:i + 1], vn[i:i + 1], kr[i:i + 1], vr[i:i + 1], 1, hkv, d, ms,
                             int(pos[i]))
        assert np.array_equal(kd.cpu().numpy(), kr) and np.array_equal(vd.cpu().numpy(), vr)
        ref = oracle.decode_varlen(q, kr, vr, pos + 1, b, hq, hkv, d, ms, 0, w.scale)
        vmax = max(float(np.abs(vr[i, :, :pos[i] + 1]).max()) for i in range(b))
        _assert_close(out.cpu().numpy(), ref, vmax, f"replay {rep}")
        assert bool(torch.isfinite(junk))


def test_serving_calls_replay_from_a_hip_graph(dev):
    """Prefill, bulk append and the rotary decode step captured in one HIP
    graph: every replay gives the eager results bit for bit."""
    m, hq, hpk, d, ms = 200, 12, 6, 128, 256
    hkv = hq // hpk
    w = synth.PrefillWorkload("g", m=m, num_q_heads=hq, heads_per_kv=hpk, head_dim=d,
                              q_stride=hq * d, kv_stride=hkv * d, seed=61)
    q, k, v = (torch.from_numpy(x).to(dev) for x in synth.prefill_inputs(w))
    qn = torch.randn(1, hq, d, device=dev)
    kn = torch.randn(1, hkv, d, device=dev)
    vn = torch.randn(1, hkv, d, device=dev)
    cos_t, sin_t = (torch.from_numpy(x).to(dev) for x in synth.rope_tables(d, m))
    ws = A.decode_workspace(1, hq, hkv, d, m + 1, 0, device=dev)

    def run(o, kc, vc, out):
        A.attn_prefill_causal(q, k, v, o, m, hq * d, hkv * d, hq, hpk, d)
        A.kv_append_rows(k, v, kc, vc, m, hkv * d, hkv, d, ms, 0)
        A.attn_decode_rope_append(qn, kn, vn, cos_t, sin_t, kc, vc, out, 1, hq, hkv, d, ms, m,
                                  0, 0.08838835, ws)

    def fresh():
        return (torch.full((m, hq * d), float("nan"), device=dev),
                torch.full((1, hkv, ms, d), float("nan"), device=dev),
                torch.full((1, hkv, ms, d), float("nan"), device=dev),
                torch.full((1, hq, d), float("nan"), device=dev))
    eager = fresh()
    run(*eager)
    torch.cuda.synchronize()
    graph_bufs = fresh()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(*graph_bufs)
    for rep in range(3):
        for t in graph_bufs:
            t.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=dev).sum()
        g.replay()
        torch.cuda.synchronize()
        for a_, b_ in zip(eager[:1] + eager[3:], graph_bufs[:1] + graph_bufs[3:]):
            assert torch.equal(a_, b_), f"replay {rep}"
        # cache rows 0..m are written (m by the decode step); the rest stay NaN
        for a_, b_ in zip(eager[1:3], graph_bufs[1:3]):
            assert torch.equal(a_[:, :, :m + 1], b_[:, :, :m + 1]), f"replay {rep}"
            assert bool(torch.isnan(b_[:, :, m + 1:]).all())
        assert bool(torch.isfinite(junk))
    assert bool(torch.isfinite(eager[3]).all())


# ------------------------------------------------------------- large offsets

def test_decode_one_sequence_of_a_million_rows(dev):
    """One sequence with 2^20 cached rows and 8 KV heads: 4 GiB per cache, so
    byte offsets pass 2^32 (the caches are drawn on the GPU and copied back
    for the oracle)."""
    w = synth.DecodeWorkload("long", batch=1, num_heads=16, kv_heads=8, head_dim=128,
                             max_seq=1 << 20, total_seq=1 << 20, seed=77)
    q, k, v = synth.decode_inputs_device(w, 77, dev)
    out = torch.full((1, 16, 128), float("nan"), device=dev)
    ws = A.decode_workspace(1, 16, 8, 128, w.total_seq, 0, device=dev)
    A.attn_decode(q, k, v, out, 1, 16, 8, 128, w.max_seq, w.total_seq, 0, w.scale, ws)
    torch.cuda.synchronize()
    qn, kn, vn = q.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy()
    del k, v
    torch.cuda.empty_cache()
    ref = oracle.decode(qn, kn, vn, 1, 16, 8, 128, w.max_seq, w.total_seq, 0, w.scale)
    _assert_close(out.cpu().numpy(), ref, float(np.abs(vn).max()), "2^20 rows")


def test_prefill_past_two_gib_of_q(dev):
    """m = 65536 rows of 64 query heads (Q and O 2 GiB each): byte offsets of
    late rows pass 2^31. Sample: the last row of every head plus 256 seeded
    (row, head) pairs from the second half."""
    w = synth.PrefillWorkload("big", m=65536, num_q_heads=64, heads_per_kv=8, head_dim=128,
                              q_stride=64 * 128, kv_stride=8 * 128, seed=65)
    q, k, v = synth.prefill_inputs_device(w, 65, dev)
    o = torch.full((w.m, w.q_stride), float("nan"), device=dev)
    A.attn_prefill_causal(q, k, v, o, w.m, w.q_stride, w.kv_stride, 64, 8, 128)
    torch.cuda.synchronize()
    rng = np.random.default_rng(66)
    rows = np.concatenate([np.full(64, w.m - 1), rng.integers(w.m // 2, w.m, 256)])
    heads = np.concatenate([np.arange(64), rng.integers(0, 64, 256)])
    got = o.view(w.m, 64, 128)[torch.from_numpy(rows).to(dev), torch.from_numpy(heads).to(dev)]
    got = got.cpu().numpy()
    del o
    qn, kn, vn = q.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy()
    del q, k, v
    torch.cuda.empty_cache()
    ref = oracle.prefill_causal(qn, kn, vn, w.m, w.q_stride, w.kv_stride, 64, 8, 128,
                                rows=rows.astype(np.uint32), heads=heads.astype(np.uint32))
    _assert_close(got, ref, float(np.abs(vn).max()), "m 65536")


@pytest.mark.parametrize("kvs", [(1 << 24) - 4, 1 << 24], ids=["fast_copy_edge", "general_copy"])
def test_prefill_kv_stride_at_the_copy_offset_limit(dev, kvs):
    """K/V rows 2^24 - 4 or 2^24 floats apart (about 8.7 GB per tensor at 130
    rows): full tiles are copied with 32-bit per-lane offsets only below
    2^24, so the first case takes that copy near its widest span (head_dim
    32: 8 rows per copy instruction) and the second every tile the general
    copy. The same rows at a compact stride go to the oracle."""
    m, hq, hpk, d = 130, 2, 2, 32
    w = synth.PrefillWorkload("kvs", m=m, num_q_heads=hq, heads_per_kv=hpk, head_dim=d,
                              q_stride=hq * d, kv_stride=d, seed=71)
    q, k, v = synth.prefill_inputs_device(w, 71, dev)
    kb = torch.full((m, kvs), float("nan"), device=dev)
    vb = torch.full((m, kvs), float("nan"), device=dev)
    kb[:, :d] = k
    vb[:, :d] = v
    o = torch.full((m, hq * d), float("nan"), device=dev)
    A.attn_prefill_causal(q, kb, vb, o, m, hq * d, kvs, hq, hpk, d)
    torch.cuda.synchronize()
    got = o.cpu().numpy()
    del kb, vb
    torch.cuda.empty_cache()
    qn, kn, vn = q.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy()
    ref = oracle.prefill_causal(qn, kn, vn, m, hq * d, d, hq, hpk, d)
    _assert_close(got.reshape(ref.shape), ref, float(np.abs(vn).max()), f"kv_stride {kvs}")


@pytest.mark.parametrize("per_tile,m", [(6.0, 700), (9.0, 700), (25.0, 256)])
def test_prefill_rising_scores(dev, per_tile, m):
    """Scores that rise along the keys by `per_tile` log2 units per 64 keys
    (below, just above and far above the point where the kernel raises its
    reference maximum); the top score stays near 100 log2 units, where fp32
    scores still meet the bar (a dot product of magnitude S carries a
    rounding error of order S * 2^-24)."""
    hq, hpk, d = 4, 2, 64
    hkv = hq // hpk
    rng = np.random.default_rng(int(per_tile * 10))
    scale = 1.0 / np.sqrt(d)
    q = np.zeros((m, hq * d), np.float32)
    k = np.zeros((m, hkv * d), np.float32)
    q[:, :] = (rng.standard_normal((m, hq * d)) * 0.1 + 1.0).astype(np.float32)
    # score_j ~ scale * <q, k_j> * log2(e) = per_tile * j / 64 (+ noise)
    slope = per_tile / 64.0 / (scale * np.log2(np.e) * d)
    k[:, :] = (np.arange(m)[:, None] * slope
               + rng.standard_normal((m, hkv * d)) * 0.05).astype(np.float32)
    v = rng.standard_normal((m, hkv * d)).astype(np.float32)
    w = synth.PrefillWorkload("rise", m=m, num_q_heads=hq, heads_per_kv=hpk, head_dim=d,
                              q_stride=hq * d, kv_stride=hkv * d, seed=0)
    o = _gpu_prefill(dev, w, q, k, v)
    _assert_close(_heads(w, o), _ref_prefill(w, q, k, v), float(np.abs(v).max()),
                  f"rising {per_tile}")


def test_prefill_wide_score_spread(dev):
    """q and K with standard deviation 6: scores spread over hundreds of log2
    units, most weights underflow, the reference maximum moves often."""
    w = synth.PrefillWorkload("wide", m=900, num_q_heads=8, heads_per_kv=4, head_dim=128,
                              q_stride=8 * 128, kv_stride=2 * 128, sigma=6.0, seed=901)
    q, k, v = synth.prefill_inputs(w)
    o = _gpu_prefill(dev, w, q, k, v)
    _assert_close(_heads(w, o), _ref_prefill(w, q, k, v), _vmax_prefill(w, v), "wide")


# ------------------------------------------------- invariants on GPU outputs

def test_prefill_future_rows_do_not_reach_earlier_rows(dev):
    """Rewriting the K/V rows from row 192 on leaves the outputs of rows
    0-191 bit for bit (the tiles those rows read end before row 192, and the
    kernel is deterministic); the later rows change."""
    w = synth.PrefillWorkload("fut", m=500, num_q_heads=12, heads_per_kv=6, head_dim=128,
                              q_stride=12 * 128, kv_stride=2 * 128, seed=505)
    q, k, v = synth.prefill_inputs(w)
    o1 = _gpu_prefill(dev, w, q, k, v)
    k2, v2 = k.copy(), v.copy()
    rng = np.random.default_rng(506)
    k2[192:] = rng.standard_normal(k2[192:].shape).astype(np.float32)
    v2[192:] = rng.standard_normal(v2[192:].shape).astype(np.float32)
    o2 = _gpu_prefill(dev, w, q, k2, v2)
    assert np.array_equal(o1[:192], o2[:192])
    assert not np.array_equal(o1[192:], o2[192:])


def test_prefill_gqa_equals_mha_with_repeated_kv_heads(dev):
    """GQA with 4 query heads per KV head gives the same bits as MHA over
    K/V heads repeated consecutively (each query head's arithmetic is the
    same; only the grouping of waves differs)."""
    m, hq, hpk, d = 333, 8, 4, 64
    hkv = hq // hpk
    w = synth.PrefillWorkload("gqa", m=m, num_q_heads=hq, heads_per_kv=hpk, head_dim=d,
                              q_stride=hq * d, kv_stride=hkv * d, seed=77)
    q, k, v = synth.prefill_inputs(w)
    o_gqa = _gpu_prefill(dev, w, q, k, v)
    rep = lambda x: np.ascontiguousarray(
        np.repeat(x.reshape(m, hkv, d), hpk, axis=1).reshape(m, hq * d))
    w_mha = w.with_(heads_per_kv=1, kv_stride=hq * d)
    o_mha = _gpu_prefill(dev, w_mha, q, rep(k), rep(v))
    assert np.array_equal(o_gqa, o_mha)


def test_decode_gqa_equals_mha_with_repeated_kv_heads(dev):
    """The same for decode, within the bar (the work split differs with the
    head count, so the summation order does too)."""
    b, hq, hkv, d, t = 3, 12, 2, 128, 700
    w, (q, k, v) = _decode_case(b, hq, hkv, d, t, t, seed=88)
    got = _gpu_decode(dev, w, q, k, v)
    kr = np.ascontiguousarray(np.repeat(k, hq // hkv, axis=1))
    vr = np.ascontiguousarray(np.repeat(v, hq // hkv, axis=1))
    w_mha = w.with_(kv_heads=hq)
    got_mha = _gpu_decode(dev, w_mha, q, kr, vr)
    _assert_close(got, got_mha.astype(np.float64), _vmax_decode(w, v), "gqa vs mha")


@pytest.mark.parametrize("case", [(5, 12, 2, 128, 300, 300, 0), (4, 8, 8, 64, 90, 90, 17),
                                  (3, 10, 2, 224, 200, 150, 0), (32, 12, 2, 128, 4096, 4096, 0),
                                  (40, 8, 2, 64, 128, 128, 0)],
                         ids=lambda c: "b{}_hq{}_hkv{}_d{}_ms{}_bd{}_w{}".format(*c))
def test_decode_rope_append_varlen_matches_oracle(dev, case):
    """Rotary decode step with one position and one angle table per sequence
    against the oracle's fused step run sequence by sequence."""
    b, hq, hkv, d, ms, bound, win = case
    seed = sum(case) % 863
    w = synth.DecodeWorkload("rv", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=ms, total_seq=bound, window=win, seed=seed)
    q, k, v = synth.decode_inputs(w)
    kn, vn = synth.append_inputs(b, hkv, d, seed=seed + 1)
    pos = synth.seq_lengths(b, bound, seed=seed + 2) - 1
    tabs = [synth.rope_tables(d, int(p)) for p in pos]
    cos_t = np.ascontiguousarray(np.stack([t[0] for t in tabs]))
    sin_t = np.ascontiguousarray(np.stack([t[1] for t in tabs]))
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    out = torch.full((b, hq, d), float("nan"), device=dev)
    ws = _poisoned_ws(A.attn_decode_workspace_bytes(b, hq, hkv, d, bound, win), b, hq, dev)
    A.attn_decode_rope_append_varlen(
        torch.from_numpy(q).to(dev), torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev),
        torch.from_numpy(cos_t).to(dev), torch.from_numpy(sin_t).to(dev), kd, vd, out,
        torch.from_numpy(pos.astype(np.int32)).to(dev), b, hq, hkv, d, ms, bound, win,
        w.scale, ws)
    torch.cuda.synchronize()
    k0 = k.copy()
    ref = np.empty((b, hq, d))
    for i in range(b):   # the oracle's fused step, sequence by sequence (updates k, v)
        ref[i] = oracle.decode_rope_append(q[i:i + 1], kn[i:i + 1], vn[i:i + 1], cos_t[i],
                                           sin_t[i], k[i:i + 1], v[i:i + 1], 1, hq, hkv, d, ms,
                                           int(pos[i]), win, w.scale)[0]
    kc, vc = kd.cpu().numpy(), vd.cpu().numpy()
    assert np.array_equal(vc, v)
    for i in range(b):
        keep = np.arange(ms) != pos[i]
        assert np.array_equal(kc[i][:, keep], k0[i][:, keep])
        err = np.abs(kc[i, :, pos[i]].astype(np.float64) - k[i, :, pos[i]])
        assert np.all(err <= _rope_row_bound(kn[i])), (i, float(err.max()))
    _assert_close(out.cpu().numpy(), ref, _vmax_varlen(w, v, pos, plus=1), str(case))


def test_decode_rope_append_varlen_no_heads_rotates_each_row(dev):
    """num_heads == 0: each sequence appends its row rotated by its own table."""
    b, hkv, d, ms, bound = 3, 2, 64, 16, 12
    ks, vs = synth.append_inputs(b, hkv, d, seed=9)
    pos = np.array([11, 0, 5], np.uint32)
    tabs = [synth.rope_tables(d, 100.0 * (i + 1)) for i in range(b)]
    cos_t = np.ascontiguousarray(np.stack([t[0] for t in tabs]))
    sin_t = np.ascontiguousarray(np.stack([t[1] for t in tabs]))
    kc = torch.full((b, hkv, ms, d), -2.0, device=dev)
    vc = torch.full((b, hkv, ms, d), 3.0, device=dev)
    A.attn_decode_rope_append_varlen(
        0, torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev),
        torch.from_numpy(cos_t).to(dev), torch.from_numpy(sin_t).to(dev), kc, vc, 0,
        torch.from_numpy(pos.astype(np.int32)).to(dev), b, 0, hkv, d, ms, bound, 0, 0.125, None)
    torch.cuda.synchronize()
    kn, vn = kc.cpu().numpy(), vc.cpu().numpy()
    for i in range(b):
        assert np.array_equal(vn[i, :, pos[i]], vs[i])
        err = np.abs(kn[i, :, pos[i]].astype(np.float64) - oracle.rope(ks[i], cos_t[i], sin_t[i]))
        assert np.all(err <= _rope_row_bound(ks[i])), float(err.max())
        keep = np.arange(ms) != pos[i]
        assert np.all(kn[i][:, keep] == -2.0) and np.all(vn[i][:, keep] == 3.0)


def test_decode_rope_append_varlen_invalid_position(dev):
    """positions[b] + 1 > seq_bound: NaN output and no cache write for that
    sequence; the others are the oracle's fused rotary step."""
    b, hq, hkv, d, ms, bound = 3, 6, 2, 64, 32, 20
    w = synth.DecodeWorkload("rv", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=ms, total_seq=bound, seed=31)
    q, k, v = synth.decode_inputs(w)
    kn, vn = synth.append_inputs(b, hkv, d, seed=32)
    pos = np.array([19, 20, 4], np.uint32)
    tabs = [synth.rope_tables(d, int(p)) for p in pos]
    cos_t = np.ascontiguousarray(np.stack([t[0] for t in tabs]))
    sin_t = np.ascontiguousarray(np.stack([t[1] for t in tabs]))
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    out = torch.zeros((b, hq, d), device=dev)
    A.attn_decode_rope_append_varlen(
        torch.from_numpy(q).to(dev), torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev),
        torch.from_numpy(cos_t).to(dev), torch.from_numpy(sin_t).to(dev), kd, vd, out,
        torch.from_numpy(pos.astype(np.int32)).to(dev), b, hq, hkv, d, ms, bound, 0, w.scale,
        A.decode_workspace(b, hq, hkv, d, bound, 0))
    torch.cuda.synchronize()
    got, kc, vc = out.cpu().numpy(), kd.cpu().numpy(), vd.cpu().numpy()
    assert np.all(np.isnan(got[1]))
    assert np.array_equal(kc[1], k[1]) and np.array_equal(vc[1], v[1])
    for i in (0, 2):
        kr, vr = k[i:i + 1].copy(), v[i:i + 1].copy()
        ref = oracle.decode_rope_append(q[i:i + 1], kn[i:i + 1], vn[i:i + 1], cos_t[i], sin_t[i],
                                        kr, vr, 1, hq, hkv, d, ms, int(pos[i]), 0, w.scale)
        assert np.array_equal(vc[i], vr[0])
        keep = np.arange(ms) != pos[i]
        assert np.array_equal(kc[i][:, keep], k[i][:, keep])
        err = np.abs(kc[i, :, pos[i]].astype(np.float64) - kr[0, :, pos[i]])
        assert np.all(err <= _rope_row_bound(kn[i])), float(err.max())
        vmax = float(np.abs(vr[0, :, :pos[i] + 1]).max())  # rows the step attends
        _assert_close(got[i:i + 1], ref, vmax, f"sequence {i}")
