"""attn_decode_append_noalloc: the decode step with the library's own
per-GPU workspace array instead of a caller's buffer.

CPU: the argument rules and the array's size limit (host checks that return
before any HIP call). GPU: calls in a row through the C ABI, the second with
a smaller input and the third with the first one's again, each compared with
attn_decode_append on the same inputs (the same kernels and work split, so
the same bits) and with the fp64 oracle at max|err| <= 2e-5 * max|V|.
"""
import ctypes
import os

import numpy as np
import pytest

import attention_gqa_online_amd as A
import oracle
import synth

P = 0x10000  # a 16-byte aligned stand-in address; never dereferenced on the CPU
TOL = 2e-5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(A.SO_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return A.library()


def _noalloc(lib, b=2, hq=12, hkv=2, d=128, max_seq=64, pos=63, window=0, scale=0.088,
             ptrs=(P,) * 6):
    return lib.attn_decode_append_noalloc(*ptrs, b, hq, hkv, d, max_seq, pos, window,
                                          ctypes.c_float(scale), None)


def test_noalloc_argument_rules(lib):
    INVALID, UNSUPPORTED = A.ATTN_ERR_INVALID, A.ATTN_ERR_UNSUPPORTED
    assert _noalloc(lib, d=48) == INVALID
    assert _noalloc(lib, d=352) == UNSUPPORTED
    assert _noalloc(lib, hkv=0) == INVALID
    assert _noalloc(lib, hq=12, hkv=5) == INVALID
    assert _noalloc(lib, pos=64, max_seq=64) == INVALID
    assert _noalloc(lib, scale=float("nan")) == INVALID
    for i in range(6):
        for bad in (0, P + 4):
            ptrs = tuple(bad if j == i else P for j in range(6))
            assert _noalloc(lib, ptrs=ptrs) == INVALID, (i, bad)
    assert _noalloc(lib, b=0) == A.ATTN_OK


def test_noalloc_rejects_shapes_past_the_array(lib):
    """More than 16384 work units (more arrival counters than the array's
    fixed counter block), or partial states past its 16 MiB: both
    ATTN_ERR_UNSUPPORTED, decided on the host."""
    assert _noalloc(lib, b=16385, hq=1, hkv=1, max_seq=100, pos=99) == A.ATTN_ERR_UNSUPPORTED
    # 1024 sequences x 8 KV heads of 8 Q heads at head_dim 256: one split per
    # unit, 8192 x 8 x 260 floats of partial states = 68 MB
    assert _noalloc(lib, b=1024, hq=64, hkv=8, d=256, max_seq=1000,
                    pos=999) == A.ATTN_ERR_UNSUPPORTED
    # the batched decode step of 32 sequences fits at every position
    need = A.attn_decode_workspace_bytes(32, 12, 2, 128, 4096, 0)
    assert 0 < need < 1 << 20


# (batch, hq, hkv, d, max_seq, position, window, seed): the second call's
# input is smaller; the third repeats the first shape on new inputs
CALLS = [(32, 12, 2, 128, 4096, 4095, 0, 61), (3, 8, 2, 64, 700, 640, 129, 62),
         (32, 12, 2, 128, 4096, 4095, 0, 63)]


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_step_on_calls_in_a_row():
    import torch
    dev = torch.device("cuda:0")
    for b, hq, hkv, d, ms, pos, win, seed in CALLS:
        case = f"b{b} hq{hq} hkv{hkv} d{d} max_seq{ms} pos{pos} window{win}"
        print("noalloc call:", case, flush=True)
        w = synth.DecodeWorkload("noalloc", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                                 max_seq=ms, total_seq=pos + 1, window=win, seed=seed)
        q, kc, vc = synth.decode_inputs(w)
        kn, vn = synth.append_inputs(b, hkv, d, seed=seed + 1000)
        t = {n: torch.from_numpy(x).to(dev) for n, x in
             (("q", q), ("kn", kn), ("vn", vn), ("kc", kc), ("vc", vc))}
        kc2, vc2 = t["kc"].clone(), t["vc"].clone()
        out_ws = torch.full((b, hq, d), float("nan"), device=dev)
        out_na = torch.full((b, hq, d), float("nan"), device=dev)
        ws = A.decode_workspace(b, hq, hkv, d, pos + 1, win, device=dev)
        A.attn_decode_append(t["q"], t["kn"], t["vn"], t["kc"], t["vc"], out_ws, b, hq, hkv,
                             d, ms, pos, win, w.scale, ws)
        A.attn_decode_append_noalloc(t["q"], t["kn"], t["vn"], kc2, vc2, out_na, b, hq, hkv,
                                     d, ms, pos, win, w.scale)
        torch.cuda.synchronize()
        got, want = out_na.cpu().numpy(), out_ws.cpu().numpy()
        # the same kernels, work split and fold order: the same bits
        assert np.array_equal(got, want), case
        assert torch.equal(kc2, t["kc"]) and torch.equal(vc2, t["vc"]), case
        # and the fp64 oracle's bar, as for the workspace step
        oracle.kv_append(kn, vn, kc, vc, b, hkv, d, ms, pos)
        ref = oracle.decode(q, kc, vc, b, hq, hkv, d, ms, pos + 1, win, w.scale)
        vmax = float(np.abs(vc[:, :, w.window_start:pos + 1]).max())
        err = float(np.abs(got.astype(np.float64) - ref).max())
        assert err <= TOL * vmax, f"{case}: max|err| {err:.3e} > {TOL * vmax:.3e}"


@pytest.mark.gpu
def test_noalloc_step_replays_from_a_hip_graph():
    """The no-allocation step captured in a HIP graph (the callers it is
    for): every replay, with eager work between replays that includes an
    eager no-allocation call of another shape on the same array, gives the
    bits of the eager workspace step."""
    import torch
    dev = torch.device("cuda:0")
    b, hq, hkv, d, ms, pos = 8, 12, 2, 128, 2100, 2047
    w = synth.DecodeWorkload("noalloc_graph", batch=b, num_heads=hq, kv_heads=hkv, head_dim=d,
                             max_seq=ms, total_seq=pos + 1, seed=71)
    q, kc, vc = synth.decode_inputs(w)
    kn, vn = synth.append_inputs(b, hkv, d, seed=72)
    qd, kd, vd, knd, vnd = (torch.from_numpy(x).to(dev) for x in (q, kc, vc, kn, vn))
    ws = A.decode_workspace(b, hq, hkv, d, pos + 1, 0, device=dev)
    out_e = torch.empty(b, hq, d, device=dev)
    A.attn_decode_append(qd, knd, vnd, kd, vd, out_e, b, hq, hkv, d, ms, pos, 0, w.scale, ws)
    # another shape for the eager calls between replays
    w2 = synth.DecodeWorkload("noalloc_other", batch=3, num_heads=8, kv_heads=2, head_dim=64,
                              max_seq=900, total_seq=800, window=300, seed=73)
    q2, k2, v2 = synth.decode_inputs(w2)
    kn2, vn2 = synth.append_inputs(3, 2, 64, seed=74)
    q2d, k2d, v2d, kn2d, vn2d = (torch.from_numpy(x).to(dev) for x in (q2, k2, v2, kn2, vn2))
    out2_e = torch.empty(3, 8, 64, device=dev)
    ws2 = A.decode_workspace(3, 8, 2, 64, 800, 300, device=dev)
    A.attn_decode_append(q2d, kn2d, vn2d, k2d, v2d, out2_e, 3, 8, 2, 64, 900, 799, 300,
                         w2.scale, ws2)
    out_g = torch.empty(b, hq, d, device=dev)
    out2_n = torch.empty(3, 8, 64, device=dev)
    # a first call on this device looks up the array outside the capture
    A.attn_decode_append_noalloc(qd, knd, vnd, kd, vd, out_g, b, hq, hkv, d, ms, pos, 0, w.scale)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.attn_decode_append_noalloc(qd, knd, vnd, kd, vd, out_g, b, hq, hkv, d, ms, pos, 0,
                                     w.scale)
    for rep in range(4):
        print("noalloc graph replay", rep, flush=True)
        out_g.fill_(float("nan"))
        out2_n.fill_(float("nan"))
        A.attn_decode_append_noalloc(q2d, kn2d, vn2d, k2d, v2d, out2_n, 3, 8, 2, 64, 900, 799,
                                     300, w2.scale)
        junk = torch.randn(1 << 20, device=dev).sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}"
        assert torch.equal(out2_n, out2_e), f"eager call before replay {rep}"
        assert bool(torch.isfinite(junk))
