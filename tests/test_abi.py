"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/attn.h declares, and rejects invalid arguments on the host before any
HIP call (so these calls are safe without a device; none of them launches).

Calls that would launch are never made here: every call below either breaks
a rule of attn.h or has zero work (m == 0, batch == 0), both of which return
before the HIP runtime is touched.
"""
import ctypes
import os
import re

import pytest

import attention_gqa_online_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED = A.ATTN_OK, A.ATTN_ERR_INVALID, A.ATTN_ERR_UNSUPPORTED
P = 0x10000  # a 16-byte aligned stand-in address; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(A.SO_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return A.library()


def _declared_functions():
    with open(os.path.join(ROOT, "include", "attn.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:attn_status|size_t|const char \*)\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_three_operations():
    names = _declared_functions()
    for n in ("attn_prefill_causal", "attn_decode", "kv_append",
              "attn_decode_workspace_bytes", "attn_status_string"):
        assert n in names
    assert tuple(sorted(A.EXPORTS)) == tuple(names)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    for s in (OK, INVALID, UNSUPPORTED, A.ATTN_ERR_HIP):
        assert A.attn_status_string(s).startswith("ATTN_")
    assert "unknown" in A.attn_status_string(99)


def _prefill(lib, m=16, q_stride=None, kv_stride=None, hq=4, hpk=2, d=32,
             ptrs=(P, P, P, P)):
    hkv = hq // hpk if hpk else 0
    q_stride = hq * d if q_stride is None else q_stride
    kv_stride = hkv * d if kv_stride is None else kv_stride
    return lib.attn_prefill_causal(*ptrs, m, q_stride, kv_stride, hq, hpk, d, None)


def test_prefill_page_constructor_cases(lib, golden):
    """The page's kernel cases: head_dim 64/128 with 6 heads per KV head and
    the MHA case are accepted; head_dim 48 and heads_per_kv 0 are rejected.
    Accepted shapes are exercised with m = 0 (no launch)."""
    for case in golden["prefill_kernel_cases"]["cases"]:
        d, hpk = case["head_dim"], case["heads_per_kv"]
        hq = 12 if hpk else 12
        st = _prefill(lib, m=0 if case["valid"] else 16, hq=hq, hpk=hpk, d=d,
                      q_stride=hq * d, kv_stride=(hq // hpk if hpk else 1) * d)
        assert st == (OK if case["valid"] else INVALID), case


def test_prefill_argument_rules(lib):
    assert _prefill(lib, d=0) == INVALID
    assert _prefill(lib, d=288) == UNSUPPORTED           # multiple of 32 past 256
    assert _prefill(lib, d=320) == UNSUPPORTED
    assert _prefill(lib, hq=5, hpk=2) == INVALID         # Hq not a multiple of hpk
    assert _prefill(lib, q_stride=4 * 32 - 4) == INVALID # row too short for Q heads
    assert _prefill(lib, kv_stride=2 * 32 - 4) == INVALID
    assert _prefill(lib, q_stride=4 * 32 + 2) == INVALID # stride not a multiple of 4
    assert _prefill(lib, kv_stride=2 * 32 + 6) == INVALID
    assert _prefill(lib, ptrs=(P, P, P, 0)) == INVALID   # null output
    assert _prefill(lib, ptrs=(P + 4, P, P, P)) == INVALID  # misaligned q
    assert _prefill(lib, ptrs=(P, P, P + 8, P)) == INVALID
    assert _prefill(lib, m=0, ptrs=(0, 0, 0, 0)) == OK   # no work, no launch
    assert _prefill(lib, hq=0, hpk=1, q_stride=0, kv_stride=0) == OK


def _decode(lib, b=2, hq=12, hkv=2, d=128, max_seq=64, t=64, window=0,
            scale=0.088, ws=P, ws_bytes=None, ptrs=(P, P, P, P)):
    if ws_bytes is None:
        ws_bytes = lib.attn_decode_workspace_bytes(b, hq, hkv, d, t, window) or 1 << 30
    return lib.attn_decode(*ptrs, b, hq, hkv, d, max_seq, t, window,
                           ctypes.c_float(scale), ws, ws_bytes, None)


def test_decode_argument_rules(lib):
    assert _decode(lib, d=48) == INVALID
    assert _decode(lib, d=288) == UNSUPPORTED
    assert _decode(lib, hkv=0) == INVALID
    assert _decode(lib, hq=12, hkv=5) == INVALID
    assert _decode(lib, t=0) == INVALID                     # nothing to attend
    assert _decode(lib, t=65, max_seq=64) == INVALID        # past the cache
    assert _decode(lib, scale=float("nan")) == INVALID
    assert _decode(lib, scale=float("inf")) == INVALID
    assert _decode(lib, ptrs=(P, 0, P, P)) == INVALID
    assert _decode(lib, ptrs=(P, P, P, P + 12)) == INVALID
    assert _decode(lib, ws=0) == INVALID
    need = lib.attn_decode_workspace_bytes(2, 12, 2, 128, 64, 0)
    assert need > 0
    assert _decode(lib, ws_bytes=0) == INVALID              # any workspace is too small
    assert _decode(lib, b=0) == OK                          # no work, no launch
    assert _decode(lib, hq=0) == OK


def test_decode_workspace_sizes(lib):
    f = lib.attn_decode_workspace_bytes
    assert f(0, 12, 2, 128, 4096, 0) == 0
    assert f(32, 12, 2, 48, 4096, 0) == 0
    assert f(32, 12, 0, 128, 4096, 0) == 0
    assert f(32, 12, 2, 128, 0, 0) == 0
    a = f(32, 12, 2, 128, 4096, 0)
    b = f(16, 32, 8, 128, 32768, 4096)
    assert a > 0 and b > 0
    # a window bounds the work: same size as an unwindowed cache of that length
    assert f(16, 32, 8, 128, 32768, 4096) == f(16, 32, 8, 128, 4096, 0)
    # the counter block (65536 bytes up to 16384 units, 4 bytes per unit past
    # that), then a generous upper bound on the partial states: one per 32
    # attended rows and head
    for args in [(32, 12, 2, 128, 4096, 0), (1, 64, 1, 64, 100000, 0), (3, 7, 7, 32, 1, 0),
                 (2048, 16, 2, 128, 64, 0)]:
        bsz, hq, hkv, d, t, w = args
        cnt = max(65536, (4 * bsz * hq + 255) // 256 * 256)
        assert 65536 < f(*args) <= cnt + 4 * bsz * hq * (d + 4) * (t // 32 + 2) * 2


def test_kv_append_argument_rules(lib):
    f = lib.kv_append
    assert f(P, P, P, P, 2, 2, 48, 16, 0, None) == INVALID
    assert f(P, P, P, P, 2, 2, 128, 16, 16, None) == INVALID   # position >= max_seq
    assert f(P, P, P, P, 2, 2, 128, 16, 99, None) == INVALID
    assert f(P, P, 0, P, 2, 2, 128, 16, 0, None) == INVALID
    assert f(P, P + 4, P, P, 2, 2, 128, 16, 0, None) == INVALID
    assert f(0, 0, 0, 0, 0, 2, 128, 16, 0, None) == OK          # no work
    assert f(0, 0, 0, 0, 2, 0, 128, 16, 0, None) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    """The Python path has no fallback: a missing library is an error."""
    monkeypatch.setattr(A, "_lib", None)
    monkeypatch.setattr(A, "SO_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        A.library()


def _decode_append(lib, b=2, hq=12, hkv=2, d=128, max_seq=64, pos=63, window=0,
                   scale=0.088, ws=P, ws_bytes=1 << 30, ptrs=(P, P, P, P, P, P)):
    return lib.attn_decode_append(*ptrs, b, hq, hkv, d, max_seq, pos, window,
                                  ctypes.c_float(scale), ws, ws_bytes, None)


def test_decode_append_argument_rules(lib):
    assert _decode_append(lib, d=48) == INVALID
    assert _decode_append(lib, d=352) == UNSUPPORTED
    assert _decode_append(lib, hkv=0) == INVALID
    assert _decode_append(lib, hq=12, hkv=5) == INVALID
    assert _decode_append(lib, pos=64, max_seq=64) == INVALID   # past the cache
    assert _decode_append(lib, scale=float("nan")) == INVALID
    assert _decode_append(lib, ptrs=(P, 0, P, P, P, P)) == INVALID
    assert _decode_append(lib, ptrs=(P, P, P, P + 4, P, P)) == INVALID
    assert _decode_append(lib, ptrs=(P, P, P, P, P, 0)) == INVALID
    assert _decode_append(lib, ws_bytes=0) == INVALID
    assert _decode_append(lib, ws=0) == INVALID
    assert _decode_append(lib, b=0) == OK                        # no work, no launch
    # with no Q heads the step only appends: the append's own size bound
    # (batch * kv_heads * head_dim / 4 < 2^31) still holds, as in kv_append
    assert _decode_append(lib, b=1 << 24, hq=0, hkv=8, max_seq=1 << 20,
                          pos=0) == UNSUPPORTED
    assert lib.kv_append(P, P, P, P, 1 << 24, 8, 128, 1 << 20, 0, None) == UNSUPPORTED


def _decode_rope(lib, b=2, hq=12, hkv=2, d=128, max_seq=64, pos=63, window=0,
                 scale=0.088, ws=P, ws_bytes=1 << 30, ptrs=(P,) * 8):
    return lib.attn_decode_rope_append(*ptrs, b, hq, hkv, d, max_seq, pos, window,
                                       ctypes.c_float(scale), ws, ws_bytes, None)


def test_decode_rope_append_argument_rules(lib):
    assert _decode_rope(lib, d=48) == INVALID
    assert _decode_rope(lib, d=384) == UNSUPPORTED
    assert _decode_rope(lib, hkv=0) == INVALID
    assert _decode_rope(lib, hq=12, hkv=5) == INVALID
    assert _decode_rope(lib, pos=64, max_seq=64) == INVALID
    assert _decode_rope(lib, scale=float("inf")) == INVALID
    for i in range(8):   # every pointer: null, then misaligned
        for bad in (0, P + 4):
            ptrs = tuple(bad if j == i else P for j in range(8))
            assert _decode_rope(lib, ptrs=ptrs) == INVALID, (i, bad)
    assert _decode_rope(lib, ws_bytes=0) == INVALID
    assert _decode_rope(lib, ws=0) == INVALID
    assert _decode_rope(lib, b=0) == OK                            # no work, no launch
    assert _decode_rope(lib, b=0, ptrs=(0,) * 8) == OK
    assert _decode_rope(lib, b=1 << 24, hq=0, hkv=8, max_seq=1 << 20, pos=0) == UNSUPPORTED


def test_kv_append_rows_argument_rules(lib):
    f = lib.kv_append_rows
    #        k  v  kc vc  m  stride hkv  d  max_seq pos
    assert f(P, P, P, P, 4, 256, 2, 48, 16, 0, None) == INVALID        # d % 32
    assert f(P, P, P, P, 4, 256, 2, 128, 16, 13, None) == INVALID      # past the cache
    assert f(P, P, P, P, 4, 255, 2, 128, 16, 0, None) == INVALID       # stride too small
    assert f(P, P, P, P, 4, 258, 2, 128, 16, 0, None) == INVALID       # stride % 4
    assert f(P, P, 0, P, 4, 256, 2, 128, 16, 0, None) == INVALID
    assert f(P, P + 8, P, P, 4, 256, 2, 128, 16, 0, None) == INVALID
    assert f(P, P, P, P, 1 << 26, 256, 2, 128, 1 << 27, 0, None) == UNSUPPORTED
    assert f(0, 0, 0, 0, 0, 256, 2, 128, 16, 16, None) == OK           # no rows
    assert f(0, 0, 0, 0, 4, 256, 0, 128, 16, 0, None) == OK            # no heads
    assert f(P, P, P, P, 4, 256, 2, 128, 16, 13, None) == INVALID


def _varlen(lib, b=2, hq=12, hkv=2, d=128, max_seq=64, bound=64, window=0,
            scale=0.088, ws=P, ws_bytes=1 << 30, ptrs=(P,) * 5):
    return lib.attn_decode_varlen(*ptrs, b, hq, hkv, d, max_seq, bound, window,
                                  ctypes.c_float(scale), ws, ws_bytes, None)


def test_decode_varlen_argument_rules(lib):
    assert _varlen(lib, d=48) == INVALID
    assert _varlen(lib, d=416) == UNSUPPORTED
    assert _varlen(lib, hkv=0) == INVALID
    assert _varlen(lib, hq=12, hkv=5) == INVALID
    assert _varlen(lib, bound=0) == INVALID
    assert _varlen(lib, bound=65, max_seq=64) == INVALID
    assert _varlen(lib, scale=float("nan")) == INVALID
    for i in range(4):
        ptrs = tuple(P + 4 if j == i else P for j in range(5))
        assert _varlen(lib, ptrs=ptrs) == INVALID, i
    assert _varlen(lib, ptrs=(P, P, P, P, 0)) == INVALID               # no lengths
    assert _varlen(lib, ptrs=(P, P, P, P, P + 2)) == INVALID
    assert _varlen(lib, ws_bytes=0) == INVALID
    assert _varlen(lib, ws=0) == INVALID
    assert _varlen(lib, b=0) == OK
    assert _varlen(lib, hq=0) == OK


def _append_varlen(lib, b=2, hq=12, hkv=2, d=128, max_seq=64, bound=64, window=0,
                   scale=0.088, ws=P, ws_bytes=1 << 30, ptrs=(P,) * 7):
    return lib.attn_decode_append_varlen(*ptrs, b, hq, hkv, d, max_seq, bound, window,
                                         ctypes.c_float(scale), ws, ws_bytes, None)


def test_decode_append_varlen_argument_rules(lib):
    assert _append_varlen(lib, d=48) == INVALID
    assert _append_varlen(lib, d=448) == UNSUPPORTED
    assert _append_varlen(lib, hkv=0) == INVALID
    assert _append_varlen(lib, bound=0) == INVALID
    assert _append_varlen(lib, bound=65, max_seq=64) == INVALID
    assert _append_varlen(lib, scale=float("inf")) == INVALID
    for i in range(6):
        for bad in (0, P + 4):
            ptrs = tuple(bad if j == i else P for j in range(7))
            assert _append_varlen(lib, ptrs=ptrs) == INVALID, (i, bad)
    assert _append_varlen(lib, ptrs=(P,) * 6 + (0,)) == INVALID
    assert _append_varlen(lib, ptrs=(P,) * 6 + (P + 1,)) == INVALID
    assert _append_varlen(lib, ws_bytes=0) == INVALID
    assert _append_varlen(lib, b=0) == OK
    assert _append_varlen(lib, b=0, ptrs=(0,) * 7) == OK


def _rope_varlen(lib, b=2, hq=12, hkv=2, d=128, max_seq=64, bound=64, window=0,
                 scale=0.088, ws=P, ws_bytes=1 << 30, ptrs=(P,) * 9):
    return lib.attn_decode_rope_append_varlen(*ptrs, b, hq, hkv, d, max_seq, bound, window,
                                              ctypes.c_float(scale), ws, ws_bytes, None)


def test_decode_rope_append_varlen_argument_rules(lib):
    assert _rope_varlen(lib, d=48) == INVALID
    assert _rope_varlen(lib, d=480) == UNSUPPORTED
    assert _rope_varlen(lib, hkv=0) == INVALID
    assert _rope_varlen(lib, bound=65, max_seq=64) == INVALID
    assert _rope_varlen(lib, scale=float("nan")) == INVALID
    for i in range(8):   # q, k, v, cos, sin, caches, out: null, then misaligned
        for bad in (0, P + 4):
            ptrs = tuple(bad if j == i else P for j in range(9))
            assert _rope_varlen(lib, ptrs=ptrs) == INVALID, (i, bad)
    assert _rope_varlen(lib, ptrs=(P,) * 8 + (0,)) == INVALID      # positions
    assert _rope_varlen(lib, ws_bytes=0) == INVALID
    assert _rope_varlen(lib, b=0, ptrs=(0,) * 9) == OK


def test_library_exports_no_other_c_symbols(lib):
    """The shared library's unmangled exports are exactly the header's."""
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", A.SO_PATH], capture_output=True,
                         text=True, check=True).stdout
    names = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    c_names = {n for n in names if not n.startswith("_Z")}
    assert c_names == set(_declared_functions())
