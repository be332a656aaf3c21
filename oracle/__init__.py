"""Oracle for fused GQA attention: plain fp64 CPU definition (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package. The HIP library never imports or links it, and the two share no
code. The arithmetic lives in ``oracle.c`` (see its header for what each
function follows on the pages); this module only compiles it with gcc and
marshals numpy arrays through ctypes.

Functions return float64 arrays:
  prefill_causal(...) -> [m, num_q_heads, head_dim], or [n_sel, head_dim]
                         for selected (row, head) pairs
  decode(...)         -> [batch, num_heads, head_dim], or [n_sel, head_dim]
                         for selected (sequence, head) pairs
  kv_append(...)      -> updates the float32 caches in place
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_default = None

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
SO_PATH = os.path.join(_HERE, "liboracle.so")

# Plain optimisation only: no -ffast-math (no reassociation of sums), no FMA
# contraction, no host-specific ISA, so the .so runs on any x86-64 host.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
          "-shared", "-Wall", "-Wextra"]
# The build that is timed as the CPU baseline, on the host that runs it:
# -O3 and that host's own ISA, still with no -ffast-math and no FMA
# contraction, so every sum is evaluated as written, in index order.
CFLAGS_NATIVE = ["-O3", "-march=native", "-std=c11", "-fopenmp", "-ffp-contract=off",
                 "-fPIC", "-shared", "-Wall", "-Wextra"]

_F32P = ctypes.POINTER(ctypes.c_float)
_U32P = ctypes.POINTER(ctypes.c_uint32)
_F64P = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True, src: str = _SRC, so_path: str = SO_PATH,
          native: bool = False) -> str:
    """Compile oracle.c (or another copy of it) into a shared library;
    ``native`` builds with CFLAGS_NATIVE for the host it runs on."""
    global _default
    if force or not os.path.exists(so_path):
        tmp = so_path + ".tmp"
        flags = CFLAGS_NATIVE if native else CFLAGS
        subprocess.check_call(["gcc", *flags, "-o", tmp, src, "-lm"])
        os.replace(tmp, so_path)
        if so_path == SO_PATH:
            _default = None
    return so_path


def _bind(lib):
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_prefill_scale.restype = ctypes.c_float
    lib.oracle_prefill_scale.argtypes = [ctypes.c_uint32]
    lib.oracle_prefill_causal.restype = ctypes.c_int
    lib.oracle_prefill_causal.argtypes = [
        _F32P, _F32P, _F32P, ctypes.c_uint32, ctypes.c_uint32,
        ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
        ctypes.c_size_t, _U32P, _U32P, _F64P]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [
        _F32P, _F32P, _F32P, ctypes.c_uint32, ctypes.c_uint32,
        ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
        ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t, _U32P, _U32P,
        _F64P]
    lib.oracle_rope.restype = ctypes.c_int
    lib.oracle_rope.argtypes = [_F32P, _F32P, _F32P, ctypes.c_size_t, ctypes.c_uint32, _F64P]
    lib.oracle_decode_rope_append.restype = ctypes.c_int
    lib.oracle_decode_rope_append.argtypes = [
        _F32P, _F32P, _F32P, _F32P, _F32P, _F32P, _F32P, ctypes.c_uint32,
        ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
        ctypes.c_uint32, ctypes.c_uint32, ctypes.c_float, _F64P]
    lib.oracle_kv_append.restype = ctypes.c_int
    lib.oracle_kv_append.argtypes = [
        _F32P, _F32P, _F32P, _F32P, ctypes.c_uint32, ctypes.c_uint32,
        ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
    lib.oracle_kv_append_rows.restype = ctypes.c_int
    lib.oracle_kv_append_rows.argtypes = [_F32P] * 4 + [ctypes.c_uint32] * 6
    lib.oracle_decode_varlen.restype = ctypes.c_int
    lib.oracle_decode_varlen.argtypes = [_F32P] * 3 + [_U32P] + [ctypes.c_uint32] * 6 + [
        ctypes.c_float, _F64P]
    return lib


def _f32(a, name, writable=False):
    if not isinstance(a, np.ndarray) or a.dtype != np.float32:
        raise TypeError(f"{name} must be a float32 numpy array")
    if not a.flags.c_contiguous:
        raise ValueError(f"{name} must be C-contiguous")
    if writable and not a.flags.writeable:
        raise ValueError(f"{name} must be writable")
    return a.ctypes.data_as(_F32P)


def _sel(a, b):
    if a is None:
        return None, None, 0
    a = np.ascontiguousarray(a, dtype=np.uint32)
    b = np.ascontiguousarray(b, dtype=np.uint32)
    if a.shape != b.shape or a.ndim != 1:
        raise ValueError("selection index arrays must be 1-D and equal length")
    return a, b, a.shape[0]


class Oracle:
    """ctypes view of one compiled copy of oracle.c."""

    def __init__(self, so_path: str = SO_PATH):
        self.so_path = so_path
        self._lib = _bind(ctypes.CDLL(so_path))

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())

    def prefill_scale(self, head_dim: int) -> float:
        """1/sqrt(head_dim) evaluated in f32, widened to a Python float."""
        return float(self._lib.oracle_prefill_scale(head_dim))

    def prefill_causal(self, q, k, v, m, q_stride, kv_stride, num_q_heads,
                       heads_per_kv, head_dim, rows=None, heads=None):
        """Causal GQA prefill in fp64 (all pairs, or the selected (row, head) ones)."""
        kv_heads = num_q_heads // max(heads_per_kv, 1)
        if num_q_heads * head_dim > q_stride:
            raise ValueError("q_stride too small")
        if kv_heads * head_dim > kv_stride:
            raise ValueError("kv_stride too small")
        # elements read: rows 0..m-1, columns [0, heads*d) of each row (so a
        # flat view starting inside a fused projection row is accepted)
        if m and (q.size < (m - 1) * q_stride + num_q_heads * head_dim
                  or k.size < (m - 1) * kv_stride + kv_heads * head_dim
                  or v.size < (m - 1) * kv_stride + kv_heads * head_dim):
            raise ValueError("input arrays smaller than the rows they must hold")
        rows, heads, n_sel = _sel(rows, heads)
        if rows is None:
            out = np.empty((m, num_q_heads, head_dim), dtype=np.float64)
        else:
            out = np.empty((n_sel, head_dim), dtype=np.float64)
        rc = self._lib.oracle_prefill_causal(
            _f32(q, "q"), _f32(k, "k"), _f32(v, "v"), m, q_stride, kv_stride,
            num_q_heads, heads_per_kv, head_dim, n_sel,
            None if rows is None else rows.ctypes.data_as(_U32P),
            None if heads is None else heads.ctypes.data_as(_U32P),
            out.ctypes.data_as(_F64P))
        if rc != 0:
            raise ValueError("oracle_prefill_causal rejected its arguments")
        return out

    def decode(self, q, k_cache, v_cache, batch, num_heads, kv_heads,
               head_dim, max_seq, total_seq, window, scale, bs=None, hs=None):
        """Single-query GQA decode with optional sliding window, in fp64."""
        n_cache = batch * kv_heads * max_seq * head_dim
        if (q.size < batch * num_heads * head_dim or k_cache.size < n_cache
                or v_cache.size < n_cache):
            raise ValueError("input arrays smaller than the stated shapes")
        bs, hs, n_sel = _sel(bs, hs)
        if bs is None:
            out = np.empty((batch, num_heads, head_dim), dtype=np.float64)
        else:
            out = np.empty((n_sel, head_dim), dtype=np.float64)
        rc = self._lib.oracle_decode(
            _f32(q, "q"), _f32(k_cache, "k_cache"), _f32(v_cache, "v_cache"),
            batch, num_heads, kv_heads, head_dim, max_seq, total_seq, window,
            ctypes.c_float(scale), n_sel,
            None if bs is None else bs.ctypes.data_as(_U32P),
            None if hs is None else hs.ctypes.data_as(_U32P),
            out.ctypes.data_as(_F64P))
        if rc != 0:
            raise ValueError("oracle_decode rejected its arguments")
        return out

    def kv_append(self, k_src, v_src, k_cache, v_cache, batch, kv_heads,
                  head_dim, max_seq, position) -> None:
        """Write the new K and V rows into the caches at ``position`` (in place)."""
        n_cache = batch * kv_heads * max_seq * head_dim
        n_src = batch * kv_heads * head_dim
        if k_cache.size < n_cache or v_cache.size < n_cache:
            raise ValueError("cache arrays smaller than the stated shape")
        if k_src.size < n_src or v_src.size < n_src:
            raise ValueError("source arrays smaller than the stated shape")
        rc = self._lib.oracle_kv_append(
            _f32(k_src, "k_src"), _f32(v_src, "v_src"),
            _f32(k_cache, "k_cache", True), _f32(v_cache, "v_cache", True),
            batch, kv_heads, head_dim, max_seq, position)
        if rc != 0:
            raise ValueError("oracle_kv_append rejected its arguments")


    def kv_append_rows(self, k_src, v_src, k_cache, v_cache, m, kv_stride, kv_heads,
                       head_dim, max_seq, position) -> None:
        """Write m prefill rows ([m, kv_stride] packed K/V) into one sequence's
        caches ([kv_heads, max_seq, head_dim]) from row ``position`` on."""
        n_cache = kv_heads * max_seq * head_dim
        if k_cache.size < n_cache or v_cache.size < n_cache:
            raise ValueError("cache arrays smaller than the stated shape")
        if m and (k_src.size < (m - 1) * kv_stride + kv_heads * head_dim
                  or v_src.size < (m - 1) * kv_stride + kv_heads * head_dim):
            raise ValueError("source arrays smaller than the stated shape")
        rc = self._lib.oracle_kv_append_rows(
            _f32(k_src, "k_src"), _f32(v_src, "v_src"),
            _f32(k_cache, "k_cache", True), _f32(v_cache, "v_cache", True),
            m, kv_stride, kv_heads, head_dim, max_seq, position)
        if rc != 0:
            raise ValueError("oracle_kv_append_rows rejected its arguments")

    def decode_varlen(self, q, k_cache, v_cache, seq_lens, batch, num_heads, kv_heads,
                      head_dim, max_seq, window, scale):
        """Decode with per-sequence lengths ``seq_lens`` ([batch] ints); a
        length-0 sequence gives zeros. Returns [B, Hq, d] float64."""
        n_cache = batch * kv_heads * max_seq * head_dim
        if (q.size < batch * num_heads * head_dim or k_cache.size < n_cache
                or v_cache.size < n_cache):
            raise ValueError("input arrays smaller than the stated shapes")
        lens = np.ascontiguousarray(seq_lens, dtype=np.uint32)
        if lens.size < batch:
            raise ValueError("seq_lens shorter than the batch")
        out = np.empty((batch, num_heads, head_dim), dtype=np.float64)
        rc = self._lib.oracle_decode_varlen(
            _f32(q, "q"), _f32(k_cache, "k_cache"), _f32(v_cache, "v_cache"),
            lens.ctypes.data_as(_U32P), batch, num_heads, kv_heads, head_dim, max_seq,
            window, ctypes.c_float(scale), out.ctypes.data_as(_F64P))
        if rc != 0:
            raise ValueError("oracle_decode_varlen rejected its arguments")
        return out

    def rope(self, x, cos_t, sin_t):
        """Rotate-half rotary embedding of the rows of x ([..., d] float32)
        with per-pair cos/sin ([d/2] float32); returns float64."""
        d = x.shape[-1]
        if cos_t.size < d // 2 or sin_t.size < d // 2:
            raise ValueError("cos/sin need d/2 entries")
        out = np.empty(x.shape, dtype=np.float64)
        rc = self._lib.oracle_rope(_f32(np.ascontiguousarray(x), "x"), _f32(cos_t, "cos_t"),
                                   _f32(sin_t, "sin_t"), x.size // d, d,
                                   out.ctypes.data_as(_F64P))
        if rc != 0:
            raise ValueError("oracle_rope rejected its arguments")
        return out

    def decode_rope_append(self, q_raw, k_raw, v_raw, cos_t, sin_t, k_cache, v_cache,
                           batch, num_heads, kv_heads, head_dim, max_seq, position,
                           window, scale):
        """Fused decode step with rotary embedding; updates the caches in
        place (rotated K, raw V at `position`) and returns [B, Hq, d] fp64."""
        n_cache = batch * kv_heads * max_seq * head_dim
        if k_cache.size < n_cache or v_cache.size < n_cache:
            raise ValueError("cache arrays smaller than the stated shape")
        out = np.empty((batch, num_heads, head_dim), dtype=np.float64)
        rc = self._lib.oracle_decode_rope_append(
            _f32(q_raw, "q_raw"), _f32(k_raw, "k_raw"), _f32(v_raw, "v_raw"),
            _f32(cos_t, "cos_t"), _f32(sin_t, "sin_t"), _f32(k_cache, "k_cache", True),
            _f32(v_cache, "v_cache", True), batch, num_heads, kv_heads, head_dim,
            max_seq, position, window, ctypes.c_float(scale), out.ctypes.data_as(_F64P))
        if rc != 0:
            raise ValueError("oracle_decode_rope_append rejected its arguments")
        return out


_default = None


def default() -> Oracle:
    """The oracle built from this directory's oracle.c (compiled on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(SO_PATH):
            build()
        _default = Oracle(SO_PATH)
    return _default


def num_threads() -> int:
    return default().num_threads()


def prefill_scale(head_dim: int) -> float:
    return default().prefill_scale(head_dim)


def prefill_causal(*args, **kw) -> np.ndarray:
    return default().prefill_causal(*args, **kw)


def decode(*args, **kw) -> np.ndarray:
    return default().decode(*args, **kw)


def kv_append(*args, **kw) -> None:
    return default().kv_append(*args, **kw)


def kv_append_rows(*args, **kw) -> None:
    return default().kv_append_rows(*args, **kw)


def decode_varlen(*args, **kw) -> np.ndarray:
    return default().decode_varlen(*args, **kw)


def rope(*args, **kw) -> np.ndarray:
    return default().rope(*args, **kw)


def decode_rope_append(*args, **kw) -> np.ndarray:
    return default().decode_rope_append(*args, **kw)
