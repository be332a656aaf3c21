"""Fused grouped-query attention on AMD Instinct MI355X (gfx950).

Thin ctypes binding of ``libattn.so`` (declared in ``include/attn.h``). The
functions carry the C entry points' names and arguments; this module only
turns torch tensors into device pointers, picks the current HIP stream, and
raises on a non-OK status. Every step of the computation runs in the HIP
kernels; there is no other code path. If the library has not been built the
import still succeeds, but the first call raises.

    attn_prefill_causal(q, k, v, o, m, q_stride, kv_stride, num_q_heads,
                        heads_per_kv, head_dim, stream=None)
    attn_decode_workspace_bytes(batch, num_heads, kv_heads, head_dim,
                                total_seq, window) -> int
    attn_decode(q, k_cache, v_cache, out, batch, num_heads, kv_heads, head_dim,
                max_seq, total_seq, window, scale, workspace,
                workspace_bytes=None, stream=None)
    kv_append(k_src, v_src, k_cache, v_cache, batch, kv_heads, head_dim,
              max_seq, position, stream=None)
    attn_decode_append(q, k_new, v_new, k_cache, v_cache, out, batch,
                       num_heads, kv_heads, head_dim, max_seq, position,
                       window, scale, workspace, workspace_bytes=None,
                       stream=None)
    attn_decode_rope_append(q_raw, k_raw, v_raw, cos_t, sin_t, k_cache,
                            v_cache, out, batch, num_heads, kv_heads,
                            head_dim, max_seq, position, window, scale,
                            workspace, workspace_bytes=None, stream=None)
    attn_decode_append_noalloc(q, k_new, v_new, k_cache, v_cache, out, batch,
                               num_heads, kv_heads, head_dim, max_seq,
                               position, window, scale, stream=None)
    kv_append_rows(k_src, v_src, k_cache, v_cache, m, kv_stride, kv_heads,
                   head_dim, max_seq, position, stream=None)
    attn_decode_varlen(q, k_cache, v_cache, out, seq_lens, batch, num_heads,
                       kv_heads, head_dim, max_seq, seq_bound, window, scale,
                       workspace, workspace_bytes=None, stream=None)
    attn_decode_append_varlen(q, k_new, v_new, k_cache, v_cache, out,
                              positions, batch, num_heads, kv_heads, head_dim,
                              max_seq, seq_bound, window, scale, workspace,
                              workspace_bytes=None, stream=None)
    attn_decode_rope_append_varlen(q_raw, k_raw, v_raw, cos_t, sin_t, k_cache,
                                   v_cache, out, positions, batch, num_heads,
                                   kv_heads, head_dim, max_seq, seq_bound,
                                   window, scale, workspace,
                                   workspace_bytes=None, stream=None)
    attn_status_string(status) -> str

Tensor arguments may be torch tensors (their ``data_ptr()`` is passed, and
their size is checked against the stated shape) or plain integer device
addresses (passed as they are).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "AttnError", "ATTN_OK", "ATTN_ERR_INVALID", "ATTN_ERR_UNSUPPORTED",
    "ATTN_ERR_HIP", "SO_PATH", "library", "attn_prefill_causal",
    "attn_decode_workspace_bytes", "attn_decode", "kv_append",
    "attn_decode_append", "attn_decode_rope_append", "attn_decode_append_noalloc",
    "kv_append_rows",
    "attn_decode_varlen", "attn_decode_append_varlen", "attn_decode_rope_append_varlen",
    "attn_status_string", "decode_workspace",
]

# ATTN_GQA_LIB names another build of the library (an instrumented one, say)
SO_PATH = os.environ.get("ATTN_GQA_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3

EXPORTS = ("attn_prefill_causal", "attn_decode_workspace_bytes", "attn_decode",
           "kv_append", "attn_decode_append", "attn_decode_rope_append",
           "attn_decode_append_noalloc",
           "kv_append_rows", "attn_decode_varlen", "attn_decode_append_varlen",
           "attn_decode_rope_append_varlen", "attn_status_string")


class AttnError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func}: {attn_status_string(status)} (status {status})")


_lib = None
_u32 = ctypes.c_uint32
_vp = ctypes.c_void_p


def library() -> ctypes.CDLL:
    """The loaded libattn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(SO_PATH):
            raise RuntimeError(
                f"{SO_PATH} is missing: build it with "
                "`python -m attention_gqa_online_amd.build` (hipcc, gfx950)")
        # torch first: it loads its own HIP runtime (soname libamdhip64.so.7,
        # the name libattn.so asks for), so the library binds to that same
        # runtime. Loaded the other way round, the process would hold two
        # HIP runtimes, and the second to start finds no device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(SO_PATH)
        lib.attn_prefill_causal.restype = ctypes.c_int
        lib.attn_prefill_causal.argtypes = [_vp, _vp, _vp, _vp, _u32, _u32, _u32,
                                            _u32, _u32, _u32, _vp]
        lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.attn_decode_workspace_bytes.argtypes = [_u32] * 6
        lib.attn_decode.restype = ctypes.c_int
        lib.attn_decode.argtypes = [_vp, _vp, _vp, _vp, _u32, _u32, _u32, _u32,
                                    _u32, _u32, _u32, ctypes.c_float, _vp,
                                    ctypes.c_size_t, _vp]
        lib.kv_append.restype = ctypes.c_int
        lib.kv_append.argtypes = [_vp, _vp, _vp, _vp, _u32, _u32, _u32, _u32,
                                  _u32, _vp]
        lib.attn_decode_append.restype = ctypes.c_int
        lib.attn_decode_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _u32, _u32, _u32,
                                           _u32, _u32, _u32, _u32, ctypes.c_float, _vp,
                                           ctypes.c_size_t, _vp]
        lib.attn_decode_rope_append.restype = ctypes.c_int
        lib.attn_decode_rope_append.argtypes = [_vp] * 8 + [_u32] * 7 + [
            ctypes.c_float, _vp, ctypes.c_size_t, _vp]
        lib.attn_decode_append_noalloc.restype = ctypes.c_int
        lib.attn_decode_append_noalloc.argtypes = [_vp] * 6 + [_u32] * 7 + [ctypes.c_float, _vp]
        lib.kv_append_rows.restype = ctypes.c_int
        lib.kv_append_rows.argtypes = [_vp] * 4 + [_u32] * 6 + [_vp]
        lib.attn_decode_varlen.restype = ctypes.c_int
        lib.attn_decode_varlen.argtypes = [_vp] * 5 + [_u32] * 7 + [
            ctypes.c_float, _vp, ctypes.c_size_t, _vp]
        lib.attn_decode_append_varlen.restype = ctypes.c_int
        lib.attn_decode_append_varlen.argtypes = [_vp] * 7 + [_u32] * 7 + [
            ctypes.c_float, _vp, ctypes.c_size_t, _vp]
        lib.attn_decode_rope_append_varlen.restype = ctypes.c_int
        lib.attn_decode_rope_append_varlen.argtypes = [_vp] * 9 + [_u32] * 7 + [
            ctypes.c_float, _vp, ctypes.c_size_t, _vp]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_status_string.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(x, name: str, min_elems: int = 0):
    """Device address of a torch tensor (size-checked) or an int address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor or an int address")
    want = {"workspace": None, "seq_lens": torch.int32, "positions": torch.int32}.get(
        name, torch.float32)
    if want is not None and x.dtype != want:
        raise TypeError(f"{name}: expected {want}, got {x.dtype}")
    if not x.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if x.numel() < min_elems:
        raise ValueError(f"{name}: has {x.numel()} elements, needs {min_elems}")
    return x.data_ptr() or None


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(func: str, status: int) -> None:
    if status != ATTN_OK:
        raise AttnError(func, status)


def attn_status_string(status: int) -> str:
    return library().attn_status_string(int(status)).decode()


def attn_prefill_causal(q, k, v, o, m, q_stride, kv_stride, num_q_heads,
                        heads_per_kv, head_dim, stream=None) -> None:
    """Causal GQA prefill; Q/O ``[m, q_stride]``, K/V ``[m, kv_stride]``."""
    st = library().attn_prefill_causal(
        _ptr(q, "q", m * q_stride), _ptr(k, "k", m * kv_stride),
        _ptr(v, "v", m * kv_stride), _ptr(o, "o", m * q_stride),
        m, q_stride, kv_stride, num_q_heads, heads_per_kv, head_dim,
        _stream(stream))
    _check("attn_prefill_causal", st)


def attn_decode_workspace_bytes(batch, num_heads, kv_heads, head_dim,
                                total_seq, window) -> int:
    return int(library().attn_decode_workspace_bytes(
        batch, num_heads, kv_heads, head_dim, total_seq, window))


def decode_workspace(batch, num_heads, kv_heads, head_dim, total_seq, window,
                     device=None):
    """A zero-filled uint8 workspace tensor sized for these decode shapes
    (the arrival counters at its start must be zero before the first call;
    every call leaves them at zero)."""
    import torch
    n = attn_decode_workspace_bytes(batch, num_heads, kv_heads, head_dim,
                                    total_seq, window)
    if n == 0:
        raise ValueError("invalid decode shapes")
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def attn_decode(q, k_cache, v_cache, out, batch, num_heads, kv_heads, head_dim,
                max_seq, total_seq, window, scale, workspace,
                workspace_bytes=None, stream=None) -> None:
    """Single-query GQA decode with optional sliding window."""
    n_cache = batch * kv_heads * max_seq * head_dim
    if workspace_bytes is None:
        import torch
        if not isinstance(workspace, torch.Tensor):
            raise ValueError("workspace_bytes is required for an int workspace")
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = library().attn_decode(
        _ptr(q, "q", batch * num_heads * head_dim), _ptr(k_cache, "k_cache", n_cache),
        _ptr(v_cache, "v_cache", n_cache), _ptr(out, "out", batch * num_heads * head_dim),
        batch, num_heads, kv_heads, head_dim, max_seq, total_seq, window,
        float(scale), _ptr(workspace, "workspace"), int(workspace_bytes),
        _stream(stream))
    _check("attn_decode", st)


def kv_append(k_src, v_src, k_cache, v_cache, batch, kv_heads, head_dim,
              max_seq, position, stream=None) -> None:
    """Write the new K and V rows of every (sequence, KV head) at ``position``."""
    n_src = batch * kv_heads * head_dim
    n_cache = batch * kv_heads * max_seq * head_dim
    st = library().kv_append(
        _ptr(k_src, "k_src", n_src), _ptr(v_src, "v_src", n_src),
        _ptr(k_cache, "k_cache", n_cache), _ptr(v_cache, "v_cache", n_cache),
        batch, kv_heads, head_dim, max_seq, position, _stream(stream))
    _check("kv_append", st)


def _workspace_bytes(workspace, workspace_bytes):
    if workspace_bytes is not None:
        return workspace_bytes
    import torch
    if workspace is None:
        return 0
    if isinstance(workspace, torch.Tensor):
        return workspace.numel() * workspace.element_size()
    raise ValueError("workspace_bytes is required for an int workspace")


def attn_decode_append(q, k_new, v_new, k_cache, v_cache, out, batch, num_heads,
                       kv_heads, head_dim, max_seq, position, window, scale,
                       workspace, workspace_bytes=None, stream=None) -> None:
    """Append the current token's K/V rows at ``position`` and decode over
    ``[w0, position]`` (one decode step)."""
    n_src = batch * kv_heads * head_dim
    n_cache = batch * kv_heads * max_seq * head_dim
    workspace_bytes = _workspace_bytes(workspace, workspace_bytes)
    st = library().attn_decode_append(
        _ptr(q, "q", batch * num_heads * head_dim), _ptr(k_new, "k_new", n_src),
        _ptr(v_new, "v_new", n_src), _ptr(k_cache, "k_cache", n_cache),
        _ptr(v_cache, "v_cache", n_cache), _ptr(out, "out", batch * num_heads * head_dim),
        batch, num_heads, kv_heads, head_dim, max_seq, position, window, float(scale),
        _ptr(workspace, "workspace"), int(workspace_bytes), _stream(stream))
    _check("attn_decode_append", st)


def attn_decode_rope_append(q_raw, k_raw, v_raw, cos_t, sin_t, k_cache, v_cache,
                            out, batch, num_heads, kv_heads, head_dim, max_seq,
                            position, window, scale, workspace,
                            workspace_bytes=None, stream=None) -> None:
    """One decode step with rotate-half rotary embedding: rotate q and the
    new K rows by ``cos_t``/``sin_t`` (``[head_dim/2]``, the angles at
    ``position``), append rotated K and raw V at ``position``, and decode."""
    n_src = batch * kv_heads * head_dim
    n_cache = batch * kv_heads * max_seq * head_dim
    workspace_bytes = _workspace_bytes(workspace, workspace_bytes)
    st = library().attn_decode_rope_append(
        _ptr(q_raw, "q_raw", batch * num_heads * head_dim), _ptr(k_raw, "k_raw", n_src),
        _ptr(v_raw, "v_raw", n_src), _ptr(cos_t, "cos_t", head_dim // 2),
        _ptr(sin_t, "sin_t", head_dim // 2), _ptr(k_cache, "k_cache", n_cache),
        _ptr(v_cache, "v_cache", n_cache), _ptr(out, "out", batch * num_heads * head_dim),
        batch, num_heads, kv_heads, head_dim, max_seq, position, window, float(scale),
        _ptr(workspace, "workspace"), int(workspace_bytes), _stream(stream))
    _check("attn_decode_rope_append", st)


def attn_decode_append_noalloc(q, k_new, v_new, k_cache, v_cache, out, batch, num_heads,
                               kv_heads, head_dim, max_seq, position, window, scale,
                               stream=None) -> None:
    """attn_decode_append with the library's own per-GPU workspace array (no
    workspace argument, nothing allocated); calls on one GPU must not overlap."""
    n_src = batch * kv_heads * head_dim
    n_cache = batch * kv_heads * max_seq * head_dim
    st = library().attn_decode_append_noalloc(
        _ptr(q, "q", batch * num_heads * head_dim), _ptr(k_new, "k_new", n_src),
        _ptr(v_new, "v_new", n_src), _ptr(k_cache, "k_cache", n_cache),
        _ptr(v_cache, "v_cache", n_cache), _ptr(out, "out", batch * num_heads * head_dim),
        batch, num_heads, kv_heads, head_dim, max_seq, position, window, float(scale),
        _stream(stream))
    _check("attn_decode_append_noalloc", st)


def kv_append_rows(k_src, v_src, k_cache, v_cache, m, kv_stride, kv_heads, head_dim,
                   max_seq, position, stream=None) -> None:
    """Write m prefill rows of packed K/V (``[m, kv_stride]``) into one
    sequence's caches (``[kv_heads, max_seq, head_dim]``) from ``position``."""
    n_src = (m - 1) * kv_stride + kv_heads * head_dim if m else 0
    n_cache = kv_heads * max_seq * head_dim
    st = library().kv_append_rows(
        _ptr(k_src, "k_src", n_src), _ptr(v_src, "v_src", n_src),
        _ptr(k_cache, "k_cache", n_cache), _ptr(v_cache, "v_cache", n_cache),
        m, kv_stride, kv_heads, head_dim, max_seq, position, _stream(stream))
    _check("kv_append_rows", st)


def attn_decode_varlen(q, k_cache, v_cache, out, seq_lens, batch, num_heads, kv_heads,
                       head_dim, max_seq, seq_bound, window, scale, workspace,
                       workspace_bytes=None, stream=None) -> None:
    """Decode with per-sequence lengths ``seq_lens`` (int32 device tensor,
    read as uint32), each at most ``seq_bound``."""
    n_cache = batch * kv_heads * max_seq * head_dim
    workspace_bytes = _workspace_bytes(workspace, workspace_bytes)
    st = library().attn_decode_varlen(
        _ptr(q, "q", batch * num_heads * head_dim), _ptr(k_cache, "k_cache", n_cache),
        _ptr(v_cache, "v_cache", n_cache), _ptr(out, "out", batch * num_heads * head_dim),
        _ptr(seq_lens, "seq_lens", batch), batch, num_heads, kv_heads, head_dim, max_seq,
        seq_bound, window, float(scale), _ptr(workspace, "workspace"), int(workspace_bytes),
        _stream(stream))
    _check("attn_decode_varlen", st)


def attn_decode_append_varlen(q, k_new, v_new, k_cache, v_cache, out, positions, batch,
                              num_heads, kv_heads, head_dim, max_seq, seq_bound, window,
                              scale, workspace, workspace_bytes=None, stream=None) -> None:
    """Decode step with per-sequence positions (int32 device tensor, read as
    uint32): sequence b appends at positions[b] and attends up to it."""
    n_src = batch * kv_heads * head_dim
    n_cache = batch * kv_heads * max_seq * head_dim
    workspace_bytes = _workspace_bytes(workspace, workspace_bytes)
    st = library().attn_decode_append_varlen(
        _ptr(q, "q", batch * num_heads * head_dim), _ptr(k_new, "k_new", n_src),
        _ptr(v_new, "v_new", n_src), _ptr(k_cache, "k_cache", n_cache),
        _ptr(v_cache, "v_cache", n_cache), _ptr(out, "out", batch * num_heads * head_dim),
        _ptr(positions, "positions", batch), batch, num_heads, kv_heads, head_dim, max_seq,
        seq_bound, window, float(scale), _ptr(workspace, "workspace"), int(workspace_bytes),
        _stream(stream))
    _check("attn_decode_append_varlen", st)


def attn_decode_rope_append_varlen(q_raw, k_raw, v_raw, cos_t, sin_t, k_cache, v_cache, out,
                                   positions, batch, num_heads, kv_heads, head_dim, max_seq,
                                   seq_bound, window, scale, workspace, workspace_bytes=None,
                                   stream=None) -> None:
    """Rotary decode step with per-sequence positions (int32 device tensor,
    read as uint32) and per-sequence tables ``cos_t``/``sin_t``
    (``[batch, head_dim/2]``, row b for positions[b])."""
    n_src = batch * kv_heads * head_dim
    n_cache = batch * kv_heads * max_seq * head_dim
    n_tab = batch * (head_dim // 2)
    workspace_bytes = _workspace_bytes(workspace, workspace_bytes)
    st = library().attn_decode_rope_append_varlen(
        _ptr(q_raw, "q_raw", batch * num_heads * head_dim), _ptr(k_raw, "k_raw", n_src),
        _ptr(v_raw, "v_raw", n_src), _ptr(cos_t, "cos_t", n_tab), _ptr(sin_t, "sin_t", n_tab),
        _ptr(k_cache, "k_cache", n_cache), _ptr(v_cache, "v_cache", n_cache),
        _ptr(out, "out", batch * num_heads * head_dim), _ptr(positions, "positions", batch),
        batch, num_heads, kv_heads, head_dim, max_seq, seq_bound, window, float(scale),
        _ptr(workspace, "workspace"), int(workspace_bytes), _stream(stream))
    _check("attn_decode_rope_append_varlen", st)
