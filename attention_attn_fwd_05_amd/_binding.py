"""ctypes marshalling for libattn.so.  No computation happens here."""

from __future__ import annotations

import ctypes
import enum
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))


class Status(enum.IntEnum):
    OK = 0
    ERR_NULL = 1
    ERR_SHAPE = 2
    ERR_UNSUPPORTED = 3
    ERR_WORKSPACE = 4
    ERR_HIP = 5


class AttnError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = Status(status)


class Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64), ("d", ctypes.c_int64)]


class Mask(ctypes.Structure):
    _fields_ = [("align", ctypes.c_int32), ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32)]


class DecodeOpts(ctypes.Structure):
    _fields_ = [("cache_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("max_pages_per_seq", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("window_left", ctypes.c_int32)]


_DTYPES = {torch.float16: 0, torch.bfloat16: 1}
_LIB = None


def lib_path() -> str:
    return os.path.join(_PKG, "libattn.so")


def load_library():
    """Load libattn.so once; raise if it is missing (there is no fallback path)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python __graft_entry__.py build)")
    lib = ctypes.CDLL(path)
    vp, i32, f32, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, Strides
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, S, S, S, S, f32, i32, i32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_fwd_masked.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, S, S, S, S, f32, Mask, i32, vp]
    lib.attn_fwd_masked.restype = i32
    lib.attn_fwd_varlen_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, S, S, S, S,
                                           f32, Mask, i32, vp]
    lib.attn_fwd_varlen_masked.restype = i32
    lib.attn_decode_ex.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, S, S, S, S, f32, i32, i32,
                                   ctypes.POINTER(DecodeOpts), vp, ctypes.c_size_t, vp]
    lib.attn_decode_ex.restype = i32
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, S, S, S, S, f32,
                                    i32, i32, vp]
    lib.attn_fwd_varlen.restype = i32
    lib.attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, S, S, S, S, f32, i32, i32,
                                vp, ctypes.c_size_t, vp]
    lib.attn_decode.restype = i32
    lib.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, S, S, S, S, f32, i32, i32,
                                        vp]
    lib.attn_decode_noalloc.restype = i32
    lib.attn_decode_varlen.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32, i32, S, S, S, S, f32, i32,
                                       i32, vp, ctypes.c_size_t, vp]
    lib.attn_decode_varlen.restype = i32
    lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, vp, i32, i32,
                                      S, S, S, S, f32, i32, i32, vp, ctypes.c_size_t, vp]
    lib.attn_decode_paged.restype = i32
    lib.kv_cache_write_paged.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, i32, vp, i32, i32, S, S, S, S,
                                         i32, vp]
    lib.kv_cache_write_paged.restype = i32
    lib.attn_bwd_workspace_bytes.argtypes = [i32, i32, i32]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, S, S, S, S, S, S, S, S,
                             f32, i32, i32, vp, ctypes.c_size_t, vp]
    lib.attn_bwd.restype = i32
    lib.attn_bwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, S, S, S, S, S, S,
                                    S, S, f32, Mask, i32, vp, ctypes.c_size_t, vp]
    lib.attn_bwd_masked.restype = i32
    lib.attn_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    i32, S, S, S, S, S, S, S, S, f32, i32, i32, vp, ctypes.c_size_t, vp]
    lib.attn_bwd_varlen.restype = i32
    lib.attn_bwd_varlen_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                           i32, i32, S, S, S, S, S, S, S, S, f32, Mask, i32, vp, ctypes.c_size_t, vp]
    lib.attn_bwd_varlen_masked.restype = i32
    lib.kv_cache_write.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, S, S, S, S, i32, vp]
    lib.kv_cache_write.restype = i32
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _check(status: int, fn: str):
    if status != 0:
        lib = load_library()
        raise AttnError(status, fn, lib.attn_status_string(status).decode())


def _strides4(t: torch.Tensor) -> Strides:
    s = t.stride()
    return Strides(s[0], s[1], s[2], s[3])


def _strides3(t: torch.Tensor) -> Strides:
    s = t.stride()
    return Strides(s[0], s[1], 0, s[2])


def _dtype_code(*ts: torch.Tensor) -> int:
    dt = ts[0].dtype
    if dt not in _DTYPES or any(t.dtype != dt for t in ts):
        raise TypeError("q/k/v (and out) must share one dtype, float16 or bfloat16")
    return _DTYPES[dt]


def _on_gpu(*ts: torch.Tensor):
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda or t.device != dev:
            raise ValueError("all tensors must be on the same GPU")


def _nbytes(ws: torch.Tensor) -> int:
    """Size in bytes of a caller's workspace tensor, which must be one contiguous block."""
    if not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")
    return ws.numel() * ws.element_size()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


_CAUSAL_ALIGN = {"top_left": 1, "bottom_right": 2}
_ALIGN = {"top_left": 0, "bottom_right": 1}


def _mask(causal: bool, causal_align: str, window) -> Mask:
    """attn_mask for a sliding window (left, right) around each query's
    diagonal position (-1 leaves a side open); ``causal`` closes the right side
    at the diagonal."""
    left, right = (int(window[0]), int(window[1]))
    if left < -1 or right < -1:
        raise ValueError("window sides must be >= -1")
    if causal:
        if right > 0:
            raise ValueError("a causal mask has no keys right of the diagonal: window right must be -1 or 0")
        right = 0
    return Mask(_ALIGN[causal_align], left, right)


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool, scale: float | None = None,
             return_lse: bool = False, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
             causal_align: str = "top_left", window=None):
    """Fused attention forward.  q (B,Hq,Nq,D), k/v (B,Hkv,Nkv,D), any strides with stride(-1) == 1.

    ``causal_align`` (when ``causal``): "top_left" -- query i sees keys j <= i;
    "bottom_right" -- j <= i + Nkv - Nq (the queries are the last Nq positions).
    ``window=(left, right)``: a sliding window around each query's diagonal
    position p (keys p - left .. p + right, -1 leaves a side open), aligned by
    ``causal_align``; calls attn_fwd_masked.
    Returns ``out`` (B,Hq,Nq,D), or ``(out, lse)`` with lse fp32 (B,Hq,Nq) when ``return_lse``.
    """
    if causal_align not in _CAUSAL_ALIGN:
        raise ValueError("causal_align must be 'top_left' or 'bottom_right'")
    lib = load_library()
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty((B, Hq, Nq, D), dtype=q.dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, Hq, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq, Nq)")
    _on_gpu(q, k, v, out, *([lse] if lse is not None else []))
    code = _dtype_code(q, k, v, out)
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D or out.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v and out")
    s = _default_scale(D) if scale is None else float(scale)
    if window is not None:
        st = lib.attn_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr() if lse is not None else None,
                                 B, Hq, Hkv, Nq, Nkv, D, _strides4(q), _strides4(k), _strides4(v), _strides4(out),
                                 s, _mask(causal, causal_align, window), code, _stream(q))
        _check(st, "attn_fwd_masked")
        return (out, lse) if return_lse else out
    st = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                      lse.data_ptr() if lse is not None else None,
                      B, Hq, Hkv, Nq, Nkv, D, _strides4(q), _strides4(k), _strides4(v), _strides4(out),
                      s, _CAUSAL_ALIGN[causal_align] if causal else 0, code, _stream(q))
    _check(st, "attn_fwd")
    return (out, lse) if return_lse else out


def _strides_packed(t: torch.Tensor) -> Strides:
    s = t.stride()
    return Strides(0, s[1], s[0], s[2])


def attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                    cu_seqlens_k: torch.Tensor, max_seqlen_q: int | None = None, *, causal: bool,
                    scale: float | None = None, return_lse: bool = False, out: torch.Tensor | None = None,
                    lse: torch.Tensor | None = None, causal_align: str = "top_left", window=None):
    """Fused attention forward over packed sequences of different lengths.

    q (total_q, Hq, D), k/v (total_k, Hkv, D), any strides with stride(-1) == 1;
    cu_seqlens_q / cu_seqlens_k: int32 (B + 1,) device offsets (sequence b owns
    rows [cu[b], cu[b+1])).  ``max_seqlen_q`` bounds every sequence's query
    count; when None it is read from ``cu_seqlens_q`` (a device-to-host copy).
    ``causal_align`` is per sequence ("bottom_right": j <= i + L_k - L_q);
    ``window=(left, right)`` as in ``attn_fwd`` (calls attn_fwd_varlen_masked).
    Returns ``out`` (total_q, Hq, D), or ``(out, lse)`` with lse fp32 (Hq, total_q).
    """
    if causal_align not in _CAUSAL_ALIGN:
        raise ValueError("causal_align must be 'top_left' or 'bottom_right'")
    lib = load_library()
    Tq, Hq, D = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    if k.shape != v.shape or k.shape[2] != D:
        raise ValueError("shape mismatch between q, k and v")
    for cu in (cu_seqlens_q, cu_seqlens_k):
        if cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous 1-D int32 tensors")
    if cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")
    B = cu_seqlens_q.shape[0] - 1
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if B > 0 else 0
        max_seqlen_q = max(max_seqlen_q, 1)
    if out is None:
        out = torch.empty((Tq, Hq, D), dtype=q.dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (Hq, Tq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor of shape (Hq, total_q)")
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _on_gpu(q, k, v, out, cu_seqlens_q, cu_seqlens_k, *([lse] if lse is not None else []))
    code = _dtype_code(q, k, v, out)
    s = _default_scale(D) if scale is None else float(scale)
    if window is not None:
        st = lib.attn_fwd_varlen_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        lse.data_ptr() if lse is not None else None,
                                        cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, int(max_seqlen_q), Tq,
                                        Tk, Hq, Hkv, D, _strides_packed(q), _strides_packed(k), _strides_packed(v),
                                        _strides_packed(out), s, _mask(causal, causal_align, window), code,
                                        _stream(q))
        _check(st, "attn_fwd_varlen_masked")
        return (out, lse) if return_lse else out
    st = lib.attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr() if lse is not None else None,
                             cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, int(max_seqlen_q), Tq, Tk,
                             Hq, Hkv, D, _strides_packed(q), _strides_packed(k), _strides_packed(v),
                             _strides_packed(out), s, _CAUSAL_ALIGN[causal_align] if causal else 0, code,
                             _stream(q))
    _check(st, "attn_fwd_varlen")
    return (out, lse) if return_lse else out


def attn_decode_workspace_bytes(B: int, Hq: int, Hkv: int, S_max: int, D: int) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, Hq, Hkv, S_max, D))


def decode_workspace(B: int, Hq: int, Hkv: int, S_max: int, D: int, device) -> torch.Tensor:
    """Scratch for attn_decode (reusable across calls on one stream; needs no initialisation)."""
    n = attn_decode_workspace_bytes(B, Hq, Hkv, S_max, D)
    if n == 0:
        raise ValueError("invalid decode sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, cache_len: int, *,
                scale: float | None = None, workspace: torch.Tensor | None = None, num_splits: int = 0,
                return_lse: bool = False, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                window_left: int = -1):
    """Decode one token per (batch, q head) over cache slots [0, cache_len).

    ``window_left`` = w >= 0 keeps only the last w + 1 slots (the query is the
    token in slot cache_len - 1); calls attn_decode_ex.

    q (B,Hq,D); caches (B,Hkv,S_max,D).  ``workspace`` is scratch of at least
    ``attn_decode_workspace_bytes`` bytes (see ``decode_workspace``); if omitted
    a fresh one is allocated for this call.
    """
    lib = load_library()
    B, Hq, D = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, Hq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq)")
    if workspace is None:
        workspace = decode_workspace(B, Hq, Hkv, S_max, D, q.device)
    _on_gpu(q, k_cache, v_cache, out, workspace, *([lse] if lse is not None else []))
    code = _dtype_code(q, k_cache, v_cache, out)
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D or out.shape != q.shape:
        raise ValueError("shape mismatch between q, caches and out")
    s = _default_scale(D) if scale is None else float(scale)
    if window_left != -1:
        opts = DecodeOpts(None, None, 0, 0, 0, int(window_left))
        st = lib.attn_decode_ex(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                lse.data_ptr() if lse is not None else None, B, Hq, Hkv, S_max, int(cache_len), D,
                                _strides3(q), _strides4(k_cache), _strides4(v_cache), _strides3(out), s, code,
                                int(num_splits), ctypes.byref(opts), workspace.data_ptr(),
                                _nbytes(workspace), _stream(q))
        _check(st, "attn_decode_ex")
        return (out, lse) if return_lse else out
    st = lib.attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                         lse.data_ptr() if lse is not None else None,
                         B, Hq, Hkv, S_max, int(cache_len), D,
                         _strides3(q), _strides4(k_cache), _strides4(v_cache), _strides3(out),
                         s, code, int(num_splits), workspace.data_ptr(), _nbytes(workspace),
                         _stream(q))
    _check(st, "attn_decode")
    return (out, lse) if return_lse else out


def attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, cache_len: int, *,
                        scale: float | None = None, num_splits: int = 0, out: torch.Tensor,
                        lse: torch.Tensor | None = None):
    """attn_decode without a workspace: the split partials go to the library's
    own fixed scratch, so the call allocates nothing (``out`` and ``lse`` are
    the caller's).  Calls that may overlap on one GPU must be serialised."""
    lib = load_library()
    B, Hq, D = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    if lse is not None and (lse.shape != (B, Hq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq)")
    _on_gpu(q, k_cache, v_cache, out, *([lse] if lse is not None else []))
    code = _dtype_code(q, k_cache, v_cache, out)
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D or out.shape != q.shape:
        raise ValueError("shape mismatch between q, caches and out")
    s = _default_scale(D) if scale is None else float(scale)
    st = lib.attn_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                 lse.data_ptr() if lse is not None else None, B, Hq, Hkv, S_max, int(cache_len), D,
                                 _strides3(q), _strides4(k_cache), _strides4(v_cache), _strides3(out), s, code,
                                 int(num_splits), _stream(q))
    _check(st, "attn_decode_noalloc")
    return out


def attn_decode_varlen(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, cache_lens: torch.Tensor,
                       max_cache_len: int | None = None, *, scale: float | None = None,
                       workspace: torch.Tensor | None = None, num_splits: int = 0, return_lse: bool = False,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None, window_left: int = -1):
    """Decode one token per (batch, q head); batch element b attends over slots [0, cache_lens[b]).

    ``window_left`` = w >= 0 keeps each sequence's last w + 1 slots (attn_decode_ex).

    ``cache_lens``: int32 tensor of B lengths on the same GPU (read by the kernel,
    no host sync; each is clamped to [0, max_cache_len]).  ``max_cache_len``:
    host bound on the lengths that sizes the split grid (default: S_max).
    """
    lib = load_library()
    B, Hq, D = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    if cache_lens.dtype != torch.int32 or cache_lens.shape != (B,) or not cache_lens.is_contiguous():
        raise ValueError("cache_lens must be a contiguous int32 tensor of shape (B,)")
    mcl = S_max if max_cache_len is None else int(max_cache_len)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, Hq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq)")
    if workspace is None:
        workspace = decode_workspace(B, Hq, Hkv, S_max, D, q.device)
    _on_gpu(q, k_cache, v_cache, out, workspace, cache_lens, *([lse] if lse is not None else []))
    code = _dtype_code(q, k_cache, v_cache, out)
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D or out.shape != q.shape:
        raise ValueError("shape mismatch between q, caches and out")
    s = _default_scale(D) if scale is None else float(scale)
    if window_left != -1:
        opts = DecodeOpts(cache_lens.data_ptr(), None, 0, 0, 0, int(window_left))
        st = lib.attn_decode_ex(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                lse.data_ptr() if lse is not None else None, B, Hq, Hkv, S_max, mcl, D,
                                _strides3(q), _strides4(k_cache), _strides4(v_cache), _strides3(out), s, code,
                                int(num_splits), ctypes.byref(opts), workspace.data_ptr(),
                                _nbytes(workspace), _stream(q))
        _check(st, "attn_decode_ex")
        return (out, lse) if return_lse else out
    st = lib.attn_decode_varlen(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                lse.data_ptr() if lse is not None else None,
                                B, Hq, Hkv, S_max, cache_lens.data_ptr(), mcl, D,
                                _strides3(q), _strides4(k_cache), _strides4(v_cache), _strides3(out),
                                s, code, int(num_splits), workspace.data_ptr(),
                                _nbytes(workspace), _stream(q))
    _check(st, "attn_decode_varlen")
    return (out, lse) if return_lse else out


def kv_cache_write(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                   pos: int) -> None:
    """Write k_new/v_new (B,Hkv,T,D) into cache slots [pos, pos+T) of (B,Hkv,S_max,D) caches."""
    lib = load_library()
    _on_gpu(k_cache, v_cache, k_new, v_new)
    code = _dtype_code(k_cache, v_cache, k_new, v_new)
    B, Hkv, S_max, D = k_cache.shape
    T = k_new.shape[2]
    if v_cache.shape != k_cache.shape or k_new.shape != v_new.shape or k_new.shape[:2] != (B, Hkv) \
            or k_new.shape[3] != D:
        raise ValueError("shape mismatch between caches and new rows")
    st = lib.kv_cache_write(k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                            B, Hkv, S_max, D, int(pos), T,
                            _strides4(k_cache), _strides4(v_cache), _strides4(k_new), _strides4(v_new),
                            code, _stream(k_cache))
    _check(st, "kv_cache_write")


def _int32_vec(t: torch.Tensor, n: int, what: str):
    if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{what} must be a contiguous int32 tensor of {n} elements")


def attn_decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                      cache_lens: torch.Tensor, max_cache_len: int | None = None, *, scale: float | None = None,
                      workspace: torch.Tensor | None = None, num_splits: int = 0, return_lse: bool = False,
                      out: torch.Tensor | None = None, lse: torch.Tensor | None = None, window_left: int = -1):
    """Decode over a paged KV cache (``window_left`` as in ``attn_decode_varlen``).

    q (B, Hq, D); k_pages, v_pages (num_pages, Hkv, page_size, D), any strides
    with stride(-1) == 1 (a (num_pages, page_size, Hkv, D) pool passes as
    ``pool.transpose(1, 2)``); block_table int32 (B, max_pages_per_seq);
    cache_lens int32 (B,).  ``max_cache_len`` defaults to
    max_pages_per_seq * page_size.  Returns ``out`` (B, Hq, D), or
    ``(out, lse)`` with lse fp32 (B, Hq).
    """
    lib = load_library()
    B, Hq, D = q.shape
    P, Hkv, ps, Dk = k_pages.shape
    if v_pages.shape != k_pages.shape or Dk != D:
        raise ValueError("page pools must share one shape (num_pages, Hkv, page_size, D) with q's D")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B \
            or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 (B, max_pages_per_seq) tensor")
    _int32_vec(cache_lens, B, "cache_lens")
    mbps = block_table.shape[1]
    if max_cache_len is None:
        max_cache_len = mbps * ps
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, Hq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq)")
    if workspace is None:
        workspace = decode_workspace(B, Hq, Hkv, int(max_cache_len), D, q.device)
    _on_gpu(q, k_pages, v_pages, out, block_table, cache_lens, workspace, *([lse] if lse is not None else []))
    code = _dtype_code(q, k_pages, v_pages, out)
    s = _default_scale(D) if scale is None else float(scale)
    if window_left != -1:
        opts = DecodeOpts(cache_lens.data_ptr(), block_table.data_ptr(), mbps, ps, P, int(window_left))
        st = lib.attn_decode_ex(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), out.data_ptr(),
                                lse.data_ptr() if lse is not None else None, B, Hq, Hkv, 0, int(max_cache_len), D,
                                _strides3(q), _strides4(k_pages), _strides4(v_pages), _strides3(out), s, code,
                                int(num_splits), ctypes.byref(opts), workspace.data_ptr(), _nbytes(workspace),
                                _stream(q))
        _check(st, "attn_decode_ex")
        return (out, lse) if return_lse else out
    st = lib.attn_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), out.data_ptr(),
                               lse.data_ptr() if lse is not None else None, B, Hq, Hkv, P, ps,
                               block_table.data_ptr(), mbps, cache_lens.data_ptr(), int(max_cache_len), D,
                               _strides3(q), _strides4(k_pages), _strides4(v_pages), _strides3(out), s, code,
                               int(num_splits), workspace.data_ptr(), _nbytes(workspace), _stream(q))
    _check(st, "attn_decode_paged")
    return (out, lse) if return_lse else out


def kv_cache_write_paged(k_pages: torch.Tensor, v_pages: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                         block_table: torch.Tensor, pos: torch.Tensor):
    """Store k_new/v_new (B, Hkv, T, D) at slots pos[b] .. pos[b] + T - 1 of each
    sequence of a paged cache (pools as in ``attn_decode_paged``; pos int32 (B,))."""
    lib = load_library()
    P, Hkv, ps, D = k_pages.shape
    B, Hn, T, Dn = k_new.shape
    if v_pages.shape != k_pages.shape or v_new.shape != k_new.shape or Hn != Hkv or Dn != D:
        raise ValueError("shape mismatch between the page pools and the new rows")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B \
            or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 (B, max_pages_per_seq) tensor")
    _int32_vec(pos, B, "pos")
    _on_gpu(k_pages, v_pages, k_new, v_new, block_table, pos)
    code = _dtype_code(k_pages, v_pages, k_new, v_new)
    st = lib.kv_cache_write_paged(k_pages.data_ptr(), v_pages.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                  B, Hkv, P, ps, block_table.data_ptr(), block_table.shape[1], pos.data_ptr(), D, T,
                                  _strides4(k_pages), _strides4(v_pages), _strides4(k_new), _strides4(v_new), code,
                                  _stream(k_pages))
    _check(st, "kv_cache_write_paged")


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
             lse: torch.Tensor, *, causal: bool, scale: float | None = None, causal_align: str = "top_left",
             dq: torch.Tensor | None = None, dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
             workspace: torch.Tensor | None = None, window=None):
    """Gradients (dq, dk, dv) of attn_fwd's output for an upstream gradient ``dout``.

    q, o, dout (B,Hq,Nq,D); k, v (B,Hkv,Nkv,D); lse fp32 (B,Hq,Nq) from attn_fwd
    with the same inputs, mask and scale.  A kv head's dk, dv sum its group's q heads.
    ``window=(left, right)`` as in ``attn_fwd`` (calls attn_bwd_masked).
    """
    if causal_align not in _CAUSAL_ALIGN:
        raise ValueError("causal_align must be 'top_left' or 'bottom_right'")
    lib = load_library()
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    if o.shape != q.shape or dout.shape != q.shape or v.shape != k.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch between q, k, v, o and dout")
    if lse.shape != (B, Hq, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq, Nq)")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("gradient buffers must have the shapes of q, k, v")
    if workspace is None:
        n = int(lib.attn_bwd_workspace_bytes(B, Hq, Nq))
        if n == 0:
            raise ValueError("invalid sizes")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    _on_gpu(q, k, v, o, dout, lse, dq, dk, dv, workspace)
    code = _dtype_code(q, k, v, o, dout, dq, dk, dv)
    s = _default_scale(D) if scale is None else float(scale)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nkv, D,
            _strides4(q), _strides4(k), _strides4(v), _strides4(o), _strides4(dout),
            _strides4(dq), _strides4(dk), _strides4(dv), s)
    tail = (code, workspace.data_ptr(), _nbytes(workspace), _stream(q))
    if window is not None:
        _check(lib.attn_bwd_masked(*args, _mask(causal, causal_align, window), *tail), "attn_bwd_masked")
    else:
        _check(lib.attn_bwd(*args, _CAUSAL_ALIGN[causal_align] if causal else 0, *tail), "attn_bwd")
    return dq, dk, dv


def attn_bwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
                    lse: torch.Tensor, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                    max_seqlen_q: int | None = None, max_seqlen_k: int | None = None, *, causal: bool,
                    scale: float | None = None, causal_align: str = "top_left", dq: torch.Tensor | None = None,
                    dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, window=None):
    """Gradients (dq, dk, dv) of attn_fwd_varlen's output over packed sequences.

    q, o, dout (total_q, Hq, D); k, v (total_k, Hkv, D); lse fp32 (Hq, total_q)
    from attn_fwd_varlen with the same offsets, mask, scale and max_seqlen_q.
    ``max_seqlen_k`` bounds every sequence's key count; either bound, when
    None, is read from its offsets (a device-to-host copy).
    """
    if causal_align not in _CAUSAL_ALIGN:
        raise ValueError("causal_align must be 'top_left' or 'bottom_right'")
    lib = load_library()
    Tq, Hq, D = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    if o.shape != q.shape or dout.shape != q.shape or v.shape != k.shape or k.shape[2] != D:
        raise ValueError("shape mismatch between q, k, v, o and dout")
    for cu in (cu_seqlens_q, cu_seqlens_k):
        if cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous 1-D int32 tensors")
    if cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")
    if lse.shape != (Hq, Tq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape (Hq, total_q)")
    B = cu_seqlens_q.shape[0] - 1

    def _bound(cu):
        return max(int((cu[1:] - cu[:-1]).max().item()) if B > 0 else 0, 1)

    max_seqlen_q = _bound(cu_seqlens_q) if max_seqlen_q is None else int(max_seqlen_q)
    max_seqlen_k = _bound(cu_seqlens_k) if max_seqlen_k is None else int(max_seqlen_k)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("gradient buffers must have the shapes of q, k, v")
    if workspace is None:
        n = int(lib.attn_bwd_workspace_bytes(1, Hq, Tq))
        if n == 0:
            raise ValueError("invalid sizes")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    _on_gpu(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, workspace)
    code = _dtype_code(q, k, v, o, dout, dq, dk, dv)
    s = _default_scale(D) if scale is None else float(scale)
    P = _strides_packed
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
            B, max_seqlen_q, max_seqlen_k, Tq, Tk, Hq, Hkv, D,
            P(q), P(k), P(v), P(o), P(dout), P(dq), P(dk), P(dv), s)
    tail = (code, workspace.data_ptr(), _nbytes(workspace), _stream(q))
    if window is not None:
        _check(lib.attn_bwd_varlen_masked(*args, _mask(causal, causal_align, window), *tail),
               "attn_bwd_varlen_masked")
    else:
        _check(lib.attn_bwd_varlen(*args, _CAUSAL_ALIGN[causal_align] if causal else 0, *tail), "attn_bwd_varlen")
    return dq, dk, dv
