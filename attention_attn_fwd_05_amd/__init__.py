"""Fused attention forward + KV-cache decode for AMD MI355X (gfx950).

A thin ctypes binding over ``libattn.so`` (C ABI in include/attn.h).  Every
step of the computation runs in the library's HIP kernels; this module only
marshals torch tensors into pointers, element strides and the current HIP
stream.  There is no fallback: if the library is missing or fails to load,
every call raises.

Entry points (same names as the C ABI):

* ``attn_fwd(q, k, v, *, causal, scale=None, return_lse=False, out=None,
  causal_align="top_left", window=None)`` (``window=(left, right)``: a
  sliding-window band, through attn_fwd_masked)
* ``attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q=None, *,
  causal, ...)`` (packed sequences of different lengths, offsets on the device)
* ``attn_decode(q, k_cache, v_cache, cache_len, *, scale=None, workspace=None,
  num_splits=0, return_lse=False, out=None, window_left=-1)`` (every decode
  form takes ``window_left``, through attn_decode_ex)
* ``attn_decode_varlen(q, k_cache, v_cache, cache_lens, max_cache_len=None, ...)``
  (one cache length per sequence, read on the device)
* ``attn_decode_noalloc(q, k_cache, v_cache, cache_len, *, out, lse=None, ...)``
  (attn_decode with the library's own fixed scratch: allocates nothing)
* ``attn_decode_workspace_bytes(B, Hq, Hkv, S_max, D)`` /
  ``decode_workspace(...)`` (a uint8 scratch tensor of that size)
* ``kv_cache_write(k_cache, v_cache, k_new, v_new, pos)``
* ``attn_bwd(q, k, v, o, dout, lse, *, causal, ...)`` -> (dq, dk, dv), the
  backward of attn_fwd (GQA gradients summed over each group)
* ``attn_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k, ...)``
  -> (dq, dk, dv), the backward of attn_fwd_varlen
* ``attn_decode_paged(q, k_pages, v_pages, block_table, cache_lens, ...)`` and
  ``kv_cache_write_paged(k_pages, v_pages, k_new, v_new, block_table, pos)``
  (a paged KV cache addressed through a device block table)
"""

from ._binding import (  # noqa: F401
    AttnError,
    Status,
    attn_bwd,
    attn_bwd_varlen,
    attn_decode,
    attn_decode_noalloc,
    attn_decode_paged,
    attn_decode_varlen,
    attn_decode_workspace_bytes,
    attn_fwd,
    attn_fwd_varlen,
    decode_workspace,
    kv_cache_write,
    kv_cache_write_paged,
    lib_path,
    load_library,
)

__all__ = [
    "AttnError",
    "Status",
    "attn_fwd",
    "attn_bwd",
    "attn_bwd_varlen",
    "attn_fwd_varlen",
    "attn_decode",
    "attn_decode_noalloc",
    "attn_decode_varlen",
    "attn_decode_paged",
    "kv_cache_write_paged",
    "attn_decode_workspace_bytes",
    "decode_workspace",
    "kv_cache_write",
    "lib_path",
    "load_library",
]
