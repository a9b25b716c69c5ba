"""fp64 CPU oracle for fused attention forward, KV-cache decode and the cache write.

TEST INFRASTRUCTURE ONLY.  This module is the checker, not the product: only the
test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it.  It shares no code, constant or helper with
the HIP library and never imports it; the library never imports this.

Sources (three web pages on one subject; cited by title and section):

* [P1] "Skill: Write a Triton Attention Kernel" (ahel.ai catalog).
* [P2] "FlashAttention Kernel Optimization" (the flash-attention-kernel skill page).
* [P3] "Triton-FlashAttention" (project README: GQA/MQA prefill + KV-cache decode).

What is computed.  The tiled, online-softmax kernel of [P1] "Required reasoning
process" reaches, up to rounding order, the plain definition: [P1] "Correctness
requirements" (first bullet) requires O_i / l_i to equal the true softmax-weighted
sum of V, and [P2] "Online Softmax" describes the running-max rescale as a way to
avoid a second pass, not as a different function.  So this oracle is that plain
definition, written out in float64 with numpy (BLAS matmul as the only library
step), in the obvious two-pass form:

    S[i, j]  = scale * sum_d Q[b, h, i, d] * K[b, kvh, j, d]
    vis(i,j) = (j < N_kv) and (not causal or j <= i + off)    causal, off = 0 top-left
    m_i      = max over visible j of S[i, j]
    P[i, j]  = exp(S[i, j] - m_i) / sum over visible j' of exp(S[i, j'] - m_i)
    O[b,h,i] = sum_j P[i, j] * V[b, kvh, j, :]
    lse[b,h,i] = m_i + ln(sum over visible j of exp(S[i, j] - m_i))
    kvh      = h // (H_q // H_kv)                              GQA / MQA

Readings taken where the pages leave a step open (each also listed in the design doc):

* Causal mask is top-left aligned, kv position <= q position ([P1] step 5c; [P2]
  "Common Pitfalls": the comparison is >=, not >).  The widening to
  N_q < N_kv (chunked prefill, multi-token verify against a cache) aligns the
  mask bottom-right: query i is the token at sequence position i + off with
  off = N_kv - N_q, so it sees keys j <= i + off.  The pages fix only the
  top-left form; off = 0 reproduces it exactly.
* ``scale`` multiplies the fp32 dot product; the oracle widens the exact float32
  scale to float64 ([P1] "Inputs" item 4 and "Kernel design rules").
* lse uses the natural log of the sum of exp of *scaled* scores ([P1] step 8).
* A row with no visible key (unreachable with N_kv >= 1 and top-left causal;
  the first N_q - N_kv rows of a bottom-right mask with N_q > N_kv) gets O = 0
  and lse = -inf by convention.
* Decode is one query per (batch, head) over the first ``cache_len`` cache
  slots, every slot visible, no causal loop ([P3] decode phase).  The widening
  to per-sequence lengths (the pages' first deferred scope item) gives batch
  element b its own ``cache_lens[b]``; a length of 0 leaves no visible key.
* GQA maps q head h to kv head h // group, i.e. repeat_interleave expansion of
  K/V, not tiling ([P1] step 1; [P3] GQA phase).
* Paged KV cache (the pages' deferred scope item): cache slot r of sequence b
  lives in page ``block_table[b, r // page_size]``, row ``r % page_size``, of
  the page pools (num_pages, Hkv, page_size, D).  Decode over a paged cache is
  the per-sequence-length decode on the rows so gathered; the paged writer
  stores new rows at slots pos[b], pos[b] + 1, ... of each sequence.
* Sliding windows (the pages' "windowed attention" use case, deferred in
  their scope list): query i sits at key position p = i + offset and sees keys
  j with p - window_left <= j <= p + window_right (-1 leaves a side open); a
  causal mask is window_right = 0.  For packed sequences the window is aligned
  like the causal mask (offset from the sequence's own lengths).  Decode's
  query is the last cached token, so its window keeps the last
  window_left + 1 slots.
* Backward (the pages name it as a separate, later kernel pair and defer GQA
  backward): the gradients of the plain definition with respect to Q, K and V
  for an upstream gradient dO, with the textbook softmax Jacobian
  dS = P * (dP - rowsum(P * dP)), dP = dO V^T; a kv head's dK and dV sum the
  contributions of every q head of its group.
* Packed variable-length prefill (the pages' deferred "varlen" scope item):
  sequence b owns the packed query rows [cu_q[b], cu_q[b+1]) and key rows
  [cu_k[b], cu_k[b+1]); attention never crosses sequences, and each sequence
  is the plain definition above on its own rows, with the causal offset taken
  from its own lengths (0 top-left, L_k - L_q bottom-right).  A sequence with
  no keys gets O = 0 and lse = -inf on its rows.

Pins: tests/test_oracle_pins.py checks this module against closed forms,
hand-derived fixtures (tests/golden/), invariants and an mpmath brute force.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "kv_head_of",
    "visibility",
    "attention_probs",
    "attention_forward",
    "decode",
    "decode_varlen",
    "sequence_bounds",
    "varlen_causal_offset",
    "attention_varlen",
    "kv_cache_write",
    "attention_backward",
    "attention_varlen_backward",
    "page_slot",
    "gather_pages",
    "decode_paged",
    "kv_cache_write_paged",
]


def _f64(x) -> np.ndarray:
    """Exact widening to float64 (fp16, bf16-as-fp32 and fp32 all embed exactly)."""
    a = np.asarray(x)
    return a if a.dtype == np.float64 else a.astype(np.float64)


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by q head ``h``: h // (Hq // Hkv).

    [P1] "Required reasoning process" step 1 and "Kernel design rules" (GQA);
    [P3] GQA/MQA design bullet: MHA is Hkv == Hq, MQA is Hkv == 1, one mapping.
    """
    return h // (Hq // Hkv)


def visibility(q_pos: np.ndarray, Nkv: int, causal: bool, offset: int = 0, window_left: int = -1,
               window_right: int = -1) -> np.ndarray:
    """Boolean (len(q_pos), Nkv): may query at position i attend to key j?

    Keys exist only for j < Nkv ([P1] "Correctness requirements", KV boundary
    bullet).  Query i sits at key position p = i + offset (0 top-left; the
    bottom-right alignment uses offset = Nkv - Nq).  With ``causal`` a key is
    visible when j <= p ([P1] step 5c).  A sliding window ([P1] "Use this
    when": windowed attention) also bounds j to [p - window_left,
    p + window_right]; -1 leaves that side open.
    """
    j = np.arange(Nkv)[None, :]
    p = q_pos[:, None] + offset
    vis = np.ones((q_pos.shape[0], Nkv), dtype=bool)
    if causal:
        vis &= j <= p
    if window_left >= 0:
        vis &= j >= p - window_left
    if window_right >= 0:
        vis &= j <= p + window_right
    return vis


def _scores(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T in float64 ([P1] step 5b)."""
    return np.float64(scale) * (q_rows @ k.T)


def _masked_softmax(S: np.ndarray, vis: np.ndarray):
    """Row-wise softmax over visible entries; returns (P, lse).

    Two-pass, max-subtracted.  The mask is applied to S before the row max
    ([P1] "Correctness requirements", causal bullet).
    """
    Sm = np.where(vis, S, -np.inf)
    m = Sm.max(axis=1) if Sm.shape[1] else np.full(Sm.shape[0], -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    E = np.where(vis, np.exp(Sm - m_safe[:, None]), 0.0)
    l = E.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(empty[:, None], 0.0, E / np.where(empty, 1.0, l)[:, None])
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return P, lse


def attention_probs(q, k, scale: float, causal: bool, causal_offset: int = 0) -> np.ndarray:
    """Full softmax matrix P (B, Hq, Nq, Nkv) for small shapes (pin P1 uses it)."""
    q = _f64(q)
    k = _f64(k)
    B, Hq, Nq, _ = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    out = np.zeros((B, Hq, Nq, Nkv))
    vis = visibility(np.arange(Nq), Nkv, causal, causal_offset)
    for b in range(B):
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            out[b, h], _ = _masked_softmax(_scores(q[b, h], k[b, kvh], scale), vis)
    return out


def attention_forward(q, k, v, scale: float, causal: bool, rows=None, chunk: int = 512, causal_offset: int = 0,
                      window=(-1, -1)):
    """O1: prefill attention by the plain definition.

    q: (B, Hq, Nq, D); k, v: (B, Hkv, Nkv, D), any float dtype (widened exactly).
    causal_offset: query i sits at key position i + causal_offset (0 is the
    pages' top-left mask; Nkv - Nq aligns it bottom-right).  window: (left,
    right) sliding-window bounds around that position, -1 for an open side
    (see ``visibility``).
    rows: optional 1-D array of query positions to evaluate (sampling at large
    sizes); default all Nq positions.  Evaluated in row chunks so that the score
    block stays small; chunking does not change any value.

    Returns (O, lse): O (B, Hq, R, D) float64 and lse (B, Hq, R) float64 where R
    is the number of evaluated rows ([P1] steps 6 and 8).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nkv, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape or Hq % Hkv != 0:
        raise ValueError("shape mismatch")
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    O = np.zeros((B, Hq, R, D))
    lse = np.zeros((B, Hq, R))
    for b in range(B):
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            kb, vb = k[b, kvh], v[b, kvh]
            for r0 in range(0, R, chunk):
                sel = rows[r0:r0 + chunk]
                S = _scores(q[b, h, sel], kb, scale)
                P, ls = _masked_softmax(S, visibility(sel, Nkv, causal, causal_offset, window[0], window[1]))
                O[b, h, r0:r0 + chunk] = P @ vb
                lse[b, h, r0:r0 + chunk] = ls
    return O, lse


def attention_backward(q, k, v, do, scale: float, causal: bool, causal_offset: int = 0, window=(-1, -1)):
    """Gradients of ``attention_forward``'s O with respect to Q, K and V.

    For each (b, h) with kv head g = h // (Hq / Hkv), in float64:
        P   = the masked softmax of scale * Q K^T (as in the forward)
        dV[g] += P^T dO
        dP  = dO V^T
        dS  = P * (dP - rowsum(P * dP))        (softmax Jacobian applied to dP)
        dQ  = scale * dS K
        dK[g] += scale * dS^T Q
    Rows with no visible key have P = 0 and contribute nothing.  q, do:
    (B, Hq, Nq, D); k, v: (B, Hkv, Nkv, D).  Returns (dQ, dK, dV) float64 with
    the shapes of q, k, v.
    """
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    if do.shape != q.shape or v.shape != k.shape or k.shape[0] != B or k.shape[3] != D or Hq % Hkv != 0:
        raise ValueError("shape mismatch")
    vis = visibility(np.arange(Nq), Nkv, causal, causal_offset, window[0], window[1])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            P, _ = _masked_softmax(_scores(q[b, h], k[b, g], scale), vis)
            dv[b, g] += P.T @ do[b, h]
            dP = do[b, h] @ v[b, g].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq[b, h] = np.float64(scale) * (dS @ k[b, g])
            dk[b, g] += np.float64(scale) * (dS.T @ q[b, h])
    return dq, dk, dv


def decode(q, k_cache, v_cache, cache_len: int, scale: float, window_left: int = -1):
    """O2: one query token per (batch, q head) over cache slots [0, cache_len).

    [P3] decode phase: every cached position is valid, so there is no causal
    mask; GQA indexing is the same as prefill.  The query is the token at the
    last cached position, cache_len - 1; a sliding window of ``window_left``
    keeps keys j >= cache_len - 1 - window_left (-1: no window).  q: (B, Hq, D);
    caches (B, Hkv, S_max, D).  Returns O (B, Hq, D) and lse (B, Hq), float64.
    """
    q = _f64(q)
    if not (1 <= cache_len <= np.asarray(k_cache).shape[2]):
        raise ValueError("cache_len out of range")
    kc = _f64(np.asarray(k_cache)[:, :, :cache_len])
    vc = _f64(np.asarray(v_cache)[:, :, :cache_len])
    O, lse = attention_forward(q[:, :, None, :], kc, vc, scale, causal=False, causal_offset=cache_len - 1,
                               window=(window_left, -1))
    return O[:, :, 0, :], lse[:, :, 0]


def decode_varlen(q, k_cache, v_cache, cache_lens, scale: float, window_left: int = -1):
    """O2 per sequence: batch element b attends over its own slots [0, cache_lens[b]).

    [P3] decode phase, widened as its deferred-scope list names (per-sequence
    lengths): every slot below a sequence's length is visible, none above it.
    q: (B, Hq, D); caches (B, Hkv, S_max, D); cache_lens: B integers in
    [0, S_max].  A sequence of length 0 has no visible key: O = 0, lse = -inf.
    Returns O (B, Hq, D) and lse (B, Hq), float64.
    """
    q = _f64(q)
    lens = [int(x) for x in np.asarray(cache_lens).reshape(-1)]
    B, Hq, D = q.shape
    S_max = np.asarray(k_cache).shape[2]
    if len(lens) != B or any(L < 0 or L > S_max for L in lens):
        raise ValueError("cache_lens must hold B values in [0, S_max]")
    O = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b, L in enumerate(lens):
        if L == 0:
            continue
        Ob, lb = decode(q[b:b + 1], np.asarray(k_cache)[b:b + 1], np.asarray(v_cache)[b:b + 1], L, scale,
                        window_left)
        O[b], lse[b] = Ob[0], lb[0]
    return O, lse


def sequence_bounds(cu_seqlens, b: int):
    """Packed rows [cu[b], cu[b+1]) belong to sequence b (cumulative-length offsets)."""
    cu = np.asarray(cu_seqlens).reshape(-1)
    return int(cu[b]), int(cu[b + 1])


def varlen_causal_offset(Lq: int, Lk: int, bottom_right: bool) -> int:
    """Causal offset of one packed sequence: query i sees keys j <= i + offset.

    Top-left ([P1] step 5c) is 0; bottom-right treats the L_q queries as the
    last L_q of the sequence's L_k positions, offset L_k - L_q."""
    return Lk - Lq if bottom_right else 0


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool,
                     bottom_right: bool = False, rows=None, window=(-1, -1)):
    """O1 over a batch of packed sequences of different lengths.

    The pages defer variable-length batches ([P3] deferred scope); this is the
    plain definition of ``attention_forward`` applied to each sequence's own
    rows.  q: (T_q, Hq, D) packed query rows; k, v: (T_k, Hkv, D) packed key
    rows; cu_seqlens_q / cu_seqlens_k: B + 1 non-decreasing offsets from 0 to
    T_q / T_k.  causal with ``bottom_right`` uses ``varlen_causal_offset``.
    rows: optional packed query-row indices to evaluate (sampling at large
    sizes); default all T_q rows.

    Returns O (R, Hq, D) and lse (Hq, R), float64, R = number of evaluated rows.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    Tq, Hq, D = q.shape
    Tk, Hkv, Dk = k.shape
    cq = np.asarray(cu_seqlens_q, dtype=np.int64).reshape(-1)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64).reshape(-1)
    B = cq.shape[0] - 1
    if (Dk != D or v.shape != k.shape or Hq % Hkv != 0 or B < 1 or ck.shape[0] != B + 1
            or cq[0] != 0 or ck[0] != 0 or cq[-1] != Tq or ck[-1] != Tk
            or np.any(np.diff(cq) < 0) or np.any(np.diff(ck) < 0)):
        raise ValueError("shape or offsets mismatch")
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    O = np.zeros((R, Hq, D))
    lse = np.full((Hq, R), -np.inf)
    seq_of_row = np.searchsorted(cq, rows, side="right") - 1
    for b in range(B):
        q0, q1 = sequence_bounds(cq, b)
        k0, k1 = sequence_bounds(ck, b)
        pick = np.nonzero((seq_of_row == b) & (rows >= q0) & (rows < q1))[0]
        if pick.size == 0 or k1 == k0:
            continue  # no rows asked for, or no keys: O = 0, lse = -inf
        off = varlen_causal_offset(q1 - q0, k1 - k0, bottom_right) if (causal or window != (-1, -1)) else 0
        qs = q[q0:q1].transpose(1, 0, 2)[None]
        ks = k[k0:k1].transpose(1, 0, 2)[None]
        vs = v[k0:k1].transpose(1, 0, 2)[None]
        Ob, lb = attention_forward(qs, ks, vs, scale, causal, rows=rows[pick] - q0, causal_offset=off,
                                   window=window)
        O[pick] = Ob[0].transpose(1, 0, 2)
        lse[:, pick] = lb[0]
    return O, lse


def attention_varlen_backward(q, k, v, do, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool,
                              bottom_right: bool = False, window=(-1, -1)):
    """Gradients of ``attention_varlen``'s O: ``attention_backward`` on each
    sequence's own rows (no gradient crosses sequences).

    q, do: (T_q, Hq, D); k, v: (T_k, Hkv, D); offsets as ``attention_varlen``.
    Returns (dQ, dK, dV) float64 with the shapes of q, k, v; rows of a sequence
    with no keys, and keys of a sequence with no queries, get zero gradients.
    """
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    cq = np.asarray(cu_seqlens_q, dtype=np.int64).reshape(-1)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64).reshape(-1)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(cq.shape[0] - 1):
        q0, q1 = sequence_bounds(cq, b)
        k0, k1 = sequence_bounds(ck, b)
        if q1 == q0 or k1 == k0:
            continue
        masked = causal or window != (-1, -1)
        off = varlen_causal_offset(q1 - q0, k1 - k0, bottom_right) if masked else 0
        tq = lambda x, a, z: x[a:z].transpose(1, 0, 2)[None]
        gq, gk, gv = attention_backward(tq(q, q0, q1), tq(k, k0, k1), tq(v, k0, k1), tq(do, q0, q1), scale, causal,
                                        causal_offset=off, window=window)
        dq[q0:q1] = gq[0].transpose(1, 0, 2)
        dk[k0:k1] = gk[0].transpose(1, 0, 2)
        dv[k0:k1] = gv[0].transpose(1, 0, 2)
    return dq, dk, dv


def kv_cache_write(k_cache, v_cache, k_new, v_new, pos: int):
    """O3: copies of the caches with slots [pos, pos + T) replaced by the new rows.

    [P3] decode phase: a preallocated cache written by a separate helper.
    Works on any dtype (including raw uint16 views of fp16/bf16); every other
    element is left bit-for-bit unchanged.  Caches (B, Hkv, S_max, D); new rows
    (B, Hkv, T, D).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    T = np.asarray(k_new).shape[2]
    if pos < 0 or pos + T > kc.shape[2]:
        raise ValueError("write outside the cache")
    kc[:, :, pos:pos + T] = k_new
    vc[:, :, pos:pos + T] = v_new
    return kc, vc


def page_slot(block_table, b: int, r: int, page_size: int):
    """(page, row) that hold cache slot r of sequence b in a paged cache."""
    return int(np.asarray(block_table)[b, r // page_size]), r % page_size


def gather_pages(pages, block_table, b: int, length: int, page_size: int) -> np.ndarray:
    """Sequence b's first ``length`` cache slots as a contiguous (Hkv, length, D) array."""
    pages = np.asarray(pages)
    out = np.zeros((pages.shape[1], length, pages.shape[3]), dtype=pages.dtype)
    for r in range(length):
        p, i = page_slot(block_table, b, r, page_size)
        out[:, r] = pages[p, :, i]
    return out


def decode_paged(q, k_pages, v_pages, block_table, cache_lens, page_size: int, scale: float,
                 window_left: int = -1):
    """O2 over a paged cache: ``decode_varlen`` on each sequence's gathered slots.

    q: (B, Hq, D); k_pages, v_pages: (num_pages, Hkv, page_size, D); block_table:
    (B, max_pages) page ids; cache_lens: B lengths in [0, max_pages * page_size].
    Returns O (B, Hq, D) and lse (B, Hq), float64 (length 0: O = 0, lse = -inf).
    """
    q = _f64(q)
    lens = [int(x) for x in np.asarray(cache_lens).reshape(-1)]
    B = q.shape[0]
    tbl = np.asarray(block_table)
    if len(lens) != B or tbl.shape[0] != B or any(L < 0 or L > tbl.shape[1] * page_size for L in lens):
        raise ValueError("cache_lens must hold B values within the block table's pages")
    S = max(max(lens), 1)
    Hkv, D = np.asarray(k_pages).shape[1], np.asarray(k_pages).shape[3]
    kc = np.zeros((B, Hkv, S, D))
    vc = np.zeros((B, Hkv, S, D))
    for b, L in enumerate(lens):
        kc[b, :, :L] = gather_pages(k_pages, tbl, b, L, page_size)
        vc[b, :, :L] = gather_pages(v_pages, tbl, b, L, page_size)
    return decode_varlen(q, kc, vc, lens, scale, window_left)


def kv_cache_write_paged(k_pages, v_pages, k_new, v_new, block_table, pos, page_size: int):
    """O3 over a paged cache: copies of the pools with sequence b's slots
    pos[b] .. pos[b] + T - 1 replaced by its T new rows (B, Hkv, T, D); every
    other element is left bit-for-bit unchanged."""
    kp = np.array(k_pages, copy=True)
    vp = np.array(v_pages, copy=True)
    kn, vn = np.asarray(k_new), np.asarray(v_new)
    tbl = np.asarray(block_table)
    B, _, T, _ = kn.shape
    for b in range(B):
        p0 = int(np.asarray(pos).reshape(-1)[b])
        if p0 < 0 or p0 + T > tbl.shape[1] * page_size:
            raise ValueError("write outside the sequence's pages")
        for t in range(T):
            pg, i = page_slot(tbl, b, p0 + t, page_size)
            kp[pg, :, i] = kn[b, :, t]
            vp[pg, :, i] = vn[b, :, t]
    return kp, vp
