"""GPU parity at the addressing limits: the largest row stride the library
accepts (2^22 elements) and base / row offsets beyond 2^31 bytes (and
elements), for prefill, packed prefill, decode (contiguous and paged) and the
backward, against the fp64 oracle on small dense copies.

Each big tensor is a strided view into a buffer filled with NaN first, so a
read of any element outside the view shows up as a non-finite output.  The
buffers take a few GiB each; every test frees them before it returns.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_attn_fwd_05_amd as A
import oracle
import workloads as W
from gpu_util import check_lse, check_o
from test_gpu_bwd import _check, _floor

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
R_MAX = 1 << 22          # largest accepted row stride (elements)
BIG = (1 << 31) + 1024   # a batch / page offset beyond 2^31 elements (4 GiB of fp16)


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _poisoned_view(shape, strides, dtype=torch.float16):
    """A NaN-filled buffer just large enough for `shape` / `strides` (elements),
    viewed with those strides."""
    need = 1 + sum((n - 1) * s for n, s in zip(shape, strides))
    buf = torch.full((need,), float("nan"), dtype=dtype, device=DEV)
    return buf.as_strided(shape, strides)


def _place(dense, strides):
    v = _poisoned_view(tuple(dense.shape), strides, dense.dtype)
    v.copy_(dense.to(DEV))
    return v


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_prefill_max_row_stride():
    """q, k, v, o with a 2^22-element row stride ((B, N, H, D)-like views with
    padded rows): batch offsets of 2^31.6 bytes, in-tile offsets near 2^30."""
    B, Hq, Hkv, N, D = 2, 2, 1, 100, 128
    case = W.PrefillCase("max_row_stride", B, Hq, Hkv, N, N, D, "fp16", True, seed=W.BASE_SEED + 160)
    q, k, v = W.prefill_inputs(case)
    _say(f"{case.name} row stride {R_MAX}")
    st = lambda H: (N * R_MAX, D, R_MAX, 1)  # noqa: E731
    qd, kd, vd = _place(q, st(Hq)), _place(k, st(Hkv)), _place(v, st(Hkv))
    o = _poisoned_view((B, Hq, N, D), st(Hq))
    _, lse = A.attn_fwd(qd, kd, vd, causal=True, scale=case.softmax_scale, out=o, return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention_forward(_np(q), _np(k), _np(v), case.softmax_scale, True)
    check_o(o.contiguous().cpu(), Oref, torch.float16)
    check_lse(lse.cpu(), Lref)


def test_prefill_kv_batch_offset_beyond_2g_elements():
    B, Hq, Hkv, N, D = 2, 4, 2, 300, 128
    case = W.PrefillCase("kv_offset", B, Hq, Hkv, N, N, D, "bf16", False, seed=W.BASE_SEED + 161)
    q, k, v = W.prefill_inputs(case)
    _say(f"{case.name} k/v batch stride {BIG}")
    st = (BIG, N * D, D, 1)
    kd, vd = _place(k, st), _place(v, st)
    o, lse = A.attn_fwd(q.to(DEV), kd, vd, causal=False, scale=case.softmax_scale, return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention_forward(_np(q), _np(k), _np(v), case.softmax_scale, False)
    check_o(o.cpu(), Oref, torch.bfloat16)
    check_lse(lse.cpu(), Lref)


def test_prefill_varlen_rows_beyond_2g_bytes():
    """A packed batch whose second sequence starts 2^23 key rows in (2^31 bytes
    of K and of V before it); the first sequence has one query (top-left
    causal: it sees key 0 only)."""
    Hq, Hkv, D, L0, L1 = 4, 1, 128, 1 << 23, 300
    g = torch.Generator(device=DEV).manual_seed(W.BASE_SEED + 162)
    _say(f"varlen K/V rows from {L0}")
    q = torch.randn(1 + L1, Hq, D, generator=g, device=DEV).half()
    k = torch.randn(L0 + L1, Hkv, D, generator=g, device=DEV).half()
    v = torch.randn(L0 + L1, Hkv, D, generator=g, device=DEV).half()
    cq = torch.tensor([0, 1, 1 + L1], dtype=torch.int32, device=DEV)
    ck = torch.tensor([0, L0, L0 + L1], dtype=torch.int32, device=DEV)
    scale = D ** -0.5
    o, lse = A.attn_fwd_varlen(q, k, v, cq, ck, L1, causal=True, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    # sequence 0: O = V[0] exactly, lse = its one score
    assert torch.equal(o[0], v[0].expand(Hq, D))
    s0 = (q[0].float() @ k[0, 0].float()) * scale
    assert torch.allclose(lse[:, 0], s0, rtol=0, atol=1e-4 * max(1.0, float(s0.abs().max())))
    # sequence 1 against the oracle
    qs, ks, vs = q[1:].cpu(), k[L0:].cpu(), v[L0:].cpu()
    Oref, Lref = oracle.attention_varlen(_np(qs), _np(ks), _np(vs), [0, L1], [0, L1], scale, True)
    check_o(o[1:].cpu(), Oref, torch.float16)
    check_lse(lse[:, 1:].cpu(), Lref)


def test_decode_max_row_stride_and_batch_offset():
    """Caches with a 2^22-element slot stride (batch offsets of 2^30.3
    elements), cache_len across the 128-row tile."""
    B, Hq, Hkv, S, D, L = 2, 8, 2, 160, 128, 150
    case = W.DecodeCase("decode_max_stride", B, Hq, Hkv, S, L, D, "fp16", seed=W.BASE_SEED + 163)
    q, kc, vc = W.decode_inputs(case)
    _say(f"{case.name} slot stride {R_MAX}")
    st = (S * R_MAX, D, R_MAX, 1)
    kd, vd = _place(kc, st), _place(vc, st)
    o, lse = A.attn_decode(q.to(DEV), kd, vd, L, scale=case.softmax_scale, return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.decode(_np(q), _np(kc), _np(vc), L, case.softmax_scale)
    check_o(o.cpu(), Oref, torch.float16)
    check_lse(lse.cpu(), Lref)


def test_decode_batch_offset_beyond_2g_elements():
    B, Hq, Hkv, S, D, L = 2, 8, 2, 512, 128, 500
    case = W.DecodeCase("decode_offset", B, Hq, Hkv, S, L, D, "bf16", seed=W.BASE_SEED + 164)
    q, kc, vc = W.decode_inputs(case)
    _say(f"{case.name} cache batch stride {BIG}")
    st = (BIG, S * D, D, 1)
    kd, vd = _place(kc, st), _place(vc, st)
    o, lse = A.attn_decode(q.to(DEV), kd, vd, L, scale=case.softmax_scale, num_splits=3, return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.decode(_np(q), _np(kc), _np(vc), L, case.softmax_scale)
    check_o(o.cpu(), Oref, torch.bfloat16)
    check_lse(lse.cpu(), Lref)


def test_decode_paged_pages_beyond_2g_elements():
    """Pages taken from the top of a 2^20 + 8 page pool (page offsets beyond
    2^31 elements); every other page is NaN."""
    B, Hq, Hkv, D, ps, S = 2, 8, 1, 128, 16, 256
    case = W.DecodeCase("paged_offset", B, Hq, Hkv, S, S, D, "fp16", seed=W.BASE_SEED + 165)
    q, kc, vc = W.decode_inputs(case)
    lens = [256, 201]
    P = (1 << 20) + 8
    npb = S // ps
    _say(f"{case.name} pool of {P} pages")
    perm = torch.randperm(B * npb, generator=torch.Generator().manual_seed(5)) + (P - B * npb)
    tbl = perm.reshape(B, npb).to(torch.int32)
    pools = []
    for c in (kc, vc):
        pool = torch.full((P, Hkv, ps, D), float("nan"), dtype=torch.float16, device=DEV)
        pool[perm.to(DEV)] = c.reshape(B, Hkv, npb, ps, D).permute(0, 2, 1, 3, 4).reshape(B * npb, Hkv, ps, D).to(DEV)
        pools.append(pool)
    ld = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = A.attn_decode_paged(q.to(DEV), pools[0], pools[1], tbl.to(DEV), ld, scale=case.softmax_scale,
                                 return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.decode_varlen(_np(q), _np(kc), _np(vc), lens, case.softmax_scale)
    check_o(o.cpu(), Oref, torch.float16)
    check_lse(lse.cpu(), Lref)


def test_bwd_kv_batch_offset_beyond_2g_elements():
    """K, V and their gradients as views with a batch stride beyond 2^31
    elements; the gradient views' other elements stay NaN-filled around them."""
    B, Hq, Hkv, N, D = 2, 4, 2, 200, 128
    case = W.PrefillCase("bwd_offset", B, Hq, Hkv, N, N, D, "fp16", True, seed=W.BASE_SEED + 166)
    q, k, v = W.prefill_inputs(case)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(W.BASE_SEED + 167)).half()
    _say(f"{case.name} k/v/dk/dv batch stride {BIG}")
    st = (BIG, N * D, D, 1)
    kd, vd = _place(k, st), _place(v, st)
    dk = _poisoned_view((B, Hkv, N, D), st)
    dv = _poisoned_view((B, Hkv, N, D), st)
    qd, dod = q.to(DEV), do.to(DEV)
    sc = case.softmax_scale
    o, lse = A.attn_fwd(qd, kd, vd, causal=True, scale=sc, return_lse=True)
    dq, dk, dv = A.attn_bwd(qd, kd, vd, o, dod, lse, causal=True, scale=sc, dk=dk, dv=dv)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(_np(q), _np(k), _np(v), _np(do), sc, True)
    _check("dQ", dq, rq, torch.float16, _floor(D, N, do, v.float(), sc, k.float()))
    _check("dK", dk.contiguous(), rk, torch.float16, _floor(D, N, do, v.float(), sc, q.float()))
    _check("dV", dv.contiguous(), rv, torch.float16)
