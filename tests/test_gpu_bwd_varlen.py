"""GPU parity of attn_bwd_varlen (the backward over packed sequences of
different lengths) against the fp64 oracle, plus bitwise equivalence with
attn_bwd when every sequence has the same length.

The GPU backward takes attn_fwd_varlen's O and lse.  Tolerance as in the dense
backward's tests (4 u max|ref| + an fp32 floor per gradient tensor), with the
floor sized by the longest sequence.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_attn_fwd_05_amd as A
import oracle
import workloads as W
from test_gpu_bwd import _check, _floor, _np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENTINEL = 7.0


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _cu(lens):
    return torch.tensor(W.VarlenPrefillCase._cu(lens), dtype=torch.int32, device=DEV)


def _dout(case, seed):
    g = torch.Generator().manual_seed(W.BASE_SEED + 240 + seed)
    return torch.randn(case.total_q, case.Hq, case.D, generator=g).to(case.torch_dtype)


def run_bwd_varlen(case: W.VarlenPrefillCase, window=None, seed=0):
    q, k, v = W.varlen_prefill_inputs(case)
    do = _dout(case, seed)
    align = "bottom_right" if case.bottom_right else "top_left"
    _say(f"{case.name} q_lens={case.q_lens} k_lens={case.k_lens} causal={case.causal} align={align} "
         f"window={window}")
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    cq, ck = _cu(case.q_lens), _cu(case.k_lens)
    o, lse = A.attn_fwd_varlen(qd, kd, vd, cq, ck, case.max_q, causal=case.causal, causal_align=align,
                               scale=case.softmax_scale, return_lse=True, window=window)
    dq, dk, dv = A.attn_bwd_varlen(qd, kd, vd, o, dod, lse, cq, ck, case.max_q, max(max(case.k_lens), 1),
                                   causal=case.causal, causal_align=align, scale=case.softmax_scale, window=window)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_varlen_backward(_np(q), _np(k), _np(v), _np(do), case.cu_q, case.cu_k,
                                                  case.softmax_scale, case.causal, bottom_right=case.bottom_right,
                                                  window=window or (-1, -1))
    sc, Lk, Lq = case.softmax_scale, max(case.k_lens), max(case.q_lens)
    _check("dQ", dq, rq, case.torch_dtype, _floor(case.D, Lk, do, v.float(), sc, k.float()))
    _check("dK", dk, rk, case.torch_dtype, _floor(case.D, Lq, do, v.float(), sc, q.float()))
    _check("dV", dv, rv, case.torch_dtype)
    return dq, dk, dv


MODES = [(False, False), (True, False), (True, True)]
MODE_IDS = ["full", "top_left", "bottom_right"]


@pytest.mark.parametrize("causal,br", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("Hq,Hkv,D,dtype", [(8, 2, 128, "fp16"), (4, 1, 64, "bf16")])
def test_bwd_varlen_mixed_lengths(causal, br, Hq, Hkv, D, dtype):
    """Lengths across the 256-row dQ block, the 128-key dK/dV block and the
    64-row tile, incl. 0 and 1."""
    lens = (1, 255, 256, 257, 0, 700, 64, 1000, 129)
    run_bwd_varlen(W.VarlenPrefillCase(f"bwd_mixed_h{Hq}_{Hkv}_d{D}_{dtype}", lens, lens, Hq, Hkv, D, dtype, causal,
                                       br, seed=W.BASE_SEED + 140 + D + Hkv), seed=D + Hkv)


@pytest.mark.parametrize("causal,br", MODES, ids=MODE_IDS)
def test_bwd_varlen_queries_differ_from_keys(causal, br):
    """L_q < L_k, L_q > L_k (bottom-right: leading rows see nothing, dQ = 0),
    queries with no keys (dQ = 0) and keys with no queries (dK = dV = 0)."""
    case = W.VarlenPrefillCase("bwd_chunks", (100, 256, 1, 300, 0, 5, 129), (1000, 256, 2000, 100, 50, 0, 129),
                               8, 2, 128, "fp16", causal, br, seed=W.BASE_SEED + 145)
    run_bwd_varlen(case, seed=5)


@pytest.mark.parametrize("br", [False, True], ids=["top_left", "bottom_right"])
def test_bwd_varlen_causal_window(br):
    case = W.VarlenPrefillCase("bwd_varlen_window", (1, 255, 700, 0, 1000, 64), (1, 300, 700, 20, 1300, 64), 8, 2,
                               128, "fp16", True, br, seed=W.BASE_SEED + 146)
    run_bwd_varlen(case, window=(199, -1), seed=6)


def test_bwd_varlen_two_sided_window():
    case = W.VarlenPrefillCase("bwd_varlen_band", (300, 77, 513), (300, 77, 513), 4, 2, 64, "bf16", False,
                               seed=W.BASE_SEED + 147)
    run_bwd_varlen(case, window=(50, 20), seed=7)


def test_bwd_varlen_equal_lengths_is_bwd_bitwise():
    """B equal-length sequences packed: identical bits to attn_bwd on the
    (B, N, H, D) layout, for every mask form."""
    B, N, Hq, Hkv, D = 3, 1000, 8, 2, 128
    _say("varlen bwd vs attn_bwd, equal lengths")
    g = torch.Generator().manual_seed(W.BASE_SEED + 148)
    q, do = (torch.randn(B, N, Hq, D, generator=g).half().to(DEV) for _ in range(2))
    k, v = (torch.randn(B, N, Hkv, D, generator=g).half().to(DEV) for _ in range(2))
    cu = _cu([N] * B)
    T = lambda x: x.transpose(1, 2)  # noqa: E731
    P = lambda x, H: x.reshape(B * N, H, D)  # noqa: E731
    for causal, align, window in ((True, "top_left", None), (False, "top_left", None), (True, "bottom_right", None),
                                  (True, "top_left", (255, -1))):
        o, lse = A.attn_fwd(T(q), T(k), T(v), causal=causal, causal_align=align, return_lse=True, window=window)
        g1 = A.attn_bwd(T(q), T(k), T(v), o, T(do), lse, causal=causal, causal_align=align, window=window)
        o_p = T(o).reshape(B * N, Hq, D)
        lse_p = lse.permute(1, 0, 2).reshape(Hq, B * N).contiguous()
        g2 = A.attn_bwd_varlen(P(q, Hq), P(k, Hkv), P(v, Hkv), o_p, P(do, Hq), lse_p, cu, cu, N, N, causal=causal,
                               causal_align=align, window=window)
        torch.cuda.synchronize()
        for a_, b_, H in zip(g1, g2, (Hq, Hkv, Hkv)):
            assert torch.equal(T(a_).reshape(B * N, H, D), b_), (causal, align, window)


@pytest.mark.parametrize("br", [False, True], ids=["top_left", "bottom_right"])
def test_bwd_varlen_max_seqlen_caps_rows(br):
    """Query rows at positions >= max_seqlen_q (not computed by the forward)
    get no dQ and add nothing to dK, dV: the oracle sees them with dO = 0."""
    case = W.VarlenPrefillCase("bwd_capped", (600, 100, 300), (900, 100, 300), 4, 1, 128, "fp16", True, br,
                               seed=W.BASE_SEED + 149)
    cap = 260
    q, k, v = W.varlen_prefill_inputs(case)
    do = _dout(case, 9)
    align = "bottom_right" if br else "top_left"
    _say(f"{case.name} cap={cap} align={align}")
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    cq, ck = _cu(case.q_lens), _cu(case.k_lens)
    o = torch.full((case.total_q, case.Hq, case.D), SENTINEL, dtype=torch.float16, device=DEV)
    lse = torch.full((case.Hq, case.total_q), SENTINEL, dtype=torch.float32, device=DEV)
    A.attn_fwd_varlen(qd, kd, vd, cq, ck, cap, causal=True, out=o, lse=lse, causal_align=align)
    dq = torch.full_like(qd, SENTINEL)
    dq, dk, dv = A.attn_bwd_varlen(qd, kd, vd, o, dod, lse, cq, ck, cap, 900, causal=True, causal_align=align, dq=dq)
    torch.cuda.synchronize()
    c = case.cu_q
    done = np.concatenate([np.arange(c[b], c[b] + min(cap, case.q_lens[b])) for b in range(case.B)])
    skipped = np.setdiff1d(np.arange(case.total_q), done)
    assert torch.all(dq[torch.as_tensor(skipped).to(DEV)] == SENTINEL)
    do_ref = do.clone()
    do_ref[torch.as_tensor(skipped)] = 0
    rq, rk, rv = oracle.attention_varlen_backward(_np(q), _np(k), _np(v), _np(do_ref), case.cu_q, case.cu_k,
                                                  case.softmax_scale, True, bottom_right=br)
    sc = case.softmax_scale
    _check("dQ", dq[torch.as_tensor(done).to(DEV)], rq[done], case.torch_dtype,
           _floor(case.D, 900, do, v.float(), sc, k.float()))
    _check("dK", dk, rk, case.torch_dtype, _floor(case.D, cap, do, v.float(), sc, q.float()))
    _check("dV", dv, rv, case.torch_dtype)


def test_bwd_varlen_neighbour_nan_never_leaks():
    """NaN in every Q/K/V/dO row of sequence 1 leaves the gradients of
    sequences 0 and 2 exact."""
    case = W.VarlenPrefillCase("bwd_nan_neighbour", (130, 70, 300), (130, 70, 300), 4, 2, 128, "fp16", True,
                               seed=W.BASE_SEED + 150)
    q, k, v = W.varlen_prefill_inputs(case)
    do = _dout(case, 10)
    _say(case.name)
    c = case.cu_q
    for t in (q, k, v, do):
        t[c[1]:c[2]] = float("nan")
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    cq = _cu(case.q_lens)
    o, lse = A.attn_fwd_varlen(qd, kd, vd, cq, cq, case.max_q, causal=True, return_lse=True)
    dq, dk, dv = A.attn_bwd_varlen(qd, kd, vd, o, dod, lse, cq, cq, causal=True)
    torch.cuda.synchronize()
    keep = np.r_[c[0]:c[1], c[2]:c[3]]
    q2, k2, v2, do2 = (x[torch.as_tensor(keep)] for x in (q, k, v, do))
    cu2 = [0, 130, 430]
    rq, rk, rv = oracle.attention_varlen_backward(_np(q2), _np(k2), _np(v2), _np(do2), cu2, cu2,
                                                  case.softmax_scale, True)
    ki = torch.as_tensor(keep).to(DEV)
    sc = case.softmax_scale
    _check("dQ", dq[ki], rq, case.torch_dtype, _floor(case.D, 300, do2, v2.float(), sc, k2.float()))
    _check("dK", dk[ki], rk, case.torch_dtype, _floor(case.D, 300, do2, v2.float(), sc, q2.float()))
    _check("dV", dv[ki], rv, case.torch_dtype)


def test_bwd_varlen_serving_batch_sampled():
    """The 16-sequence packed serving batch (lengths up to 4096, Hq=32, Hkv=8,
    D=128, causal): the gradients of the shortest, a middle and the longest
    sequence, on one kv head's group, against the oracle."""
    case = W.varlen_serving_case()
    q, k, v = W.varlen_prefill_inputs(case)
    do = _dout(case, 11)
    _say(f"{case.name} sampled")
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    cq = _cu(case.q_lens)
    o, lse = A.attn_fwd_varlen(qd, kd, vd, cq, cq, case.max_q, causal=True, scale=case.softmax_scale,
                               return_lse=True)
    dq, dk, dv = A.attn_bwd_varlen(qd, kd, vd, o, dod, lse, cq, cq, case.max_q, case.max_q, causal=True,
                                   scale=case.softmax_scale)
    torch.cuda.synchronize()
    order = np.argsort(case.q_lens)
    G = case.Hq // case.Hkv
    kvh = 5
    hs = slice(kvh * G, (kvh + 1) * G)
    c = case.cu_q
    sc = case.softmax_scale
    for b in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        r = slice(c[b], c[b + 1])
        L = c[b + 1] - c[b]
        tq = lambda x, h: _np(x[r, h]).transpose(1, 0, 2)[None]  # noqa: E731
        rq, rk, rv = oracle.attention_backward(tq(q, hs), tq(k, slice(kvh, kvh + 1)), tq(v, slice(kvh, kvh + 1)),
                                               tq(do, hs), sc, True)
        back = lambda t, h: t[r, h].permute(1, 0, 2)[None]  # noqa: E731
        print(f"    sequence {b}, length {L}", flush=True)
        _check("dQ", back(dq, hs), rq, case.torch_dtype, _floor(case.D, L, do, v.float(), sc, k.float()))
        _check("dK", back(dk, slice(kvh, kvh + 1)), rk, case.torch_dtype,
               _floor(case.D, L, do, v.float(), sc, q.float()))
        _check("dV", back(dv, slice(kvh, kvh + 1)), rv, case.torch_dtype)
