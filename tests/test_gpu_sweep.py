"""Seeded randomized parity sweep against the fp64 oracle: combinations of
dtype, head dim, GQA ratio, lengths (ragged, incl. 1 and 0 in packed
batches), mask form (none, causal top-left / bottom-right, sliding windows of
either alignment, causal windows), scale (incl. negative), tensor layout and
split count that the fixed cases do not enumerate, for the forward (dense and
packed), decode (contiguous, per-sequence and paged caches) and the backward
(dense and packed).

The case list is drawn once from a fixed seed, so every run checks the same
cases; each case prints its parameters before it touches the GPU.
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
_DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _rand(shape, dtype, g, sd=1.0):
    return (sd * torch.randn(shape, generator=g)).to(_DT[dtype])


def _mask_choice(rng, Nq, Nkv):
    """(causal, align, window or None)."""
    kind = rng.integers(0, 6)
    align = "bottom_right" if rng.integers(0, 2) else "top_left"
    if kind == 0:
        return False, "top_left", None
    if kind == 1:
        return True, "top_left", None
    if kind == 2:
        return True, "bottom_right", None
    span = max(Nq, Nkv)
    if kind == 3:  # causal sliding window
        return True, align, (int(rng.integers(0, span + 2)), -1)
    if kind == 4:  # two-sided band
        return False, align, (int(rng.integers(-1, span // 2 + 2)), int(rng.integers(-1, span // 2 + 2)))
    return False, align, (-1, int(rng.integers(0, span // 3 + 2)))  # right-only band


def _compare_rows(o, l, Oref, Lref, dtype, row_axis_o, row_axis_l=None):
    """Rows the oracle leaves empty (lse = -inf) must be o = 0, lse = -inf."""
    o, l = o.cpu(), l.cpu()
    empty = ~np.isfinite(Lref)
    if empty.any():
        assert torch.all(l[torch.from_numpy(empty)] == float("-inf"))
    live = torch.from_numpy(~empty)
    if row_axis_o == "packed":  # o (T, Hq, D), l (Hq, T)
        if empty.any():
            assert torch.all(o[torch.from_numpy(empty.T)] == 0)
        check_o(o[live.T], Oref[(~empty).T], dtype)
    else:  # o (..., R, D), l (..., R)
        if empty.any():
            assert torch.all(o[torch.from_numpy(empty)] == 0)
        check_o(o[live], Oref[~empty], dtype)
    check_lse(l[live], Lref[~empty])


# ---- forward, dense

def _fwd_cases(n=48, seed=7001):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        Nq, Nkv = int(rng.integers(1, 700)), int(rng.integers(1, 700))
        causal, align, window = _mask_choice(rng, Nq, Nkv)
        out.append(dict(i=i, B=int(rng.integers(1, 3)), Hq=Hkv * G, Hkv=Hkv, Nq=Nq, Nkv=Nkv,
                        D=int(rng.choice([64, 128])), dtype=str(rng.choice(["fp16", "bf16"])), causal=causal,
                        align=align, window=window, neg=bool(rng.integers(0, 4) == 0),
                        bnhd=bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("cs", _fwd_cases(), ids=lambda c: f"fwd{c['i']}")
def test_sweep_forward(cs):
    _run_forward(cs, 9000)


def _run_forward(cs, seed_base):
    _say(cs)
    g = torch.Generator().manual_seed(seed_base + cs["i"])
    B, Hq, Hkv, Nq, Nkv, D, dt = cs["B"], cs["Hq"], cs["Hkv"], cs["Nq"], cs["Nkv"], cs["D"], cs["dtype"]
    q, k, v = _rand((B, Hq, Nq, D), dt, g), _rand((B, Hkv, Nkv, D), dt, g), _rand((B, Hkv, Nkv, D), dt, g)
    scale = (-1.0 if cs["neg"] else 1.0) * D ** -0.5
    dev = [t.to(DEV) for t in (q, k, v)]
    if cs["bnhd"]:  # (B, N, H, D) storage viewed as (B, H, N, D)
        dev = [t.transpose(1, 2).contiguous().transpose(1, 2) for t in dev]
    o, l = A.attn_fwd(*dev, causal=cs["causal"], causal_align=cs["align"], window=cs["window"], scale=scale,
                      return_lse=True)
    torch.cuda.synchronize()
    off = Nkv - Nq if cs["align"] == "bottom_right" else 0
    masked = cs["causal"] or cs["window"] is not None
    Oref, Lref = oracle.attention_forward(_np(q), _np(k), _np(v), scale, cs["causal"],
                                          causal_offset=off if masked else 0, window=cs["window"] or (-1, -1))
    _compare_rows(o, l, Oref, Lref, _DT[dt], "dense")



def _fwd_large_cases(n=24, seed=7005):
    """Grids of more than 128 blocks of 256 rows (the one-key-group kernels,
    the counted ring on masked ones) with ragged lengths."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.choice([2, 4, 8]))
        Hq = Hkv * int(rng.choice([2, 4]))
        Nq, Nkv = int(rng.integers(257, 1100)), int(rng.integers(257, 1100))
        B = 1
        while B * Hq * ((Nq + 255) // 256) <= 128:
            B += 1
        causal, align, window = _mask_choice(rng, Nq, Nkv)
        out.append(dict(i=i, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nkv=Nkv, D=int(rng.choice([64, 128])),
                        dtype=str(rng.choice(["fp16", "bf16"])), causal=causal, align=align, window=window,
                        neg=bool(rng.integers(0, 4) == 0), bnhd=bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("cs", _fwd_large_cases(), ids=lambda c: f"fwdL{c['i']}")
def test_sweep_forward_large_grid(cs):
    _run_forward(cs, 9500)


# ---- forward, packed

def _varlen_cases(n=20, seed=7002):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        nb = int(rng.integers(1, 7))
        ql = [int(x) for x in rng.integers(0, 400, nb)]
        kl = ql if rng.integers(0, 2) else [int(x) for x in rng.integers(0, 400, nb)]
        Hkv = int(rng.choice([1, 2, 4]))
        causal, align, window = _mask_choice(rng, max(ql + [1]), max(kl + [1]))
        out.append(dict(i=i, ql=ql, kl=kl, Hq=Hkv * int(rng.choice([1, 2, 4])), Hkv=Hkv,
                        D=int(rng.choice([64, 128])), dtype=str(rng.choice(["fp16", "bf16"])), causal=causal,
                        align=align, window=window))
    return out


@pytest.mark.parametrize("cs", _varlen_cases(), ids=lambda c: f"varlen{c['i']}")
def test_sweep_forward_packed(cs):
    _say(cs)
    case = W.VarlenPrefillCase(f"sweep{cs['i']}", tuple(cs["ql"]), tuple(cs["kl"]), cs["Hq"], cs["Hkv"], cs["D"],
                               cs["dtype"], cs["causal"], cs["align"] == "bottom_right", seed=9100 + cs["i"])
    if case.total_q == 0 or case.total_k == 0:
        pytest.skip("empty packed batch")
    q, k, v = W.varlen_prefill_inputs(case)
    cq = torch.tensor(case.cu_q, dtype=torch.int32, device=DEV)
    ck = torch.tensor(case.cu_k, dtype=torch.int32, device=DEV)
    o, l = A.attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq, ck, max(case.max_q, 1), causal=cs["causal"],
                             causal_align=cs["align"], window=cs["window"], scale=case.softmax_scale,
                             return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention_varlen(_np(q), _np(k), _np(v), case.cu_q, case.cu_k, case.softmax_scale,
                                         cs["causal"], bottom_right=cs["align"] == "bottom_right",
                                         window=cs["window"] or (-1, -1))
    _compare_rows(o, l, Oref, Lref, case.torch_dtype, "packed")


# ---- decode

def _decode_cases(n=30, seed=7003):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 5))
        S = int(rng.choice([256, 1024, 2048]))
        mode = str(rng.choice(["uniform", "varlen", "paged"]))
        lens = [int(x) for x in rng.integers(0 if mode != "uniform" else 1, S + 1, B)]
        if mode == "uniform":
            lens = [lens[0]] * B
        out.append(dict(i=i, B=B, Hq=Hkv * int(rng.choice([1, 2, 4, 8])), Hkv=Hkv, S=S, D=int(rng.choice([64, 128])),
                        dtype=str(rng.choice(["fp16", "bf16"])), mode=mode, lens=lens,
                        wl=int(rng.choice([-1, -1, 0, int(rng.integers(1, S))])),
                        ns=int(rng.choice([0, 0, 1, int(rng.integers(2, 20))])), ps=int(rng.choice([16, 32, 64]))))
    return out


@pytest.mark.parametrize("cs", _decode_cases(), ids=lambda c: f"dec{c['i']}_{c['mode']}")
def test_sweep_decode(cs):
    from test_gpu_decode_paged import make_paged
    from test_gpu_window import _poison_outside
    _say(cs)
    case = W.DecodeCase(f"sweep{cs['i']}", cs["B"], cs["Hq"], cs["Hkv"], cs["S"], max(cs["lens"] + [1]), cs["D"],
                        cs["dtype"], seed=9200 + cs["i"])
    q, kc, vc = W.decode_inputs(case)
    lens, sc = cs["lens"], case.softmax_scale
    qd = q.to(DEV)
    # every slot a call must not read (past a length, before a window) is NaN
    # on the GPU side; the oracle gets the clean caches
    kx, vx = _poison_outside(kc, lens, cs["wl"]), _poison_outside(vc, lens, cs["wl"])
    if cs["mode"] == "uniform":
        o, l = A.attn_decode(qd, kx.to(DEV), vx.to(DEV), lens[0], scale=sc, num_splits=cs["ns"],
                             window_left=cs["wl"], return_lse=True)
    elif cs["mode"] == "varlen":
        ld = torch.tensor(lens, dtype=torch.int32, device=DEV)
        o, l = A.attn_decode_varlen(qd, kx.to(DEV), vx.to(DEV), ld, scale=sc, num_splits=cs["ns"],
                                    window_left=cs["wl"], return_lse=True)
    else:
        kp, vp, tbl = make_paged(kx, vx, lens, cs["ps"], seed=cs["i"])
        ld = torch.tensor(lens, dtype=torch.int32, device=DEV)
        o, l = A.attn_decode_paged(qd, kp.to(DEV), vp.to(DEV), tbl.to(DEV), ld, scale=sc, num_splits=cs["ns"],
                                   window_left=cs["wl"], return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.decode_varlen(_np(q), _np(kc), _np(vc), lens, sc, window_left=cs["wl"])
    _compare_rows(o, l, Oref, Lref, case.torch_dtype, "dense")


# ---- backward

def _bwd_cases(n=24, seed=7004):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        packed = bool(rng.integers(0, 3) == 0)
        Nq, Nkv = int(rng.integers(1, 500)), int(rng.integers(1, 500))
        causal, align, window = _mask_choice(rng, Nq, Nkv)
        nb = int(rng.integers(1, 5))
        ql = [int(x) for x in rng.integers(0, 300, nb)]
        out.append(dict(i=i, packed=packed, B=int(rng.integers(1, 3)), Hq=Hkv * int(rng.choice([1, 2, 4])),
                        Hkv=Hkv, Nq=Nq, Nkv=Nkv, ql=ql, kl=ql if rng.integers(0, 2) else
                        [int(x) for x in rng.integers(0, 300, nb)], D=int(rng.choice([64, 128])),
                        dtype=str(rng.choice(["fp16", "bf16"])), causal=causal, align=align, window=window))
    return out


@pytest.mark.parametrize("cs", _bwd_cases(), ids=lambda c: f"bwd{c['i']}{'_packed' if c['packed'] else ''}")
def test_sweep_backward(cs):
    _say(cs)
    g = torch.Generator().manual_seed(9300 + cs["i"])
    Hq, Hkv, D, dt = cs["Hq"], cs["Hkv"], cs["D"], cs["dtype"]
    win, br = cs["window"], cs["align"] == "bottom_right"
    scale = D ** -0.5
    if cs["packed"]:
        case = W.VarlenPrefillCase(f"bsweep{cs['i']}", tuple(cs["ql"]), tuple(cs["kl"]), Hq, Hkv, D, dt,
                                   cs["causal"], br, seed=9400 + cs["i"])
        if case.total_q == 0 or case.total_k == 0:
            pytest.skip("empty packed batch")
        q, k, v = W.varlen_prefill_inputs(case)
        do = _rand(q.shape, dt, g)
        cq = torch.tensor(case.cu_q, dtype=torch.int32, device=DEV)
        ck = torch.tensor(case.cu_k, dtype=torch.int32, device=DEV)
        qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
        mq, mk = max(case.max_q, 1), max(max(case.k_lens), 1)
        o, l = A.attn_fwd_varlen(qd, kd, vd, cq, ck, mq, causal=cs["causal"], causal_align=cs["align"], window=win,
                                 scale=scale, return_lse=True)
        dq, dk, dv = A.attn_bwd_varlen(qd, kd, vd, o, dod, l, cq, ck, mq, mk, causal=cs["causal"],
                                       causal_align=cs["align"], window=win, scale=scale)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.attention_varlen_backward(_np(q), _np(k), _np(v), _np(do), case.cu_q, case.cu_k, scale,
                                                      cs["causal"], bottom_right=br, window=win or (-1, -1))
        Lq, Lk = max(case.q_lens), max(case.k_lens)
    else:
        B, Nq, Nkv = cs["B"], cs["Nq"], cs["Nkv"]
        q, k, v = _rand((B, Hq, Nq, D), dt, g), _rand((B, Hkv, Nkv, D), dt, g), _rand((B, Hkv, Nkv, D), dt, g)
        do = _rand(q.shape, dt, g)
        qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
        o, l = A.attn_fwd(qd, kd, vd, causal=cs["causal"], causal_align=cs["align"], window=win, scale=scale,
                          return_lse=True)
        dq, dk, dv = A.attn_bwd(qd, kd, vd, o, dod, l, causal=cs["causal"], causal_align=cs["align"], window=win,
                                scale=scale)
        torch.cuda.synchronize()
        masked = cs["causal"] or win is not None
        off = Nkv - Nq if (masked and br) else 0
        rq, rk, rv = oracle.attention_backward(_np(q), _np(k), _np(v), _np(do), scale, cs["causal"],
                                               causal_offset=off, window=win or (-1, -1))
        Lq, Lk = Nq, Nkv
    _check("dQ", dq, rq, _DT[dt], _floor(D, Lk, do, v.float(), scale, k.float()))
    _check("dK", dk, rk, _DT[dt], _floor(D, Lq, do, v.float(), scale, q.float()))
    _check("dV", dv, rv, _DT[dt])
