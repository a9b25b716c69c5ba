"""GPU parity of attn_bwd (dQ, dK, dV) against the fp64 oracle.

The GPU backward takes the GPU forward's O and lse, as a training step would.
Tolerance, per gradient tensor X: max|X_gpu - X_oracle| <= 4 u max|X_oracle|
+ floor, u = 2^-11 (fp16) or 2^-8 (bf16).  Each gradient element is a sum of
products in which one factor was rounded once to 16 bits (P for dV, dS for dQ
and dK), and delta comes from the forward's 16-bit O; the rows of dS sum to
zero, so small elements are differences of large terms, which is why the
bound is relative to the tensor's largest element rather than to each
element.  The floor covers the fp32 rounding of dP - delta (two sums of D
products, each at most max|dO| max|V|) carried into dQ (dK) by one more
product with scale K (Q) per key (query): 2^-24 D N max|dO| max|V| |scale|
max|K| (resp. max|Q|); it matters only where the exact gradient is 0 (one key:
dS = 0).  Under an earlier bound of 16 u the largest error any backward test
measured was 8 % of it, 1.3 u max|X|; 4 u leaves a factor of about 3.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_attn_fwd_05_amd as A
import oracle
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
TOL_U = 4  # multiples of u * max|X_oracle|


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _floor(D, N, do, v, scale, x):
    return 2.0 ** -24 * D * N * float(do.abs().max()) * float(v.abs().max()) * abs(scale) * float(x.abs().max())


def _check(name, got, ref, dtype, floor=0.0):
    g = _np(got)
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    err = float(np.abs(g - ref).max())
    scale = float(np.abs(ref).max())
    tol = TOL_U * U[dtype] * scale + floor
    print(f"    {name}: max|err| = {err:.3e}, max|ref| = {scale:.3e}, err/tol = {err / tol:.3f}", flush=True)
    assert err <= tol, f"{name}: max|err| {err:.3e} > {tol:.3e}"


def run_bwd(name, B, Hq, Hkv, Nq, Nkv, D, dtype, causal, align="top_left", seed=0, window=None, rising=False):
    case = W.PrefillCase(name, B, Hq, Hkv, Nq, Nkv, D, dtype, causal, seed=W.BASE_SEED + 120 + seed)
    q, k, v = W.rising_score_inputs(case) if rising else W.prefill_inputs(case)
    g = torch.Generator().manual_seed(W.BASE_SEED + 220 + seed)
    do = torch.randn(B, Hq, Nq, D, generator=g).to(case.torch_dtype)
    _say(f"{name} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} D={D} {dtype} causal={causal} align={align} "
         f"window={window}")
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = A.attn_fwd(qd, kd, vd, causal=causal, causal_align=align, scale=case.softmax_scale, return_lse=True,
                        window=window)
    dq, dk, dv = A.attn_bwd(qd, kd, vd, o, dod, lse, causal=causal, causal_align=align, scale=case.softmax_scale,
                            window=window)
    torch.cuda.synchronize()
    off = Nkv - Nq if ((causal or window is not None) and align == "bottom_right") else 0
    rq, rk, rv = oracle.attention_backward(_np(q), _np(k), _np(v), _np(do), case.softmax_scale, causal,
                                           causal_offset=off, window=window or (-1, -1))
    sc = case.softmax_scale
    _check("dQ", dq, rq, case.torch_dtype, _floor(D, Nkv, do, v.float(), sc, k.float()))
    _check("dK", dk, rk, case.torch_dtype, _floor(D, Nq, do, v.float(), sc, q.float()))
    _check("dV", dv, rv, case.torch_dtype)
    return dq, dk, dv


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_bwd_rising_scores(causal):
    """Scores that step up by ~16 log2 units per 64-key tile (lse up to ~170):
    P = exp(S scale - lse) spans the whole fp32 range along each row."""
    run_bwd("bwd_rising", 1, 4, 2, 1000, 1000, 128, "fp16", causal, seed=60 + causal, rising=True)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("N", [1, 65, 257, 1000])
def test_bwd_lengths(N, causal):
    run_bwd(f"bwd_n{N}", 1, 4, 2, N, N, 128, "fp16", causal, seed=N)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (8, 1)])
@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (128, "bf16"), (64, "fp16")])
def test_bwd_heads_dtypes(Hq, Hkv, D, dtype):
    run_bwd(f"bwd_h{Hq}_{Hkv}_d{D}_{dtype}", 2, Hq, Hkv, 515, 515, D, dtype, True, seed=Hq + Hkv + D)


@pytest.mark.parametrize("Nq,Nkv", [(300, 1000), (700, 300), (1, 777)])
def test_bwd_bottom_right(Nq, Nkv):
    run_bwd(f"bwd_br_{Nq}_{Nkv}", 1, 4, 2, Nq, Nkv, 128, "fp16", True, align="bottom_right", seed=Nq)


BWD_BANDS = [
    # name, Nq, Nkv, D, dtype, causal, align, window
    ("causal_window256", 1000, 1000, 128, "fp16", True, "top_left", (255, -1)),
    ("two_sided", 777, 777, 64, "bf16", False, "top_left", (100, 37)),
    ("zero_width", 300, 300, 128, "fp16", False, "top_left", (0, 0)),
    ("chunk_window", 300, 1500, 128, "fp16", True, "bottom_right", (511, -1)),
    ("left_only_br", 400, 900, 64, "fp16", False, "bottom_right", (200, -1)),
    ("right_only", 500, 500, 128, "bf16", False, "top_left", (-1, 64)),
    # window sides at INT32_MAX: opened on the host (they reach past every key)
    ("right_side_int_max", 300, 700, 128, "fp16", False, "top_left", (-1, 2 ** 31 - 1)),
    ("br_left_int_max_q_longer", 700, 300, 128, "fp16", True, "bottom_right", (2 ** 31 - 1, -1)),
    ("left_int_max_right_5", 500, 500, 64, "bf16", False, "top_left", (2 ** 31 - 1, 5)),
]


@pytest.mark.parametrize("band", BWD_BANDS, ids=[b[0] for b in BWD_BANDS])
def test_bwd_band(band):
    name, Nq, Nkv, D, dtype, causal, align, window = band
    run_bwd(f"bwd_{name}", 1, 4, 2, Nq, Nkv, D, dtype, causal, align=align, seed=Nq + Nkv, window=window)


def test_bwd_band_wider_than_sequence_is_causal_bitwise():
    case = W.PrefillCase("bwd_wide", 2, 8, 2, 1000, 1000, 128, "fp16", True, seed=W.BASE_SEED + 132)
    q, k, v = (t.to(DEV) for t in W.prefill_inputs(case))
    do = torch.randn_like(q)
    _say(case.name)
    o, lse = A.attn_fwd(q, k, v, causal=True, return_lse=True)
    g1 = A.attn_bwd(q, k, v, o, do, lse, causal=True)
    g2 = A.attn_bwd(q, k, v, o, do, lse, causal=True, window=(5000, -1))
    torch.cuda.synchronize()
    for a_, b_ in zip(g1, g2):
        assert torch.equal(a_, b_)


def test_bwd_cross_lengths_full():
    run_bwd("bwd_cross", 2, 4, 1, 200, 1300, 64, "bf16", False, seed=7)


def test_bwd_deterministic():
    """No atomics: two runs give the same bits."""
    case = W.PrefillCase("bwd_det", 2, 8, 2, 1024, 1024, 128, "fp16", True, seed=W.BASE_SEED + 130)
    q, k, v = (t.to(DEV) for t in W.prefill_inputs(case))
    do = torch.randn_like(q)
    _say(case.name)
    o, lse = A.attn_fwd(q, k, v, causal=True, return_lse=True)
    g1 = A.attn_bwd(q, k, v, o, do, lse, causal=True)
    g2 = A.attn_bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for a_, b_ in zip(g1, g2):
        assert torch.equal(a_, b_)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_bwd_serving_slices(causal):
    """The serving shape (B=2, Hq=32, Hkv=8, N=4096, D=128): the gradients of
    two (batch, kv head) groups against the oracle on those slices."""
    case = W.serving(4096, causal)
    q, k, v = W.prefill_inputs(case)
    g = torch.Generator().manual_seed(W.BASE_SEED + 131)
    do = torch.randn(q.shape, generator=g).half()
    _say(f"{case.name} slices")
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = A.attn_fwd(qd, kd, vd, causal=causal, scale=case.softmax_scale, return_lse=True)
    dq, dk, dv = A.attn_bwd(qd, kd, vd, o, dod, lse, causal=causal, scale=case.softmax_scale)
    torch.cuda.synchronize()
    G = case.Hq // case.Hkv
    for b, kvh in ((0, 0), (1, 7)):
        hs = slice(kvh * G, (kvh + 1) * G)
        rq, rk, rv = oracle.attention_backward(_np(q[b:b + 1, hs]), _np(k[b:b + 1, kvh:kvh + 1]),
                                               _np(v[b:b + 1, kvh:kvh + 1]), _np(do[b:b + 1, hs]),
                                               case.softmax_scale, causal)
        sc = case.softmax_scale
        _check(f"dQ[{b},{kvh}]", dq[b:b + 1, hs], rq, torch.float16, _floor(128, 4096, do, v.float(), sc, k.float()))
        _check(f"dK[{b},{kvh}]", dk[b:b + 1, kvh:kvh + 1], rk, torch.float16,
               _floor(128, 4096, do, v.float(), sc, q.float()))
        _check(f"dV[{b},{kvh}]", dv[b:b + 1, kvh:kvh + 1], rv, torch.float16)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_bwd_remapped_grid_matches_per_unit_calls(causal):
    """The serving shape (B=2, Hq=32, Hkv=8, N=2048, D=128) runs both backward
    passes in the XCD-aware block order (its grids split into whole (batch, kv
    head) units per XCD); each unit run alone (B=1, Hkv=1: a grid too small for
    that order) must give the same bits for every unit's dQ, dK and dV."""
    case = W.serving(2048, causal)
    q, k, v = (t.to(DEV) for t in W.prefill_inputs(case))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(W.BASE_SEED + 133)).half().to(DEV)
    _say(f"{case.name} remapped grid vs per-unit calls")
    sc = case.softmax_scale
    o, lse = A.attn_fwd(q, k, v, causal=causal, scale=sc, return_lse=True)
    dq, dk, dv = A.attn_bwd(q, k, v, o, do, lse, causal=causal, scale=sc)
    G = case.Hq // case.Hkv
    for b in range(case.B):
        for kvh in range(case.Hkv):
            hs = slice(kvh * G, (kvh + 1) * G)
            qs, ks, vs = q[b:b + 1, hs].contiguous(), k[b:b + 1, kvh:kvh + 1].contiguous(), v[b:b + 1, kvh:kvh + 1].contiguous()
            os_, dos, ls = o[b:b + 1, hs].contiguous(), do[b:b + 1, hs].contiguous(), lse[b:b + 1, hs].contiguous()
            gq, gk, gv = A.attn_bwd(qs, ks, vs, os_, dos, ls, causal=causal, scale=sc)
            torch.cuda.synchronize()
            assert torch.equal(gq, dq[b:b + 1, hs]), (b, kvh, "dQ")
            assert torch.equal(gk, dk[b:b + 1, kvh:kvh + 1]), (b, kvh, "dK")
            assert torch.equal(gv, dv[b:b + 1, kvh:kvh + 1]), (b, kvh, "dV")
