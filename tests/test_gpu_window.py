"""GPU parity of sliding-window (band) masks against the fp64 oracle:
attn_fwd_masked / attn_fwd_varlen_masked for prefill and attn_decode_ex for
decode over contiguous, per-sequence and paged caches.

Decode runs poison every hidden slot (before the window and past the length)
with NaN on the GPU side, so a read of any of them shows up in the output; the
oracle is given the clean caches.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_attn_fwd_05_amd as A
import oracle
import workloads as W
from gpu_util import O_TOL, check_lse, check_o, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _np(t):
    return t.float().numpy().astype(np.float64)


def _compare(o, l, Oref, Lref, dtype):
    """o (..., R, D) / l (..., R) against the oracle; rows with no visible key
    must be exactly o = 0 and lse = -inf."""
    o, l = o.cpu(), l.cpu()
    empty = torch.from_numpy(~np.isfinite(Lref))
    if empty.any():
        assert torch.all(l[empty] == float("-inf")) and torch.all(o[empty] == 0)
    live = ~empty
    e = check_o(o[live], Oref[live.numpy()], dtype)
    r = check_lse(l[live], Lref[live.numpy()])
    print(f"    max|dO| = {e:.3e} (tol {O_TOL[dtype]}), worst lse err/bound = {r:.3f}", flush=True)


BANDS = [
    # name, B, Hq, Hkv, Nq, Nkv, D, dtype, align, causal, window
    ("causal_window256", 2, 8, 2, 1000, 1000, 128, "fp16", "top_left", True, (255, -1)),
    ("two_sided", 1, 8, 8, 777, 777, 64, "bf16", "top_left", False, (100, 37)),
    ("right_only", 1, 4, 1, 500, 500, 128, "fp16", "top_left", False, (-1, 64)),
    ("diagonal_only", 1, 4, 2, 300, 300, 128, "fp16", "top_left", False, (0, 0)),
    ("chunk_causal_window", 2, 8, 2, 300, 1500, 128, "fp16", "bottom_right", True, (511, -1)),
    ("left_only_br", 1, 4, 2, 400, 900, 64, "fp16", "bottom_right", False, (200, -1)),
    ("ragged_small_window", 1, 4, 4, 1, 129, 128, "bf16", "bottom_right", True, (3, -1)),
    ("q_longer_than_k", 1, 4, 2, 700, 300, 128, "fp16", "bottom_right", True, (64, -1)),
    # window sides at INT32_MAX: opened on the host (they reach past every key)
    ("right_side_int_max", 1, 4, 2, 300, 700, 128, "fp16", "top_left", False, (-1, 2 ** 31 - 1)),
    ("br_left_int_max_q_longer", 1, 4, 2, 700, 300, 128, "fp16", "bottom_right", True, (2 ** 31 - 1, -1)),
    ("both_sides_int_max", 1, 4, 4, 257, 513, 64, "bf16", "bottom_right", False, (2 ** 31 - 1, 2 ** 31 - 1)),
    ("left_int_max_right_5", 1, 4, 2, 500, 500, 128, "fp16", "top_left", False, (2 ** 31 - 1, 5)),
    # grids of more than 128 blocks of 256 rows, so masked ones keep their KV
    # ring with counters instead of barriers: a block whose rows see no key
    # runs no tile at all; one key per row; a 4-key window; a two-sided band
    ("grid_br_q_longer", 4, 16, 4, 700, 300, 128, "fp16", "bottom_right", True, (-1, -1)),
    ("grid_diagonal_only", 4, 16, 4, 600, 600, 64, "bf16", "top_left", False, (0, 0)),
    ("grid_br_window3", 4, 16, 4, 600, 900, 128, "fp16", "bottom_right", True, (3, -1)),
    ("grid_two_sided", 4, 16, 2, 777, 777, 64, "fp16", "top_left", False, (100, 37)),
    # the same grids with no band: ragged 256-row blocks, every row compared
    ("grid_causal_ragged", 4, 16, 4, 777, 777, 128, "fp16", "top_left", True, (-1, -1)),
    ("grid_full_ragged", 4, 16, 4, 777, 777, 64, "bf16", "top_left", False, (-1, -1)),
]


@pytest.mark.parametrize("band", BANDS, ids=[b[0] for b in BANDS])
def test_prefill_band(band):
    name, B, Hq, Hkv, Nq, Nkv, D, dtype, align, causal, window = band
    case = W.PrefillCase(name, B, Hq, Hkv, Nq, Nkv, D, dtype, causal, seed=W.BASE_SEED + 100 + len(name))
    q, k, v = W.prefill_inputs(case)
    _say(f"{name} align={align} causal={causal} window={window}")
    o, l = A.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, causal_align=align, window=window,
                      scale=case.softmax_scale, return_lse=True)
    torch.cuda.synchronize()
    off = 0 if align == "top_left" else Nkv - Nq
    Oref, Lref = oracle.attention_forward(_np(q), _np(k), _np(v), case.softmax_scale, causal, causal_offset=off,
                                          window=window)
    _compare(o, l, Oref, Lref, case.torch_dtype)


@pytest.mark.parametrize("window", [(300, 0), (200, 200)])
def test_prefill_band_rising_scores(window):
    """A band over scores that step up from each 64-key tile to the next: the
    reference max moves on every tile a row sees, on the band kernel's masked
    and unmasked tiles alike."""
    causal = window[1] == 0  # a two-sided band goes with no causal mask
    case = W.PrefillCase(f"band_rising_{window[0]}_{window[1]}", 2, 32, 8, 1000, 1000, 128, "fp16", causal,
                         seed=W.BASE_SEED + 180 + window[1])
    q, k, v = W.rising_score_inputs(case)
    _say(f"{case.name} window={window}")
    o, l = A.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window, scale=case.softmax_scale,
                      return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention_forward(_np(q), _np(k), _np(v), case.softmax_scale, causal, window=window)
    _compare(o, l, Oref, Lref, case.torch_dtype)


def test_prefill_band_identities_bitwise():
    """(-1, -1) is attn_fwd without a mask, (-1, 0) attn_fwd causal, and a
    causal window wider than the sequence takes the band path to the same bits."""
    case = W.PrefillCase("ident", 2, 8, 2, 1000, 1000, 128, "fp16", True, seed=W.BASE_SEED + 110)
    q, k, v = (t.to(DEV) for t in W.prefill_inputs(case))
    _say("band identities")
    for causal in (False, True):
        o1, l1 = A.attn_fwd(q, k, v, causal=causal, return_lse=True)
        o2, l2 = A.attn_fwd(q, k, v, causal=causal, window=(-1, -1), return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), causal
    o1, l1 = A.attn_fwd(q, k, v, causal=True, return_lse=True)
    o3, l3 = A.attn_fwd(q, k, v, causal=True, window=(5000, -1), return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


@pytest.mark.parametrize("window", [4095, 1000])
def test_prefill_band_serving_sampled(window):
    """Causal sliding window on the serving shape (B=2, Hq=32, Hkv=8, N=8192, D=128)."""
    case = W.serving(8192, True)
    q, k, v = W.prefill_inputs(case)
    rows = sample_rows(8192, True, np.random.default_rng(window))
    _say(f"{case.name} window={window} rows={len(rows)}")
    o, l = A.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, window=(window, -1), scale=case.softmax_scale,
                      return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention_forward(_np(q), _np(k), _np(v), case.softmax_scale, True, rows=rows,
                                          window=(window, -1))
    ri = torch.as_tensor(rows)
    assert torch.isfinite(o.float()).all()
    _compare(o[:, :, ri.to(DEV)], l[:, :, ri.to(DEV)], Oref, Lref, case.torch_dtype)


@pytest.mark.parametrize("align", ["top_left", "bottom_right"])
def test_prefill_varlen_band(align):
    case = W.VarlenPrefillCase("varlen_window", (1, 255, 700, 0, 1000, 64), (1, 300, 700, 20, 1300, 64), 8, 2, 128,
                               "fp16", True, align == "bottom_right", seed=W.BASE_SEED + 111)
    q, k, v = W.varlen_prefill_inputs(case)
    _say(f"{case.name} align={align}")
    cq = torch.tensor(case.cu_q, dtype=torch.int32, device=DEV)
    ck = torch.tensor(case.cu_k, dtype=torch.int32, device=DEV)
    o, l = A.attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq, ck, case.max_q, causal=True, causal_align=align,
                             window=(199, -1), scale=case.softmax_scale, return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention_varlen(_np(q), _np(k), _np(v), case.cu_q, case.cu_k, case.softmax_scale, True,
                                         bottom_right=align == "bottom_right", window=(199, -1))
    # packed layouts: o (T, Hq, D), lse (Hq, T)
    _compare(o.permute(1, 0, 2), l, Oref.transpose(1, 0, 2), Lref, case.torch_dtype)


# ---- decode

def _poison_outside(cache, lens, w):
    c = cache.clone()
    for b, L in enumerate(lens):
        lo = max(0, L - 1 - w) if w >= 0 else 0
        c[b, :, :lo] = float("nan")
        c[b, :, L:] = float("nan")
    return c


@pytest.mark.parametrize("w", [0, 1, 127, 128, 4095, 8191, 20000])
def test_decode_window(w):
    case = W.decode_case(8192)
    q, kc, vc = W.decode_inputs(case)
    _say(f"decode window={w}")
    L = case.cache_len
    kd, vd = _poison_outside(kc, [L] * case.B, w).to(DEV), _poison_outside(vc, [L] * case.B, w).to(DEV)
    o, l = A.attn_decode(q.to(DEV), kd, vd, L, scale=case.softmax_scale, window_left=w, return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.decode(_np(q), _np(kc), _np(vc), L, case.softmax_scale, window_left=w)
    check_o(o, Oref, case.torch_dtype)
    check_lse(l, Lref)


@pytest.mark.parametrize("w,ns", [(300, 0), (0, 0), (300, 1), (300, 2), (1000, 64)])
def test_decode_varlen_window(w, ns):
    case = W.DecodeCase("varlen_window", 6, 16, 4, 6000, 6000, 128, "fp16", seed=W.BASE_SEED + 112)
    q, kc, vc = W.decode_inputs(case)
    lens = [0, 1, 129, 5000, 301, 6000]
    _say(f"decode varlen window={w} splits={ns}")
    kd, vd = _poison_outside(kc, lens, w).to(DEV), _poison_outside(vc, lens, w).to(DEV)
    ld = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, l = A.attn_decode_varlen(q.to(DEV), kd, vd, ld, scale=case.softmax_scale, window_left=w, num_splits=ns,
                                return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.decode_varlen(_np(q), _np(kc), _np(vc), lens, case.softmax_scale, window_left=w)
    assert torch.all(o[0] == 0) and torch.all(l[0] == float("-inf"))
    check_o(o[1:], Oref[1:], case.torch_dtype)
    check_lse(l[1:], Lref[1:])


@pytest.mark.parametrize("ps", [16, 128])
def test_decode_paged_window(ps):
    from test_gpu_decode_paged import make_paged
    case = W.DecodeCase("paged_window", 4, 8, 2, 2048, 2048, 128, "bf16", seed=W.BASE_SEED + 113)
    q, kc, vc = W.decode_inputs(case)
    lens, w = [2048, 17, 700, 0], 250
    _say(f"decode paged ps={ps} window={w}")
    # hidden slots poisoned before the scatter; the pages holding only hidden
    # slots get an out-of-range id in the block table, which must never be read
    kp, vp, tbl = make_paged(_poison_outside(kc, lens, w), _poison_outside(vc, lens, w), lens, ps, seed=ps)
    for b, L in enumerate(lens):
        lo = max(0, L - 1 - w)
        tbl[b, :lo // ps] = -1
    ld = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, l = A.attn_decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), tbl.to(DEV), ld, scale=case.softmax_scale,
                               window_left=w, return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.decode_varlen(_np(q), _np(kc), _np(vc), lens, case.softmax_scale, window_left=w)
    assert torch.all(o[3] == 0) and torch.all(l[3] == float("-inf"))
    check_o(o[:3], Oref[:3], case.torch_dtype)
    check_lse(l[:3], Lref[:3])
