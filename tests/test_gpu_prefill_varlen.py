"""GPU parity of attn_fwd_varlen (packed sequences of different lengths)
against the fp64 oracle, plus bitwise equivalences with attn_fwd.

Every case prints its name before touching the GPU so a failure is attributable.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_attn_fwd_05_amd as A
import oracle
import workloads as W
from gpu_util import O_TOL, check_lse, check_o

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENTINEL = 7.0


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _np(t):
    return t.float().numpy().astype(np.float64)


def _cu(lens):
    return torch.tensor(W.VarlenPrefillCase._cu(lens), dtype=torch.int32, device=DEV)


def _compare(o, l, Oref, Lref, dtype):
    """o (R, Hq, D) / l (Hq, R) from the GPU against the oracle; rows that see
    no key must be exactly o = 0 and lse = -inf."""
    o, l = o.cpu(), l.cpu()
    empty = ~np.isfinite(Lref)  # (Hq, R)
    if empty.any():
        assert torch.all(l[torch.from_numpy(empty)] == float("-inf"))
        e_rows = torch.from_numpy(empty.T)  # (R, Hq)
        assert torch.all(o[e_rows] == 0)
    live = ~empty
    if live.any():
        lt = torch.from_numpy(live)
        e = check_o(o[lt.T], Oref[live.T], dtype)
        r = check_lse(l[lt], Lref[live])
        print(f"    max|dO| = {e:.3e} (tol {O_TOL[dtype]}), worst lse err/bound = {r:.3f}", flush=True)


def run_varlen(case: W.VarlenPrefillCase, rows=None, max_seqlen_q=None):
    q, k, v = W.varlen_prefill_inputs(case)
    _say(f"{case.name} q_lens={case.q_lens} k_lens={case.k_lens} causal={case.causal} "
         f"bottom_right={case.bottom_right} max_seqlen_q={max_seqlen_q}")
    o, l = A.attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), _cu(case.q_lens), _cu(case.k_lens),
                             max_seqlen_q or case.max_q, causal=case.causal, scale=case.softmax_scale,
                             return_lse=True, causal_align="bottom_right" if case.bottom_right else "top_left")
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention_varlen(_np(q), _np(k), _np(v), case.cu_q, case.cu_k, case.softmax_scale,
                                         case.causal, bottom_right=case.bottom_right, rows=rows)
    if rows is None:
        _compare(o, l, Oref, Lref, case.torch_dtype)
    else:
        ri = torch.as_tensor(rows)
        _compare(o[ri.to(DEV)], l[:, ri.to(DEV)], Oref, Lref, case.torch_dtype)
    return o, l


MODES = [(False, False), (True, False), (True, True)]
MODE_IDS = ["full", "top_left", "bottom_right"]


@pytest.mark.parametrize("causal,br", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("Hq,Hkv,D,dtype", [(8, 2, 128, "fp16"), (4, 1, 64, "bf16"), (8, 8, 128, "bf16")])
def test_varlen_mixed_lengths(causal, br, Hq, Hkv, D, dtype):
    """Lengths across the 256-row query block and 64-key tile boundaries, incl. 0 and 1."""
    lens = (1, 255, 256, 257, 0, 700, 64, 1000)
    run_varlen(W.VarlenPrefillCase(f"mixed_h{Hq}_{Hkv}_d{D}_{dtype}", lens, lens, Hq, Hkv, D, dtype, causal, br,
                                   seed=W.BASE_SEED + 80 + D + Hkv))


@pytest.mark.parametrize("causal,br", MODES, ids=MODE_IDS)
def test_varlen_queries_differ_from_keys(causal, br):
    """L_q < L_k (chunks at the end of a context), L_q > L_k (bottom-right: the
    first L_q - L_k rows see nothing), queries with no keys and keys with no queries."""
    case = W.VarlenPrefillCase("chunks", (100, 256, 1, 300, 0, 5, 129), (1000, 256, 4000, 100, 50, 0, 129),
                               8, 2, 128, "fp16", causal, br, seed=W.BASE_SEED + 85)
    run_varlen(case)


@pytest.mark.parametrize("causal,br", MODES, ids=MODE_IDS)
def test_varlen_rising_scores(causal, br):
    """Two packed sequences (1000 and 700 rows) of the rising-score inputs: the
    reference max moves on every tile the packed kernel visits."""
    case = W.PrefillCase("varlen_rising", 2, 4, 2, 1000, 1000, 128, "fp16", causal, seed=W.BASE_SEED + 190 + causal + br)
    q, k, v = W.rising_score_inputs(case)
    lens = [1000, 700]
    pack = lambda x: torch.cat([x[0].transpose(0, 1), x[1, :, :lens[1]].transpose(0, 1)]).contiguous()  # noqa: E731
    qp, kp, vp = pack(q), pack(k), pack(v)
    cu = [0, lens[0], lens[0] + lens[1]]
    _say(f"varlen rising causal={causal} bottom_right={br}")
    o, l = A.attn_fwd_varlen(qp.to(DEV), kp.to(DEV), vp.to(DEV), _cu(lens), _cu(lens), max(lens), causal=causal,
                             scale=case.softmax_scale, return_lse=True,
                             causal_align="bottom_right" if br else "top_left")
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention_varlen(_np(qp), _np(kp), _np(vp), cu, cu, case.softmax_scale, causal,
                                         bottom_right=br)
    _compare(o, l, Oref, Lref, case.torch_dtype)


@pytest.mark.parametrize("N", [1000, 6500], ids=["short_128row", "long_256row"])
def test_varlen_equal_lengths_is_fwd_bitwise(N):
    """B equal-length sequences packed: identical bits to attn_fwd on the (B, N, H, D) layout.
    attn_fwd runs 256-row blocks of one key group (a grid of 3 x 32 heads x >= 4 query
    blocks); the packed path runs 128-row blocks of 4 waves for a mean length of 1000 and
    256-row blocks for 6500 (above the 6144-row mean where it switches), the same per-row
    arithmetic either way."""
    B, Hq, Hkv, D = 3, 32, 8, 128
    _say(f"varlen vs attn_fwd, equal lengths N={N}")
    g = torch.Generator().manual_seed(W.BASE_SEED + 86)
    q = torch.randn(B, N, Hq, D, generator=g).half().to(DEV)
    k = torch.randn(B, N, Hkv, D, generator=g).half().to(DEV)
    v = torch.randn(B, N, Hkv, D, generator=g).half().to(DEV)
    cu = _cu([N] * B)
    for causal, align in ((True, "top_left"), (False, "top_left"), (True, "bottom_right")):
        o1, l1 = A.attn_fwd(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), causal=causal,
                            return_lse=True, causal_align=align)
        o2, l2 = A.attn_fwd_varlen(q.reshape(B * N, Hq, D), k.reshape(B * N, Hkv, D), v.reshape(B * N, Hkv, D),
                                   cu, cu, N, causal=causal, return_lse=True, causal_align=align)
        torch.cuda.synchronize()
        assert torch.equal(o1.transpose(1, 2).reshape(B * N, Hq, D), o2), (causal, align)
        assert torch.equal(l1.permute(1, 0, 2).reshape(Hq, B * N), l2), (causal, align)


def test_varlen_chunk_is_fwd_bottom_right_bitwise():
    """One packed chunk of 300 queries against 2000 keys equals attn_fwd bottom-right bit for bit
    (72 heads x 2 query blocks: a grid large enough for 256-row blocks on both paths)."""
    Lq, Lk, Hq, Hkv, D = 300, 2000, 72, 8, 64
    _say("varlen chunk vs attn_fwd bottom_right")
    g = torch.Generator().manual_seed(W.BASE_SEED + 87)
    q = torch.randn(Lq, Hq, D, generator=g).bfloat16().to(DEV)
    k = torch.randn(Lk, Hkv, D, generator=g).bfloat16().to(DEV)
    v = torch.randn(Lk, Hkv, D, generator=g).bfloat16().to(DEV)
    o1, l1 = A.attn_fwd(q.transpose(0, 1)[None], k.transpose(0, 1)[None], v.transpose(0, 1)[None], causal=True,
                        return_lse=True, causal_align="bottom_right")
    o2, l2 = A.attn_fwd_varlen(q, k, v, _cu([Lq]), _cu([Lk]), Lq, causal=True, return_lse=True,
                               causal_align="bottom_right")
    torch.cuda.synchronize()
    assert torch.equal(o1[0].transpose(0, 1), o2)
    assert torch.equal(l1[0], l2)


def test_varlen_neighbour_nan_never_leaks():
    """NaN in every Q/K/V row of sequence 1 leaves sequences 0 and 2 exact."""
    case = W.VarlenPrefillCase("nan_neighbour", (130, 70, 300), (130, 70, 300), 4, 2, 128, "fp16", True,
                               seed=W.BASE_SEED + 88)
    q, k, v = W.varlen_prefill_inputs(case)
    _say(case.name)
    cq, ck = case.cu_q, case.cu_k
    for t, cu in ((q, cq), (k, ck), (v, ck)):
        t[cu[1]:cu[2]] = float("nan")
    o, l = A.attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), _cu(case.q_lens), _cu(case.k_lens), case.max_q,
                             causal=True, return_lse=True)
    torch.cuda.synchronize()
    rows = np.r_[cq[0]:cq[1], cq[2]:cq[3]]
    Oref, Lref = oracle.attention_varlen(_np(q), _np(k), _np(v), cq, ck, case.softmax_scale, True, rows=rows)
    ri = torch.as_tensor(rows).to(DEV)
    _compare(o[ri], l[:, ri], Oref, Lref, case.torch_dtype)


@pytest.mark.parametrize("br", [False, True], ids=["top_left", "bottom_right"])
def test_varlen_max_seqlen_caps_rows(br):
    """Rows at positions >= max_seqlen_q are left untouched; the rows computed
    keep the whole sequence's mask (bottom-right offset from the true lengths)."""
    case = W.VarlenPrefillCase("capped", (600, 100, 300), (900, 100, 300), 4, 1, 128, "fp16", True, br,
                               seed=W.BASE_SEED + 89)
    cap = 260
    q, k, v = W.varlen_prefill_inputs(case)
    _say(f"{case.name} cap={cap} bottom_right={br}")
    o = torch.full((case.total_q, case.Hq, case.D), SENTINEL, dtype=torch.float16, device=DEV)
    lse = torch.full((case.Hq, case.total_q), SENTINEL, dtype=torch.float32, device=DEV)
    A.attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), _cu(case.q_lens), _cu(case.k_lens), cap, causal=True,
                      out=o, lse=lse, causal_align="bottom_right" if br else "top_left")
    torch.cuda.synchronize()
    cq = case.cu_q
    done = np.concatenate([np.arange(cq[b], cq[b] + min(cap, case.q_lens[b])) for b in range(case.B)])
    skipped = np.setdiff1d(np.arange(case.total_q), done)
    assert skipped.size == (600 - cap) + (300 - cap)
    assert torch.all(o[torch.as_tensor(skipped).to(DEV)] == SENTINEL)
    assert torch.all(lse[:, torch.as_tensor(skipped).to(DEV)] == SENTINEL)
    Oref, Lref = oracle.attention_varlen(_np(q), _np(k), _np(v), cq, case.cu_k, case.softmax_scale, True,
                                         bottom_right=br, rows=done)
    di = torch.as_tensor(done).to(DEV)
    _compare(o[di], lse[:, di], Oref, Lref, case.torch_dtype)


def test_varlen_malformed_offsets_stay_in_bounds():
    """Decreasing and out-of-range offsets are clamped on the device: the call
    completes, writes nothing outside its tensors (guard rows after them stay
    untouched), and a following well-formed call is still exact."""
    Hq, Hkv, D, T = 4, 2, 64, 700
    _say("malformed offsets")
    g = torch.Generator().manual_seed(W.BASE_SEED + 90)
    q = torch.randn(T + 64, Hq, D, generator=g).half().to(DEV)
    k = torch.randn(T + 64, Hkv, D, generator=g).half().to(DEV)
    v = torch.randn(T + 64, Hkv, D, generator=g).half().to(DEV)
    o = torch.full((T + 64, Hq, D), SENTINEL, dtype=torch.float16, device=DEV)
    lse = torch.full((Hq, T + 64), SENTINEL, dtype=torch.float32, device=DEV)
    bad = torch.tensor([0, 500, 300, 9999, -5], dtype=torch.int32, device=DEV)
    A.attn_fwd_varlen(q[:T], k[:T], v[:T], bad, bad, 1000, causal=True, out=o[:T], lse=None)
    torch.cuda.synchronize()
    assert torch.all(o[T:] == SENTINEL)
    case = W.VarlenPrefillCase("after_malformed", (300, 400), (300, 400), Hq, Hkv, D, "fp16", True,
                               seed=W.BASE_SEED + 91)
    run_varlen(case)


def test_varlen_long_mixed_sampled():
    """A packed batch of long sequences (mean 7000 rows: 256-row blocks) against the
    oracle on the first, last and two inner rows of every sequence, causal and not."""
    lens = (5000, 9000, 7000)
    for causal in (True, False):
        case = W.VarlenPrefillCase(f"long_mixed_{'causal' if causal else 'full'}", lens, lens, 16, 4, 128, "fp16",
                                   causal, seed=W.BASE_SEED + 192)
        cq = case.cu_q
        rows = sorted({r for b in range(case.B)
                       for r in (cq[b], cq[b] + 255, cq[b] + 256, (cq[b] + cq[b + 1]) // 2, cq[b + 1] - 1)})
        run_varlen(case, rows=np.array(rows))


def test_varlen_serving_batch_sampled():
    """The 16-sequence packed serving batch (lengths up to 4096, Hq=32, D=128):
    the first, last and a middle row of every sequence against the oracle."""
    case = W.varlen_serving_case()
    cq = case.cu_q
    rows = sorted({r for b in range(case.B) for r in (cq[b], (cq[b] + cq[b + 1]) // 2, cq[b + 1] - 1)})
    run_varlen(case, rows=np.array(rows))
