"""GPU parity of attn_decode_paged and kv_cache_write_paged against the fp64
oracle, plus bitwise equivalence with attn_decode_varlen on the same rows.

Contiguous caches are scattered into a shuffled page pool; spare pages and the
slots past each sequence's length hold NaN, so any read outside a sequence's
first cache_lens[b] slots shows up in the output.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_attn_fwd_05_amd as A
import oracle
import workloads as W
from gpu_util import check_lse, check_o

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _np(t):
    return t.float().numpy().astype(np.float64)


def make_paged(kc, vc, lens, ps, seed, spare=5):
    """Scatter (B, Hkv, S, D) caches into a shuffled (P, Hkv, ps, D) pool.

    Slots >= lens[b] and the spare pages are NaN.  Returns (k_pool, v_pool,
    table) on the CPU; table is int32 (B, S // ps)."""
    B, H, S, D = kc.shape
    assert S % ps == 0
    npb = S // ps
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(B * npb + spare, generator=g)[:B * npb]
    pools = []
    for c in (kc, vc):
        c = c.clone()
        for b, L in enumerate(lens):
            c[b, :, L:] = float("nan")
        pool = torch.full((B * npb + spare, H, ps, D), float("nan"), dtype=c.dtype)
        pool[perm] = c.reshape(B, H, npb, ps, D).permute(0, 2, 1, 3, 4).reshape(B * npb, H, ps, D)
        pools.append(pool)
    return pools[0], pools[1], perm.reshape(B, npb).to(torch.int32)


def run_paged(case: W.DecodeCase, lens, ps, num_splits=0, max_len=None):
    q, kc, vc = W.decode_inputs(case)
    _say(f"{case.name} paged ps={ps} lens={list(lens)} splits={num_splits} max_len={max_len}")
    kp, vp, tbl = make_paged(kc, vc, lens, ps, seed=case.seed + ps)
    ld = torch.tensor(list(lens), dtype=torch.int32, device=DEV)
    o, l = A.attn_decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), tbl.to(DEV), ld, max_len,
                               scale=case.softmax_scale, num_splits=num_splits, return_lse=True)
    torch.cuda.synchronize()
    Oref, Lref = oracle.decode_paged(_np(q), _np(kp), _np(vp), tbl.numpy(), list(lens), ps, case.softmax_scale)
    live = [b for b, L in enumerate(lens) if L > 0]
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.all(o[b] == 0) and torch.all(l[b] == float("-inf")), f"sequence {b} of length 0"
    e = check_o(o[live], Oref[live], case.torch_dtype)
    r = check_lse(l[live], Lref[live])
    print(f"    max|dO| = {e:.3e}, worst lse err/bound = {r:.3f}", flush=True)
    return o, l


@pytest.mark.parametrize("ps", [16, 32, 64, 128, 256])
def test_paged_page_sizes(ps):
    """Lengths across page, tile (128) and chunk boundaries, incl. 0 and 1."""
    case = W.DecodeCase("paged_h32_8_d128", 5, 32, 8, 1024, 1024, 128, "fp16", seed=W.BASE_SEED + 92)
    run_paged(case, [1000, 1, 0, 513, 1024], ps)


@pytest.mark.parametrize("dtype,D,Hkv,ps", [("bf16", 64, 1, 16), ("bf16", 128, 2, 32), ("fp16", 64, 8, 128)])
def test_paged_dtypes_heads(dtype, D, Hkv, ps):
    case = W.DecodeCase(f"paged_{dtype}_d{D}_hkv{Hkv}", 3, 8, Hkv, 512, 512, D, dtype, seed=W.BASE_SEED + 93 + D)
    run_paged(case, [300, 17, 512], ps)


@pytest.mark.parametrize("ns", [1, 3, 64])
def test_paged_split_counts(ns):
    case = W.DecodeCase("paged_splits", 4, 8, 4, 2048, 2048, 128, "fp16", seed=W.BASE_SEED + 94)
    run_paged(case, [2048, 1537, 0, 129], 16, num_splits=ns)


def test_paged_max_len_bound():
    case = W.DecodeCase("paged_bound", 3, 8, 8, 1024, 1024, 128, "fp16", seed=W.BASE_SEED + 95)
    run_paged(case, [700, 33, 256], 64, max_len=700)


def test_paged_equals_varlen_bitwise():
    """The serving batch (16 sequences, seeded lengths up to 8192) in a
    (B, S, Hkv, D) cache read as 16-row pages in order gives the same bits as
    attn_decode_varlen on that cache."""
    case = W.decode_varlen_case()
    q, kc, vc = W.decode_inputs(case)
    lens = W.decode_varlen_lens(case)
    _say(f"paged vs varlen, {case.name}")
    ps = 16
    B, H, S, D = kc.shape
    kb = kc.permute(0, 2, 1, 3).contiguous().to(DEV)  # (B, S, Hkv, D)
    vb = vc.permute(0, 2, 1, 3).contiguous().to(DEV)
    kpool = kb.view(B * S // ps, ps, H, D).transpose(1, 2)  # (P, Hkv, ps, D) view
    vpool = vb.view(B * S // ps, ps, H, D).transpose(1, 2)
    tbl = torch.arange(B * S // ps, dtype=torch.int32, device=DEV).view(B, S // ps)
    qd, ld = q.to(DEV), lens.to(DEV)
    o1, l1 = A.attn_decode_varlen(qd, kb.transpose(1, 2), vb.transpose(1, 2), ld, S, scale=case.softmax_scale,
                                  return_lse=True)
    o2, l2 = A.attn_decode_paged(qd, kpool, vpool, tbl, ld, S, scale=case.softmax_scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # and three sequences against the oracle
    pick = [0, 5, 11]
    Oref, Lref = oracle.decode_varlen(_np(q[pick]), _np(kc[pick]), _np(vc[pick]), [int(lens[b]) for b in pick],
                                      case.softmax_scale)
    check_o(o2[pick], Oref, case.torch_dtype)
    check_lse(l2[pick], Lref)


def test_paged_page_ids_are_clamped():
    """Page ids outside [0, num_pages) read the first or last page (clamped on
    the device) instead of leaving the pool."""
    case = W.DecodeCase("paged_clamp", 2, 8, 2, 256, 256, 128, "fp16", seed=W.BASE_SEED + 96)
    q, kc, vc = W.decode_inputs(case)
    _say(case.name)
    ps = 32
    kp, vp, tbl = make_paged(kc, vc, [256, 256], ps, seed=5, spare=0)
    P = kp.shape[0]
    bad = tbl.clone()
    bad[0, 1] = -7
    bad[1, 3] = P + 1000
    ld = torch.tensor([256, 256], dtype=torch.int32, device=DEV)
    o, l = A.attn_decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), bad.to(DEV), ld, scale=case.softmax_scale,
                               return_lse=True)
    torch.cuda.synchronize()
    clamped = np.clip(bad.numpy(), 0, P - 1)
    Oref, Lref = oracle.decode_paged(_np(q), _np(kp), _np(vp), clamped, [256, 256], ps, case.softmax_scale)
    check_o(o, Oref, case.torch_dtype)
    check_lse(l, Lref)


def test_kv_cache_write_paged_bitwise():
    B, H, S, D, ps, T = 3, 4, 256, 128, 16, 5
    _say("kv_cache_write_paged")
    g = torch.Generator().manual_seed(W.BASE_SEED + 97)
    kc = torch.randn(B, H, S, D, generator=g).bfloat16()
    vc = torch.randn(B, H, S, D, generator=g).bfloat16()
    kp, vp, tbl = make_paged(kc, vc, [S] * B, ps, seed=6)
    kn = torch.randn(B, H, T, D, generator=g).bfloat16()
    vn = torch.randn(B, H, T, D, generator=g).bfloat16()
    pos = [0, 14, S - T]  # the middle one crosses a page boundary
    kd, vd = kp.to(DEV), vp.to(DEV)
    A.kv_cache_write_paged(kd, vd, kn.to(DEV), vn.to(DEV), tbl.to(DEV), torch.tensor(pos, dtype=torch.int32,
                                                                                       device=DEV))
    torch.cuda.synchronize()
    ke, ve = oracle.kv_cache_write_paged(kp.view(torch.int16).numpy(), vp.view(torch.int16).numpy(),
                                         kn.view(torch.int16).numpy(), vn.view(torch.int16).numpy(), tbl.numpy(),
                                         pos, ps)
    assert np.array_equal(kd.cpu().view(torch.int16).numpy(), ke)
    assert np.array_equal(vd.cpu().view(torch.int16).numpy(), ve)


def test_kv_cache_write_paged_skips_slots_past_the_table():
    """Rows whose slot lies past max_pages_per_seq * page_size are skipped; the
    rows before them are written."""
    B, H, D, ps = 2, 2, 64, 16
    _say("kv_cache_write_paged past the table")
    P, mbps, T = 8, 2, 4
    kp = torch.zeros(P, H, ps, D, dtype=torch.float16, device=DEV)
    vp = torch.zeros_like(kp)
    tbl = torch.tensor([[0, 1], [2, 3]], dtype=torch.int32, device=DEV)
    kn = torch.ones(B, H, T, D, dtype=torch.float16, device=DEV)
    vn = 2 * kn
    pos = torch.tensor([30, 29], dtype=torch.int32, device=DEV)  # capacity 32: 2 and 3 rows fit
    A.kv_cache_write_paged(kp, vp, kn, vn, tbl, pos)
    torch.cuda.synchronize()
    assert torch.all(kp[1, :, 14:16] == 1) and torch.all(kp[3, :, 13:16] == 1)
    assert int((kp != 0).sum()) == (2 + 3) * H * D
    assert torch.all(vp[1, :, 14:16] == 2) and int((vp != 0).sum()) == (2 + 3) * H * D


def test_paged_append_then_decode():
    """Eight decode steps, each appending one token through kv_cache_write_paged
    at the sequence's current length, against the oracle over the pools."""
    B, Hq, H, D, ps, S = 3, 8, 2, 128, 16, 128
    _say("paged append + decode")
    g = torch.Generator().manual_seed(W.BASE_SEED + 98)
    kc = torch.randn(B, H, S, D, generator=g).half()
    vc = torch.randn(B, H, S, D, generator=g).half()
    lens = [15, 40, 1]
    kp, vp, tbl = make_paged(kc, vc, lens, ps, seed=7, spare=2)
    kp, vp = kp.to(DEV), vp.to(DEV)
    kp.nan_to_num_(0.0)  # slots past the lengths are overwritten by the appends below
    vp.nan_to_num_(0.0)
    td = tbl.to(DEV)
    for step in range(8):
        q = torch.randn(B, Hq, D, generator=g).half()
        kn = torch.randn(B, H, 1, D, generator=g).half()
        vn = torch.randn(B, H, 1, D, generator=g).half()
        A.kv_cache_write_paged(kp, vp, kn.to(DEV), vn.to(DEV), td, torch.tensor(lens, dtype=torch.int32,
                                                                                   device=DEV))
        lens = [L + 1 for L in lens]
        o, l = A.attn_decode_paged(q.to(DEV), kp, vp, td, torch.tensor(lens, dtype=torch.int32, device=DEV),
                                   return_lse=True)
        torch.cuda.synchronize()
        Oref, Lref = oracle.decode_paged(_np(q), _np(kp.cpu()), _np(vp.cpu()), tbl.numpy(), lens, ps, D ** -0.5)
        check_o(o, Oref, torch.float16)
        check_lse(l, Lref)
