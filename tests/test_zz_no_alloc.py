"""attn_decode_noalloc -- the decode that allocates nothing, its split partials
in the library's fixed per-GPU scratch -- called through the C ABI and checked
against attn_decode (caller's workspace) on the same inputs: bit for bit (the
same kernels and split), and against the fp64 oracle to the decode tolerance.

Three calls in a row share one scratch; the second has a smaller input and
the third a different dtype, head dim and forced split count, so a partial
left over from an earlier call would show up.  Every output starts as NaN.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_attn_fwd_05_amd as A
import oracle
import workloads as W
from attention_attn_fwd_05_amd import _binding as bd
from gpu_util import check_lse, check_o

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _noalloc_c(q, kc, vc, o, lse, cache_len, scale, num_splits):
    """One call straight through the C ABI (ctypes), no workspace argument."""
    lib = bd.load_library()
    B, Hq, D = q.shape
    Hkv, S = kc.shape[1], kc.shape[2]
    code = 0 if q.dtype == torch.float16 else 1
    return lib.attn_decode_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq,
                                   Hkv, S, cache_len, D, bd._strides3(q), bd._strides4(kc), bd._strides4(vc),
                                   bd._strides3(o), scale, code, num_splits,
                                   torch.cuda.current_stream().cuda_stream)


CALLS = [
    # B, Hq, Hkv, S_max, cache_len, D, dtype, num_splits
    (2, 32, 8, 8192, 8192, 128, "fp16", 0),   # the serving decode shape, default splits
    (1, 8, 2, 2048, 1000, 128, "fp16", 0),    # smaller: fewer units and chunks
    (3, 16, 1, 640, 333, 64, "bf16", 3),      # MQA, forced split count
]


def test_noalloc_decode_matches_attn_decode():
    for i, (B, Hq, Hkv, S, L, D, dt, ns) in enumerate(CALLS):
        case = W.DecodeCase(f"noalloc_{i}", B, Hq, Hkv, S, L, D, dt, seed=W.BASE_SEED + 400 + i)
        print(f"[case] attn_decode_noalloc call {i}: B={B} Hq={Hq} Hkv={Hkv} S_max={S} cache_len={L} D={D} {dt} "
              f"num_splits={ns}", flush=True)
        q, kc, vc = W.decode_inputs(case)
        qd, kd, vd = q.to(DEV), kc.to(DEV), vc.to(DEV)
        o_ref, l_ref = A.attn_decode(qd, kd, vd, L, scale=case.softmax_scale, num_splits=ns, return_lse=True)
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
        st = _noalloc_c(qd, kd, vd, o, lse, L, case.softmax_scale, ns)
        torch.cuda.synchronize()
        assert st == 0, bd.load_library().attn_status_string(st)
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"call {i}: differs from attn_decode"
        O, Lse = oracle.decode(_np(q), _np(kc), _np(vc), L, case.softmax_scale)
        check_o(o.cpu(), O, case.torch_dtype)
        check_lse(lse.cpu(), Lse)


def test_noalloc_refuses_partials_beyond_scratch():
    """A forced split count whose partials exceed the scratch is refused before
    anything is launched, and the outputs stay untouched."""
    B, Hq, Hkv, S, D = 64, 64, 64, 8192, 128   # 4096 units x 64 chunks x 132 floats: 138 MB
    q = torch.zeros(B, Hq, D, dtype=torch.float16, device=DEV)
    kc = torch.zeros(B, Hkv, 1, D, dtype=torch.float16, device=DEV).expand(B, Hkv, S, D)  # never read
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq), 7.0, dtype=torch.float32, device=DEV)
    print("[case] attn_decode_noalloc refusal (partials beyond the scratch)", flush=True)
    st = _noalloc_c(q, kc, kc, o, lse, S, 0.088, 64)
    torch.cuda.synchronize()
    assert st == int(bd.Status.ERR_WORKSPACE)
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
