"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  1. attn_fwd: causal prefill, B=2, Hq=32, Hkv=8, N=8192, D=128, fp16;
  2. kv_cache_write of one token into an 8192-slot cache;
  3. attn_decode over cache_len=8192 (B=2, Hq=32, Hkv=8, D=128, fp16).
W untimed warm-up steps, then K timed steps between two device synchronisations.
Each launch is also bracketed by HIP events on the stream it runs on (the
current torch stream, which the binding launches on); prefill throughput is
algorithmic work per launch / average launch duration, the latter measured
right after the timed steps as R back-to-back launches between two events on
that stream, queued behind a sleep kernel so the events measure GPU time only
(the in-step per-launch event figures are reported beside it: an event pair
around each launch adds its own cost).  Decode (a ~17 us call) is timed the
same way; that figure is the reported decode GB/s.  The same
measurement on a single cache copy (resident in the Infinity Cache), a plain
256 MiB device copy's rate and a large fp16 library GEMM's rate are printed as
context (achievable HBM and dense-MFMA references on the same box).

`value` is the prefill throughput in TFLOP/s with algorithmic FLOPs counted as
4 * D per visible (query, key) pair (causal: N(N+1)/2 pairs per head).  Decode
is reported as GB/s of algorithmic bytes (K and V rows read once + q in + o
out); its caches rotate over enough copies (>= 512 MiB) that the 256 MiB
Infinity Cache cannot hold them between uses.

roofline.traffic / decode.traffic are the HBM bytes per launch that rocprofv3's
FETCH_SIZE and WRITE_SIZE counters measured (scaled by a plain copy's reading),
taken from the committed summaries under profiles/; null once the kernel
sources differ from the ones those counters were taken with.

The default run also times six widened workloads (not the headline):
decode with per-sequence cache lengths over a 16-sequence batch, the same
batch over a paged cache (16-slot pages in a shuffled pool), a chunked
prefill (1024 queries at the end of an 8192-token context, causal aligned
bottom-right), a packed prefill of 16 sequences of seeded lengths up to
4096, a causal sliding window of 4096 keys on the 8192-token serving
shape, and the backward (dQ, dK, dV) of the headline prefill; they are
printed under "widened".

"configs" times every workload of the pages at its own shape: the tiny
causal prefill, the ten GQA-sweep cases (B=2, Hq=16, Hkv 16..1, N=1023, D=64,
causal and not), the six serving prefills (B=2, Hq=32, Hkv=8, D=128,
N 2048/4096/8192, causal and not), the bf16 cross-attention MQA prefill (B=4,
Hq=32, Hkv=1, Nq=512, Nkv=16384, D=128) and decode at every cache length
(1 .. 8192), each with its seed, time, throughput and fraction of peak.

Flags: --only prefill|decode|copy|cross|gqa|packed|bwd runs just that launch
(for rocprofv3 runs; cross = the bf16 cross-attention MQA prefill, gqa = the
GQA sweep at Hkv=4, causal and not, packed = the 16-sequence packed prefill,
bwd = the headline backward), --no-cpu skips the oracle baseline,
--no-configs the per-workload block.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
CSRC = os.path.join(ROOT, "attention_attn_fwd_05_amd", "csrc")
PREFILL_SOURCES = ["prefill_fwd.hip", "lds_tile.hpp", "kernel_common.hpp", "launch.hpp", "attn_api.cpp"]
DECODE_SOURCES = ["decode.hip", "kernel_common.hpp", "launch.hpp", "attn_api.cpp"]


def measured_traffic(summary: str, sources: list[str]):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None.

    The summary records the calibrated FETCH_SIZE + WRITE_SIZE bytes and the
    sha256 of the kernel sources it was taken with; a kernel changed since then
    has no measured traffic.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        key, sep, val = line.strip().partition(" = ")
        if sep:
            fields[key] = val
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    if fields.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--only", choices=["all", "prefill", "decode", "copy", "cross", "gqa", "packed", "bwd"],
                   default="all")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-configs", action="store_true", help="skip the per-workload timing block")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--causal", type=int, default=1)
    return p.parse_args()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_baseline(case, budget_s: float):
    """The fp64 oracle, as it stands, on whole (batch, head) slices of the same workload until
    the time budget is used; reported as algorithmic TFLOP/s (same unit as `value`)."""
    import numpy as np

    import oracle
    import workloads as W

    q, k, v = W.prefill_inputs(case)
    g = case.Hq // case.Hkv
    pairs = case.visible_pairs_per_head()
    done = 0
    t0 = time.perf_counter()
    order = [(b, h) for b in range(case.B) for h in range(case.Hq)]
    for (b, h) in order:
        kvh = h // g
        qs = q[b:b + 1, h:h + 1].float().numpy().astype(np.float64)
        ks = k[b:b + 1, kvh:kvh + 1].float().numpy().astype(np.float64)
        vs = v[b:b + 1, kvh:kvh + 1].float().numpy().astype(np.float64)
        oracle.attention_forward(qs, ks, vs, case.softmax_scale, case.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4 * case.D * pairs * done
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} of {case.B * case.Hq} (batch, head) slices of {case.name}, all {case.Nq} query rows "
                      f"each, fp64 numpy (full masked score matrix), {dt:.1f} s",
            "cpu_model": cpu_model(), "host_cpu_count": os.cpu_count()}


def _back_to_back_ms(fn, reps: int, stream, sleep_cycles: int = 2_000_000) -> float:
    """Mean ms per call of `reps` back-to-back calls between two HIP events on
    `stream`, queued behind a sleep kernel so the events time GPU work only."""
    import torch
    torch.cuda.synchronize()
    torch.cuda._sleep(sleep_cycles)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_configs(A, W, dev, stream, kcs, vcs, warmup: int = 10, reps: int = 30):
    """Every workload of the pages at its own shape, with its seed, time,
    algorithmic throughput and fraction of the MI355X peak (2.5 PFLOP/s dense
    fp16/bf16 MFMA for prefill, 8 TB/s HBM for decode), every figure the mean
    of back-to-back launches between two events (at least 50 for launches
    under a millisecond, 30 for the longer ones).  Decode reads rotate
    over the cache copies in `kcs`/`vcs` (>= 512 MiB), so the Infinity Cache
    cannot hold them between calls."""
    import torch
    out = {}

    def prefill(case, back_to_back):
        q, k, v = (t.to(dev) for t in W.prefill_inputs(case))
        o = torch.empty_like(q)
        lse = torch.empty(case.B, case.Hq, case.Nq, dtype=torch.float32, device=dev)
        fn = lambda i: A.attn_fwd(q, k, v, causal=case.causal, scale=case.softmax_scale, out=o, lse=lse,  # noqa
                                  return_lse=True)
        for i in range(warmup):
            fn(i)
        ms = _back_to_back_ms(fn, max(reps, 50) if back_to_back else reps, stream)
        stat = "mean of back-to-back launches"
        fl = case.flops()
        r = {"workload": case.name, "seed": case.seed, "B": case.B, "Hq": case.Hq, "Hkv": case.Hkv, "Nq": case.Nq,
             "Nkv": case.Nkv, "D": case.D, "dtype": case.dtype, "causal": case.causal, "flops_per_launch": fl,
             "us_per_launch": round(ms * 1e3, 2), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
             "frac_of_2500_tflops": round(fl / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4), "timing": stat}
        del q, k, v, o, lse
        return r

    out["tiny"] = prefill(W.TINY, True)
    out["gqa_sweep"] = [prefill(c, True) for c in W.gqa_sweep()]
    out["serving"] = [prefill(W.serving(n, c), n < 8192) for n in (2048, 4096, 8192) for c in (True, False)]
    out["cross_mqa_bf16"] = prefill(W.CROSS, False)

    dec = []
    for L in W.DECODE_LENS:
        dc = W.decode_case(L)
        qd = W.decode_inputs(dc)[0].to(dev)
        od = torch.empty_like(qd)
        ld = torch.empty(dc.B, dc.Hq, dtype=torch.float32, device=dev)
        ws = A.decode_workspace(dc.B, dc.Hq, dc.Hkv, dc.S_max, dc.D, dev)
        rot = len(kcs)
        fn = lambda i: A.attn_decode(qd, kcs[i % rot], vcs[i % rot], L, scale=dc.softmax_scale,  # noqa
                                     workspace=ws, out=od, lse=ld, return_lse=True)
        for i in range(warmup):
            fn(i)
        ms = _back_to_back_ms(fn, max(reps, 40), stream)
        nb = dc.kv_bytes()
        dec.append({"workload": dc.name, "seed": dc.seed, "cache_len": L, "bytes_per_call": nb,
                    "us_per_call": round(ms * 1e3, 2), "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
                    "frac_of_8000_gbs": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "timing": f"mean of back-to-back calls over {rot} rotated cache copies"})
    out["decode"] = dec
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              f"(head-parallel sharding across GPUs is described in DESIGN.md but not run).", file=sys.stderr)
        sys.exit(2)

    import torch

    import attention_attn_fwd_05_amd as A
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    A.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.only in ("cross", "gqa", "packed", "bwd"):
        # one workload alone, for a profiler run: warm-up launches, then `steps` timed ones
        res = []
        if args.only in ("cross", "gqa"):
            cases = [W.CROSS] if args.only == "cross" else [c for c in W.gqa_sweep() if c.Hkv == 4]
            for case in cases:
                q, k, v = (t.to(dev) for t in W.prefill_inputs(case))
                o = torch.empty_like(q)
                fn = lambda i: A.attn_fwd(q, k, v, causal=case.causal, scale=case.softmax_scale, out=o)  # noqa
                for i in range(args.warmup):
                    fn(i)
                ms = _back_to_back_ms(fn, args.steps, stream)
                res.append({"workload": case.name, "us_per_launch": round(ms * 1e3, 2),
                            "tflops": round(case.flops() / (ms * 1e-3) / 1e12, 1)})
        elif args.only == "packed":
            # the packed 16-sequence serving batch (as widened.prefill_varlen)
            vp = W.varlen_serving_case()
            q, k, v = (t.to(dev) for t in W.varlen_prefill_inputs(vp))
            cq = torch.tensor(vp.cu_q, dtype=torch.int32, device=dev)
            o = torch.empty_like(q)
            fn = lambda i: A.attn_fwd_varlen(q, k, v, cq, cq, vp.max_q, causal=True, scale=vp.softmax_scale,  # noqa
                                             out=o)
            for i in range(args.warmup):
                fn(i)
            ms = _back_to_back_ms(fn, args.steps, stream)
            res.append({"workload": vp.name, "us_per_launch": round(ms * 1e3, 2),
                        "tflops": round(vp.flops() / (ms * 1e-3) / 1e12, 1)})
        else:
            # backward of the headline prefill (as widened.backward): the dQ and dK/dV kernels
            bc = W.serving(8192, True)
            q, k, v = (t.to(dev) for t in W.prefill_inputs(bc))
            do = torch.randn(q.shape, generator=torch.Generator().manual_seed(W.BASE_SEED + 60)).to(q.dtype).to(dev)
            o, lse = A.attn_fwd(q, k, v, causal=True, scale=bc.softmax_scale, return_lse=True)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            ws = torch.empty(A.load_library().attn_bwd_workspace_bytes(bc.B, bc.Hq, bc.Nq), dtype=torch.uint8,
                             device=dev)
            fn = lambda i: A.attn_bwd(q, k, v, o, do, lse, causal=True, scale=bc.softmax_scale, dq=dq, dk=dk,  # noqa
                                      dv=dv, workspace=ws)
            for i in range(args.warmup):
                fn(i)
            ms = _back_to_back_ms(fn, args.steps, stream)
            res.append({"workload": bc.name + "_backward", "us_per_launch": round(ms * 1e3, 2),
                        "tflops_5gemm": round(2.5 * bc.flops() / (ms * 1e-3) / 1e12, 1)})
        print(json.dumps({"only": args.only, "results": res}), flush=True)
        return

    pcase = W.serving(8192, bool(args.causal))
    dcase = W.decode_case(8192)

    # ---- resident inputs
    q, k, v = (t.to(dev) for t in W.prefill_inputs(pcase))
    o = torch.empty_like(q)
    lse = torch.empty(pcase.B, pcase.Hq, pcase.Nq, dtype=torch.float32, device=dev)
    qd, kc0, vc0 = W.decode_inputs(dcase)
    cache_bytes = 2 * kc0.numel() * kc0.element_size()
    rot = max(2, math.ceil(512 * 2 ** 20 / cache_bytes) + 1)
    kcs = [kc0.to(dev) for _ in range(rot)]
    vcs = [vc0.to(dev) for _ in range(rot)]
    qd = qd.to(dev)
    od = torch.empty_like(qd)
    lsed = torch.empty(dcase.B, dcase.Hq, dtype=torch.float32, device=dev)
    ws = A.decode_workspace(dcase.B, dcase.Hq, dcase.Hkv, dcase.S_max, dcase.D, dev)
    knew = kc0[:, :, :1].clone().to(dev)
    vnew = vc0[:, :, :1].clone().to(dev)

    copy_src = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev)
    copy_dst = torch.empty_like(copy_src)

    do_p = args.only in ("all", "prefill")
    do_d = args.only in ("all", "decode")
    do_c = args.only == "copy"

    def step(i, ev=None):
        if do_p:
            if ev: ev[0].record(stream)
            A.attn_fwd(q, k, v, causal=pcase.causal, scale=pcase.softmax_scale, out=o, lse=lse, return_lse=True)
            if ev: ev[1].record(stream)
        if do_d:
            j = i % rot
            if ev: ev[2].record(stream)
            A.kv_cache_write(kcs[j], vcs[j], knew, vnew, dcase.cache_len - 1)
            if ev: ev[3].record(stream)
            A.attn_decode(qd, kcs[j], vcs[j], dcase.cache_len, scale=dcase.softmax_scale, workspace=ws,
                          out=od, lse=lsed, return_lse=True)
            if ev: ev[4].record(stream)
        if do_c:
            if ev: ev[0].record(stream)
            copy_dst.copy_(copy_src)
            if ev: ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # steady-state prefill: R back-to-back launches between two events on the
    # launching stream, queued behind a sleep kernel so the events time GPU work
    # only; their mean is the kernel's average launch duration (an event pair
    # around every launch adds its own cost between launches, shown beside it)
    pf_ss = None
    if do_p:
        R = max(40, args.steps)
        pf_ss = _back_to_back_ms(
            lambda i: A.attn_fwd(q, k, v, causal=pcase.causal, scale=pcase.softmax_scale, out=o, lse=lse,
                                 return_lse=True), R, stream, sleep_cycles=5_000_000)

    # steady-state decode: R back-to-back decode calls (rotating caches) between
    # two events, queued behind a sleep kernel so the events time GPU work only
    dec_ss = None
    if do_d:
        R = max(20, args.steps)
        torch.cuda.synchronize()
        torch.cuda._sleep(5_000_000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(R):
            j = i % rot
            A.attn_decode(qd, kcs[j], vcs[j], dcase.cache_len, scale=dcase.softmax_scale, workspace=ws,
                          out=od, lse=lsed, return_lse=True)
        e1.record(stream)
        torch.cuda.synchronize()
        dec_ss = e0.elapsed_time(e1) / R  # ms per call
        # context: the same measurement on one cache copy, which then stays in
        # the 256 MB Infinity Cache ("warm"; not the graded figure)
        torch.cuda._sleep(5_000_000)
        e0.record(stream)
        for i in range(R):
            A.attn_decode(qd, kcs[0], vcs[0], dcase.cache_len, scale=dcase.softmax_scale, workspace=ws,
                          out=od, lse=lsed, return_lse=True)
        e1.record(stream)
        torch.cuda.synchronize()
        dec_warm = e0.elapsed_time(e1) / R

    # widened rows (not the headline): decode with per-sequence lengths over a
    # 16-sequence batch, and a chunked prefill (causal aligned bottom-right)
    widened = None
    if args.only == "all":
        widened = {}
        vc_case = W.decode_varlen_case()
        vq, vk, vv = W.decode_inputs(vc_case)
        vlens_h = W.decode_varlen_lens(vc_case)
        vq, vk, vv, vlens = vq.to(dev), vk.to(dev), vv.to(dev), vlens_h.to(dev)
        vo = torch.empty_like(vq)
        vws = A.decode_workspace(vc_case.B, vc_case.Hq, vc_case.Hkv, vc_case.S_max, vc_case.D, dev)
        vbytes = 2 * vc_case.Hkv * int(vlens_h.sum()) * vc_case.D * 2 + 2 * vc_case.B * vc_case.Hq * vc_case.D * 2
        # two cache copies used in turn: the 247 MB a call reads would otherwise
        # stay in the 256 MB Infinity Cache from one call to the next
        vks, vvs = [vk, vk.clone()], [vv, vv.clone()]
        for i in range(3):
            A.attn_decode_varlen(vq, vks[i % 2], vvs[i % 2], vlens, vc_case.S_max, workspace=vws, out=vo)
        torch.cuda.synchronize()
        torch.cuda._sleep(5_000_000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(20):
            A.attn_decode_varlen(vq, vks[i % 2], vvs[i % 2], vlens, vc_case.S_max, workspace=vws, out=vo)
        e1.record(stream)
        torch.cuda.synchronize()
        vt = e0.elapsed_time(e1) / 20
        widened["decode_varlen"] = {
            "workload": vc_case.name, "B": vc_case.B, "Hq": vc_case.Hq, "Hkv": vc_case.Hkv, "D": vc_case.D,
            "S_max": vc_case.S_max, "lengths": "seeded uniform [1, 8192]", "sum_lengths": int(vlens_h.sum()),
            "timing": "mean of 20 back-to-back calls alternating over 2 cache copies",
            "bytes_per_call": vbytes, "us_per_call": round(vt * 1e3, 2),
            "gbs": round(vbytes / (vt * 1e-3) / 1e9, 1), "frac_of_8000_gbs": round(vbytes / (vt * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # the same batch over a paged cache: 16-slot pages in a shuffled pool
        ps = 16
        npb = vc_case.S_max // ps
        perm = torch.randperm(vc_case.B * npb, generator=torch.Generator().manual_seed(W.BASE_SEED + 50)).to(dev)
        kpool = torch.empty(vc_case.B * npb, vc_case.Hkv, ps, vc_case.D, dtype=vk.dtype, device=dev)
        vpool = torch.empty_like(kpool)
        kpool[perm] = vk.reshape(vc_case.B, vc_case.Hkv, npb, ps, vc_case.D).permute(0, 2, 1, 3, 4).reshape(
            -1, vc_case.Hkv, ps, vc_case.D)
        vpool[perm] = vv.reshape(vc_case.B, vc_case.Hkv, npb, ps, vc_case.D).permute(0, 2, 1, 3, 4).reshape(
            -1, vc_case.Hkv, ps, vc_case.D)
        vtbl = perm.reshape(vc_case.B, npb).to(torch.int32)
        del vks, vvs
        kpools, vpools = [kpool, kpool.clone()], [vpool, vpool.clone()]
        for i in range(3):
            A.attn_decode_paged(vq, kpools[i % 2], vpools[i % 2], vtbl, vlens, vc_case.S_max, workspace=vws, out=vo)
        torch.cuda.synchronize()
        torch.cuda._sleep(5_000_000)
        e0.record(stream)
        for i in range(20):
            A.attn_decode_paged(vq, kpools[i % 2], vpools[i % 2], vtbl, vlens, vc_case.S_max, workspace=vws, out=vo)
        e1.record(stream)
        torch.cuda.synchronize()
        pgt = e0.elapsed_time(e1) / 20
        widened["decode_paged"] = {
            "workload": vc_case.name + "_paged16_shuffled", "page_size": ps, "pages": vc_case.B * npb,
            "lengths": "as decode_varlen", "timing": "mean of 20 back-to-back calls alternating over 2 page pools",
            "bytes_per_call": vbytes, "us_per_call": round(pgt * 1e3, 2),
            "gbs": round(vbytes / (pgt * 1e-3) / 1e9, 1),
            "frac_of_8000_gbs": round(vbytes / (pgt * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del vq, vk, vv, vo, vws, kpool, vpool, kpools, vpools
        cp = W.chunked_prefill_case()
        cq, ck, cv = (t.to(dev) for t in W.prefill_inputs(cp))
        co = torch.empty_like(cq)
        cflops = 4 * cp.D * cp.B * cp.Hq * W.bottom_right_pairs(cp.Nq, cp.Nkv)
        for _ in range(3):
            A.attn_fwd(cq, ck, cv, causal=True, causal_align="bottom_right", scale=cp.softmax_scale, out=co)
        torch.cuda.synchronize()
        torch.cuda._sleep(5_000_000)
        e0.record(stream)
        for _ in range(10):
            A.attn_fwd(cq, ck, cv, causal=True, causal_align="bottom_right", scale=cp.softmax_scale, out=co)
        e1.record(stream)
        torch.cuda.synchronize()
        ct_ = e0.elapsed_time(e1) / 10
        widened["chunked_prefill"] = {
            "workload": cp.name, "B": cp.B, "Hq": cp.Hq, "Hkv": cp.Hkv, "Nq": cp.Nq, "Nkv": cp.Nkv, "D": cp.D,
            "causal": "bottom_right", "flops_per_launch": cflops, "ms_per_launch": round(ct_, 4),
            "tflops": round(cflops / (ct_ * 1e-3) / 1e12, 1),
            "frac_of_2500_tflops": round(cflops / (ct_ * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)}
        del cq, ck, cv, co
        vp = W.varlen_serving_case()
        pq, pk, pv = (t.to(dev) for t in W.varlen_prefill_inputs(vp))
        pcq = torch.tensor(vp.cu_q, dtype=torch.int32, device=dev)
        pck = torch.tensor(vp.cu_k, dtype=torch.int32, device=dev)
        po = torch.empty_like(pq)
        for _ in range(3):
            A.attn_fwd_varlen(pq, pk, pv, pcq, pck, vp.max_q, causal=True, scale=vp.softmax_scale, out=po)
        torch.cuda.synchronize()
        torch.cuda._sleep(5_000_000)
        e0.record(stream)
        for _ in range(10):
            A.attn_fwd_varlen(pq, pk, pv, pcq, pck, vp.max_q, causal=True, scale=vp.softmax_scale, out=po)
        e1.record(stream)
        torch.cuda.synchronize()
        pt = e0.elapsed_time(e1) / 10
        widened["prefill_varlen"] = {
            "workload": vp.name, "sequences": vp.B, "Hq": vp.Hq, "Hkv": vp.Hkv, "D": vp.D, "causal": "top_left",
            "lengths": "seeded uniform [1, 4096]", "total_tokens": vp.total_q, "flops_per_launch": vp.flops(),
            "ms_per_launch": round(pt, 4), "tflops": round(vp.flops() / (pt * 1e-3) / 1e12, 1),
            "frac_of_2500_tflops": round(vp.flops() / (pt * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)}
        del pq, pk, pv, po
        # causal sliding window of 4096 keys on the serving shape (N = 8192)
        wc = W.serving(8192, True)
        wq, wk, wv = (t.to(dev) for t in W.prefill_inputs(wc))
        wo = torch.empty_like(wq)
        wwin = 4095
        wpairs = sum(min(i, wwin) + 1 for i in range(wc.Nq))
        wflops = 4 * wc.D * wc.B * wc.Hq * wpairs
        for _ in range(3):
            A.attn_fwd(wq, wk, wv, causal=True, window=(wwin, -1), scale=wc.softmax_scale, out=wo)
        torch.cuda.synchronize()
        torch.cuda._sleep(5_000_000)
        e0.record(stream)
        for _ in range(10):
            A.attn_fwd(wq, wk, wv, causal=True, window=(wwin, -1), scale=wc.softmax_scale, out=wo)
        e1.record(stream)
        torch.cuda.synchronize()
        wt = e0.elapsed_time(e1) / 10
        widened["prefill_window"] = {
            "workload": "serve_n8192_d128_causal_window4096", "B": wc.B, "Hq": wc.Hq, "Hkv": wc.Hkv, "N": wc.Nq,
            "D": wc.D, "window_left": wwin, "flops_per_launch": wflops, "ms_per_launch": round(wt, 4),
            "tflops": round(wflops / (wt * 1e-3) / 1e12, 1),
            "frac_of_2500_tflops": round(wflops / (wt * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)}
        del wq, wk, wv, wo
        # backward of the headline prefill (dQ, dK, dV from the forward's O, lse)
        bc = W.serving(8192, True)
        bq, bk, bv = (t.to(dev) for t in W.prefill_inputs(bc))
        bdo = torch.randn(bq.shape, generator=torch.Generator().manual_seed(W.BASE_SEED + 60)).to(bq.dtype).to(dev)
        bo, blse = A.attn_fwd(bq, bk, bv, causal=True, scale=bc.softmax_scale, return_lse=True)
        bdq, bdk, bdv = torch.empty_like(bq), torch.empty_like(bk), torch.empty_like(bv)
        bws = torch.empty(A.load_library().attn_bwd_workspace_bytes(bc.B, bc.Hq, bc.Nq), dtype=torch.uint8,
                          device=dev)
        run_bwd = lambda: A.attn_bwd(bq, bk, bv, bo, bdo, blse, causal=True, scale=bc.softmax_scale, dq=bdq,
                                     dk=bdk, dv=bdv, workspace=bws)
        # 5 warm-up and 20 back-to-back calls (~80 ms), as in its kernel trace
        for _ in range(5):
            run_bwd()
        bt = _back_to_back_ms(lambda i: run_bwd(), 20, stream, sleep_cycles=5_000_000)
        bflops = int(2.5 * bc.flops())  # 5 GEMMs against the forward's 2
        widened["backward"] = {
            "workload": bc.name + "_backward", "B": bc.B, "Hq": bc.Hq, "Hkv": bc.Hkv, "N": bc.Nq, "D": bc.D,
            "flops_per_launch": bflops, "flop_count": "5 GEMMs (2.5x the forward's causal count); the kernels issue 7",
            "ms_per_launch": round(bt, 4), "tflops": round(bflops / (bt * 1e-3) / 1e12, 1),
            "frac_of_2500_tflops": round(bflops / (bt * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)}
        del bq, bk, bv, bdo, bo, blse, bdq, bdk, bdv, bws
        # backward of the packed 16-sequence batch (as prefill_varlen)
        vb = W.varlen_serving_case()
        vq, vk, vv = (t.to(dev) for t in W.varlen_prefill_inputs(vb))
        vdo = torch.randn(vq.shape, generator=torch.Generator().manual_seed(W.BASE_SEED + 61)).to(vq.dtype).to(dev)
        vcq = torch.tensor(vb.cu_q, dtype=torch.int32, device=dev)
        vo, vl = A.attn_fwd_varlen(vq, vk, vv, vcq, vcq, vb.max_q, causal=True, scale=vb.softmax_scale,
                                   return_lse=True)
        vdq, vdk, vdv = torch.empty_like(vq), torch.empty_like(vk), torch.empty_like(vv)
        run_vbwd = lambda: A.attn_bwd_varlen(vq, vk, vv, vo, vdo, vl, vcq, vcq, vb.max_q, vb.max_q, causal=True,
                                             scale=vb.softmax_scale, dq=vdq, dk=vdk, dv=vdv)
        for _ in range(5):
            run_vbwd()
        vbt = _back_to_back_ms(lambda i: run_vbwd(), 20, stream, sleep_cycles=5_000_000)
        vbflops = int(2.5 * vb.flops())
        widened["backward_varlen"] = {
            "workload": vb.name + "_backward", "sequences": vb.B, "Hq": vb.Hq, "Hkv": vb.Hkv, "D": vb.D,
            "flops_per_launch": vbflops, "flop_count": "5 GEMMs (2.5x the forward's causal count)",
            "ms_per_launch": round(vbt, 4), "tflops": round(vbflops / (vbt * 1e-3) / 1e12, 1),
            "frac_of_2500_tflops": round(vbflops / (vbt * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)}
        del vq, vk, vv, vdo, vo, vl, vdq, vdk, vdv
        # the pages' GQA sweep shape (B=2, Hq=16, N=1023, D=64): a grid small
        # enough for 128-row blocks
        gs = {}
        for gc in (c for c in W.gqa_sweep() if c.Hkv == 4):
            gq, gk, gv = (t.to(dev) for t in W.prefill_inputs(gc))
            go = torch.empty_like(gq)
            for _ in range(5):
                A.attn_fwd(gq, gk, gv, causal=gc.causal, scale=gc.softmax_scale, out=go)
            torch.cuda.synchronize()
            torch.cuda._sleep(2_000_000)
            e0.record(stream)
            for _ in range(50):
                A.attn_fwd(gq, gk, gv, causal=gc.causal, scale=gc.softmax_scale, out=go)
            e1.record(stream)
            torch.cuda.synchronize()
            gt = e0.elapsed_time(e1) / 50
            gs["causal" if gc.causal else "full"] = {
                "workload": gc.name, "us_per_launch": round(gt * 1e3, 2), "flops_per_launch": gc.flops(),
                "tflops": round(gc.flops() / (gt * 1e-3) / 1e12, 1)}
            del gq, gk, gv, go
        widened["prefill_gqa_sweep"] = gs

    configs = None
    if args.only == "all" and not args.no_configs:
        configs = time_configs(A, W, dev, stream, kcs, vcs)

    # context: achievable HBM rate of a plain 256 MiB device copy (read + write)
    copy_gbs = None
    if args.only == "all":
        for _ in range(3):
            copy_dst.copy_(copy_src)
        torch.cuda.synchronize()
        torch.cuda._sleep(5_000_000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            copy_dst.copy_(copy_src)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_gbs = 2 * copy_src.numel() / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9

    # context: achievable dense fp16 MFMA rate of a large library GEMM (torch.mm,
    # 8192^3, contiguous operands) on the same box
    gemm_tflops = None
    if args.only == "all":
        n = 8192
        ga = torch.randn(n, n, device=dev, dtype=torch.float16)
        gb = torch.randn(n, n, device=dev, dtype=torch.float16)
        gcm = torch.empty(n, n, device=dev, dtype=torch.float16)
        for _ in range(3):
            torch.mm(ga, gb, out=gcm)
        torch.cuda.synchronize()
        torch.cuda._sleep(5_000_000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            torch.mm(ga, gb, out=gcm)
        e1.record(stream)
        torch.cuda.synchronize()
        gemm_tflops = 2 * n ** 3 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12
        del ga, gb, gcm

    res = {}
    if do_p:
        pt = [evs[i][0].elapsed_time(evs[i][1]) for i in range(args.steps)]  # ms
        p_mean = statistics.fmean(pt)
        p_med = statistics.median(pt)
        flops = pcase.flops()
        res["prefill"] = {"steady_ms_per_launch": pf_ss, "steady_launches": max(40, args.steps),
                          "tflops": flops / (pf_ss * 1e-3) / 1e12,
                          "in_step_ms_mean": p_mean, "in_step_ms_median": p_med, "in_step_ms_std": statistics.pstdev(pt),
                          "in_step_tflops_from_median": flops / (p_med * 1e-3) / 1e12,
                          "flops_per_launch": flops,
                          "flops_per_launch_no_causal_factor": 4 * pcase.B * pcase.Hq * pcase.Nq * pcase.Nkv * pcase.D}
    if do_d:
        dt_ = [evs[i][3].elapsed_time(evs[i][4]) for i in range(args.steps)]
        wt = [evs[i][2].elapsed_time(evs[i][3]) for i in range(args.steps)]
        d_mean = statistics.fmean(dt_)
        nbytes = dcase.kv_bytes()
        res["decode"] = {"in_step_ms_mean": d_mean, "in_step_ms_median": statistics.median(dt_),
                         "in_step_ms_std": statistics.pstdev(dt_),
                         "steady_ms_per_call": dec_ss, "steady_calls": max(20, args.steps),
                         "gbs": nbytes / (dec_ss * 1e-3) / 1e9, "in_step_gbs": nbytes / (d_mean * 1e-3) / 1e9,
                         "bytes_per_launch": nbytes, "cache_copies_rotated": rot,
                         "warm_ms_per_call": dec_warm, "warm_gbs": nbytes / (dec_warm * 1e-3) / 1e9,
                         "kv_cache_write_ms_mean": statistics.fmean(wt)}
    if do_c:
        ct = [evs[i][0].elapsed_time(evs[i][1]) for i in range(args.steps)]
        nb = copy_src.numel()
        res["copy"] = {"bytes_read": nb, "bytes_written": nb, "ms_mean": statistics.fmean(ct),
                       "gbs": 2 * nb / (statistics.fmean(ct) * 1e-3) / 1e9}

    out = {
        "metric": "causal prefill fwd TFLOPS (fp16) + decode KV-read GB/s, % of MI355X peak",
        "value": round(res["prefill"]["tflops"], 2) if do_p else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) Q/K/V at the pages' shapes)",
        "seeds": {"prefill": pcase.seed, "decode": dcase.seed},
        "config": {"workload": f"{pcase.name} prefill + kv_cache_write(T=1) + {dcase.name} decode",
                   "prefill": {"B": pcase.B, "Hq": pcase.Hq, "Hkv": pcase.Hkv, "Nq": pcase.Nq, "Nkv": pcase.Nkv,
                               "D": pcase.D, "causal": pcase.causal},
                   "decode": {"B": dcase.B, "Hq": dcase.Hq, "Hkv": dcase.Hkv, "S_max": dcase.S_max,
                              "cache_len": dcase.cache_len, "D": dcase.D}},
    }
    if do_p:
        t = res["prefill"]["tflops"]
        out["roofline"] = {"bound": "mfma", "achieved": round(t, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(t / MFMA_PEAK_TFLOPS, 4),
                           "traffic": measured_traffic("prefill_fwd_n8192_d128_causal_fp16.md", PREFILL_SOURCES),
                           "kernel": "prefill_fwd_kernel<128, f16, causal>"}
    if do_d:
        g = res["decode"]["gbs"]
        out["decode"] = {"achieved": round(g, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "bound": "hbm",
                         "frac": round(g / HBM_PEAK_GBS, 4), "us_per_call": round(dec_ss * 1e3, 2),
                         "timing": "back-to-back calls over rotating caches (split kernel + combine kernel)",
                         "kernel": "decode_kernel<128, f16, uniform lengths> + decode_combine_kernel<128, f16, uniform lengths>",
                         "traffic": measured_traffic("decode_L8192_hkv8_d128_fp16.md", DECODE_SOURCES)}
    if configs:
        out["configs"] = configs
    if widened:
        out["widened"] = widened
    if copy_gbs is not None:
        out["context"] = {"hbm_copy_gbs": round(copy_gbs, 1),
                          "note": "plain 256 MiB device copy (read+write bytes) on this box: an achievable HBM rate; "
                                  "decode.achieved / hbm_copy_gbs is the fraction of it"}
        if do_d:
            out["context"]["decode_frac_of_copy"] = round(res["decode"]["gbs"] / copy_gbs, 4)
        if gemm_tflops is not None:
            out["context"]["fp16_gemm_tflops"] = round(gemm_tflops, 1)
            if do_p:
                out["context"]["prefill_frac_of_gemm"] = round(res["prefill"]["tflops"] / gemm_tflops, 4)
            out["context"]["gemm_note"] = ("torch.mm of two 8192 x 8192 fp16 matrices (a library GEMM) on this box: an "
                                           "achievable dense-MFMA rate; roofline.achieved / fp16_gemm_tflops is the "
                                           "fraction of it")
    out["detail"] = res
    if do_p and args.only == "all" and not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(pcase, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
