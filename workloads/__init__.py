"""Seeded synthetic inputs at the pages' workload shapes.

This module holds shapes and random draws only; it contains none of the
attention arithmetic, so both the HIP-path tests/bench and the oracle can use
it without sharing any of the method.

Recipe (also stated in the design doc): a CPU ``torch.Generator`` seeded with
``42 + case_index`` (the base seed 42 is the one the Triton-FlashAttention
README's benchmark section fixes); Q, K, V drawn in that order with
``torch.randn`` in float32, then rounded to the case dtype.  The cross-attention
case draws Q with standard deviation 4.  The pages use no public dataset; these
tensors stand in for activations of the stated shapes.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BASE_SEED = 42

_DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class PrefillCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    D: int
    dtype: str
    causal: bool
    q_std: float = 1.0
    scale: float | None = None  # None -> 1/sqrt(D) rounded to float32
    seed: int = BASE_SEED

    @property
    def torch_dtype(self):
        return _DT[self.dtype]

    @property
    def softmax_scale(self) -> float:
        s = self.scale if self.scale is not None else 1.0 / math.sqrt(self.D)
        return float(torch.tensor(s, dtype=torch.float32).item())

    def visible_pairs_per_head(self) -> int:
        """Number of (i, j) pairs a head must score (the algorithmic work)."""
        if not self.causal:
            return self.Nq * self.Nkv
        # top-left causal: row i sees min(i + 1, Nkv) keys
        n = min(self.Nq, self.Nkv)
        full = n * (n + 1) // 2
        return full + max(0, self.Nq - self.Nkv) * self.Nkv

    def flops(self) -> int:
        """Algorithmic FLOPs: 2 GEMMs x 2 flops per MAC x D per visible pair."""
        return 4 * self.D * self.B * self.Hq * self.visible_pairs_per_head()


@dataclass(frozen=True)
class DecodeCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    S_max: int
    cache_len: int
    D: int
    dtype: str
    scale: float | None = None
    seed: int = BASE_SEED

    @property
    def torch_dtype(self):
        return _DT[self.dtype]

    @property
    def softmax_scale(self) -> float:
        s = self.scale if self.scale is not None else 1.0 / math.sqrt(self.D)
        return float(torch.tensor(s, dtype=torch.float32).item())

    def kv_bytes(self) -> int:
        """Algorithmic bytes: K and V rows read once, plus Q in and O out."""
        es = 2
        return 2 * self.B * self.Hkv * self.cache_len * self.D * es + 2 * self.B * self.Hq * self.D * es


@dataclass(frozen=True)
class VarlenPrefillCase:
    """A packed batch of sequences with their own query and key lengths."""
    name: str
    q_lens: tuple
    k_lens: tuple
    Hq: int
    Hkv: int
    D: int
    dtype: str
    causal: bool
    bottom_right: bool = False
    seed: int = BASE_SEED

    @property
    def torch_dtype(self):
        return _DT[self.dtype]

    @property
    def softmax_scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32).item())

    @property
    def B(self) -> int:
        return len(self.q_lens)

    @staticmethod
    def _cu(lens):
        out = [0]
        for L in lens:
            out.append(out[-1] + int(L))
        return out

    @property
    def cu_q(self):
        return self._cu(self.q_lens)

    @property
    def cu_k(self):
        return self._cu(self.k_lens)

    @property
    def total_q(self) -> int:
        return sum(self.q_lens)

    @property
    def total_k(self) -> int:
        return sum(self.k_lens)

    @property
    def max_q(self) -> int:
        return max(max(self.q_lens), 1)

    def visible_pairs_per_head(self) -> int:
        """(query, key) pairs a head must score, summed over the sequences."""
        tot = 0
        for Lq, Lk in zip(self.q_lens, self.k_lens):
            if not self.causal:
                tot += Lq * Lk
                continue
            off = Lk - Lq if self.bottom_right else 0
            i = torch.arange(Lq, dtype=torch.int64)
            tot += int(torch.clamp(i + off + 1, 0, Lk).sum())
        return tot

    def flops(self) -> int:
        return 4 * self.D * self.Hq * self.visible_pairs_per_head()


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def prefill_inputs(case: PrefillCase):
    """CPU tensors q (B,Hq,Nq,D), k, v (B,Hkv,Nkv,D) in the case dtype."""
    g = _gen(case.seed)
    dt = case.torch_dtype
    q = (torch.randn(case.B, case.Hq, case.Nq, case.D, generator=g) * case.q_std).to(dt)
    k = torch.randn(case.B, case.Hkv, case.Nkv, case.D, generator=g).to(dt)
    v = torch.randn(case.B, case.Hkv, case.Nkv, case.D, generator=g).to(dt)
    return q, k, v


def rising_score_inputs(case: PrefillCase, tile: int = 64, rise: float = 128.0, jitter: float = 8.0):
    """Inputs whose scores step up from one key tile to the next.

    Drawn as ``prefill_inputs``, then query dimension 0 is set to 1 and key
    dimension 0 to ``rise * (j // tile) + jitter * N(0, 1)``, so every row's
    largest score grows by about ``rise * scale * log2(e)`` (log2 units) from
    each tile of ``tile`` keys to the next, at a random key inside the tile.
    """
    q, k, v = prefill_inputs(case)
    g = _gen(case.seed + 1000)
    j = torch.arange(case.Nkv, dtype=torch.float32)
    k0 = rise * torch.floor(j / tile) + jitter * torch.randn(case.B, case.Hkv, case.Nkv, generator=g)
    q = q.clone()
    k = k.clone()
    q[..., 0] = 1.0
    k[..., 0] = k0.to(k.dtype)
    return q, k, v


def decode_inputs(case: DecodeCase):
    """CPU tensors q (B,Hq,D) and full caches (B,Hkv,S_max,D).

    Every slot of the cache is drawn (so slots >= cache_len hold finite data);
    parity tests poison those slots themselves when they want to check that
    they are never read.
    """
    g = _gen(case.seed)
    dt = case.torch_dtype
    q = torch.randn(case.B, case.Hq, case.D, generator=g).to(dt)
    kc = torch.randn(case.B, case.Hkv, case.S_max, case.D, generator=g).to(dt)
    vc = torch.randn(case.B, case.Hkv, case.S_max, case.D, generator=g).to(dt)
    return q, kc, vc


def varlen_prefill_inputs(case: VarlenPrefillCase):
    """CPU tensors q (total_q, Hq, D), k, v (total_k, Hkv, D): packed rows, drawn
    in that order."""
    g = _gen(case.seed)
    dt = case.torch_dtype
    q = torch.randn(case.total_q, case.Hq, case.D, generator=g).to(dt)
    k = torch.randn(case.total_k, case.Hkv, case.D, generator=g).to(dt)
    v = torch.randn(case.total_k, case.Hkv, case.D, generator=g).to(dt)
    return q, k, v


# ---- the pages' workloads -------------------------------------------------

TINY = PrefillCase("tiny_gqa2_n65_d64_causal", 1, 2, 1, 65, 65, 64, "fp16", True, seed=BASE_SEED + 0)


def gqa_sweep():
    """B=2, Hq=16, Hkv in {16,8,4,2,1}, N=1023, D=64, fp16, causal and not."""
    out = []
    i = 1
    for hkv in (16, 8, 4, 2, 1):
        for causal in (True, False):
            out.append(PrefillCase(f"gqa_hkv{hkv}_n1023_d64_{'causal' if causal else 'full'}",
                                   2, 16, hkv, 1023, 1023, 64, "fp16", causal, seed=BASE_SEED + i))
            i += 1
    return out


def serving(n: int, causal: bool):
    """Serving-shape prefill: B=2, Hq=32, Hkv=8, D=128, fp16, Nq=Nkv=n."""
    idx = {2048: 11, 4096: 13, 8192: 15}[n] + (0 if causal else 1)
    return PrefillCase(f"serve_n{n}_d128_{'causal' if causal else 'full'}",
                       2, 32, 8, n, n, 128, "fp16", causal, seed=BASE_SEED + idx)


CROSS = PrefillCase("cross_mqa_bf16_q512_kv16384_d128", 4, 32, 1, 512, 16384, 128, "bf16", False,
                    q_std=4.0, seed=BASE_SEED + 17)

DECODE_LENS = (1, 31, 33, 127, 257, 1024, 4096, 8192)


def decode_case(cache_len: int, dtype: str = "fp16", Hkv: int = 8, seed_offset: int = 0):
    """Decode: B=2, Hq=32, Hkv=8, D=128 over an 8192-slot cache."""
    return DecodeCase(f"decode_L{cache_len}_hkv{Hkv}_{dtype}", 2, 32, Hkv, 8192, cache_len, 128, dtype,
                      seed=BASE_SEED + 20 + seed_offset)


def decode_varlen_case():
    """Per-sequence lengths: a 16-sequence serving batch, Hq=32, Hkv=8, D=128,
    8192-slot caches; lengths drawn by ``decode_varlen_lens``."""
    return DecodeCase("decode_varlen_b16_hkv8_fp16", 16, 32, 8, 8192, 8192, 128, "fp16", seed=BASE_SEED + 30)


def decode_varlen_lens(case: DecodeCase) -> torch.Tensor:
    """Seeded cache lengths, uniform in [1, S_max], int32 (B,)."""
    g = _gen(case.seed + 1000)
    return torch.randint(1, case.S_max + 1, (case.B,), generator=g, dtype=torch.int32)


def chunked_prefill_case(nq: int = 1024, nkv: int = 8192):
    """Causal aligned bottom-right: the last ``nq`` queries of an ``nkv``-token
    sequence against all its keys (chunked prefill), serving heads."""
    return PrefillCase(f"chunk_q{nq}_kv{nkv}_d128_fp16_bottom_right", 2, 32, 8, nq, nkv, 128, "fp16", True,
                       seed=BASE_SEED + 31)


def bottom_right_pairs(Nq: int, Nkv: int) -> int:
    """Visible (query, key) pairs per head of a bottom-right causal mask."""
    off = Nkv - Nq
    return sum(max(0, min(Nkv, i + off + 1)) for i in range(Nq))


def varlen_serving_case():
    """Packed serving batch: 16 sequences with seeded lengths uniform in
    [1, 4096] (queries = keys), Hq=32, Hkv=8, D=128, fp16, causal."""
    g = _gen(BASE_SEED + 40 + 1000)
    lens = tuple(int(x) for x in torch.randint(1, 4097, (16,), generator=g))
    return VarlenPrefillCase("varlen_b16_upto4096_d128_fp16_causal", lens, lens, 32, 8, 128, "fp16", True,
                             seed=BASE_SEED + 40)


AR_TOKENS = 512
