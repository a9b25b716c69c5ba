"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle (looked up at call
time through ``oracle.attention``, so a test can plant a mistake in it) breaks a
fact fixed by the mathematics or by the pages' conventions:

* hand-derived closed forms (tests/golden/closed_forms.json);
* closed forms for structured inputs (equal scores -> mean of V, one key -> V[0],
  causal row 0 -> V[0]);
* invariants (rows of P sum to 1, shift and permutation invariance, linearity in
  V, GQA == repeat_interleave-expanded MHA, causal prefill row i == decode over
  i + 1 cached keys);
* an mpmath brute force written independently (explicit loops, no max
  subtraction, exact-rounded dot products, 40 significant digits).

The module has no test_ prefix: tests/test_oracle_pins.py runs every pin against
the real oracle and tests/test_oracle_mutations.py runs them against oracles
with planted bugs to show each bug is caught.
"""

from __future__ import annotations

import json
import math
import os

import mpmath
import numpy as np

import oracle.attention as OA

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


# ---------------------------------------------------------------- helpers

def _decode_value(x):
    if isinstance(x, dict):
        (key, arg), = x.items()
        if key == "ln":
            return math.log(arg)
        if key == "one_minus_ln_over_1000":
            return 1.0 - math.log(arg) / 1000.0
        if key == "plus_1000_ln":
            return 1000.0 + math.log(arg)
        raise KeyError(key)
    if isinstance(x, list):
        return [_decode_value(e) for e in x]
    return float(x)


def _arr(x):
    return np.array(_decode_value(x), dtype=np.float64)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _fp16_exact(rng, *shape, std=1.0):
    """Random values that are exactly representable in fp16 (as the kernels see them)."""
    return (rng.standard_normal(shape) * std).astype(np.float16).astype(np.float64)


# ---------------------------------------------------------------- pins

def pin_golden_prefill():
    for case in _golden()["prefill"]:
        q, k, v = _arr(case["q"]), _arr(case["k"]), _arr(case["v"])
        O, lse = OA.attention_forward(q, k, v, case["scale"], case["causal"])
        np.testing.assert_allclose(O, _arr(case["o"]), rtol=0, atol=case["tol"], err_msg=case["name"])
        np.testing.assert_allclose(lse, _arr(case["lse"]), rtol=0, atol=case["tol"], err_msg=case["name"])


def pin_golden_decode():
    for case in _golden()["decode"]:
        O, lse = OA.decode(_arr(case["q"]), _arr(case["k_cache"]), _arr(case["v_cache"]),
                           case["cache_len"], case["scale"])
        np.testing.assert_allclose(O, _arr(case["o"]), rtol=0, atol=case["tol"], err_msg=case["name"])
        np.testing.assert_allclose(lse, _arr(case["lse"]), rtol=0, atol=case["tol"], err_msg=case["name"])


def pin_golden_cache_write():
    for case in _golden()["cache_write"]:
        kc, vc = OA.kv_cache_write(_arr(case["k_cache"]), _arr(case["v_cache"]),
                                   _arr(case["k_new"]), _arr(case["v_new"]), case["pos"])
        np.testing.assert_array_equal(kc, _arr(case["k_out"]), err_msg=case["name"])
        np.testing.assert_array_equal(vc, _arr(case["v_out"]), err_msg=case["name"])


def pin_rows_sum_to_one():
    """P1: every row of P sums to 1 over visible keys and is 0 on masked keys."""
    rng = np.random.default_rng(1)
    for causal in (False, True):
        q, k = _rand(rng, 2, 4, 13, 8), _rand(rng, 2, 2, 13, 8)
        P = OA.attention_probs(q, k, 0.37, causal)
        np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
        assert (P >= 0).all()
        if causal:
            i, j = np.indices((13, 13))
            assert (P[..., j > i] == 0).all()
            assert (P[..., j <= i] > 0).all()


def pin_probs_head_mapping():
    """attention_probs maps q head h to kv head h // (Hq / Hkv): with every key
    of kv head 1 equal, the q heads of its group see equal scores, so their
    rows are uniform over the visible keys (1 / n_visible), while the group of
    kv head 0 (distinct keys) is not; and P V reproduces attention_forward's O."""
    rng = np.random.default_rng(11)
    B, Hq, Hkv, N, D = 2, 6, 3, 11, 8
    q, k, v = _rand(rng, B, Hq, N, D), _rand(rng, B, Hkv, N, D), _rand(rng, B, Hkv, N, D)
    k[:, 1] = k[:, 1, :1]  # kv head 1: one key repeated
    for causal in (False, True):
        P = OA.attention_probs(q, k, 0.41, causal)
        n_vis = (np.arange(N)[:, None] + 1) if causal else np.full((N, 1), N)
        vis = (np.arange(N)[None, :] <= np.arange(N)[:, None]) if causal else np.ones((N, N), bool)
        uniform = np.where(vis, 1.0 / n_vis, 0.0)
        for h in range(Hq):
            if h // 2 == 1:
                np.testing.assert_allclose(P[:, h], np.broadcast_to(uniform, (B, N, N)), rtol=0, atol=1e-14)
            else:
                assert np.abs(P[:, h, -1] - uniform[-1]).max() > 1e-3, h
        O, _ = OA.attention_forward(q, k, v, 0.41, causal)
        kvh = np.arange(Hq) // (Hq // Hkv)
        np.testing.assert_allclose(np.einsum("bhij,bhjd->bhid", P, v[:, kvh]), O, rtol=0, atol=1e-12)


def pin_causal_row0_is_v0():
    """P2: with top-left causal masking row 0 sees key 0 only: O = V[0] exactly."""
    rng = np.random.default_rng(2)
    q, k, v = _fp16_exact(rng, 2, 4, 9, 16), _fp16_exact(rng, 2, 2, 9, 16), _fp16_exact(rng, 2, 2, 9, 16)
    scale = 0.25
    O, lse = OA.attention_forward(q, k, v, scale, True)
    for h in range(4):
        kvh = h // 2
        np.testing.assert_array_equal(O[:, h, 0], v[:, kvh, 0])
        s00 = scale * np.einsum("bd,bd->b", q[:, h, 0], k[:, kvh, 0])
        np.testing.assert_allclose(lse[:, h, 0], s00, rtol=0, atol=1e-12)


def pin_equal_scores_give_mean():
    """P3: all scores equal (Q = 0, or scale = 0) -> O is the mean of visible V, lse = ln(count)."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, N, D = 1, 4, 2, 11, 8
    k, v = _rand(rng, B, Hkv, N, D), _rand(rng, B, Hkv, N, D)
    for (q, scale) in ((np.zeros((B, Hq, N, D)), 0.5), (_rand(rng, B, Hq, N, D), 0.0)):
        for causal in (False, True):
            O, lse = OA.attention_forward(q, k, v, scale, causal)
            for h in range(Hq):
                kvh = h // (Hq // Hkv)
                for i in range(N):
                    n = i + 1 if causal else N
                    np.testing.assert_allclose(O[0, h, i], v[0, kvh, :n].mean(0), rtol=0, atol=1e-13)
                    np.testing.assert_allclose(lse[0, h, i], math.log(n), rtol=0, atol=1e-13)


def pin_single_key():
    """P4: N_kv = 1 -> every row returns V[0] and lse = its one score."""
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 2, 4, 5, 8), _rand(rng, 2, 1, 1, 8), _rand(rng, 2, 1, 1, 8)
    O, lse = OA.attention_forward(q, k, v, 0.3, False)
    np.testing.assert_array_equal(O, np.broadcast_to(v[:, :, :1], O.shape))
    np.testing.assert_allclose(lse, 0.3 * np.einsum("bhnd,bd->bhn", q, k[:, 0, 0]), rtol=0, atol=1e-12)
    Od, lsed = OA.decode(q[:, :, 0], k, v, 1, 0.3)
    np.testing.assert_array_equal(Od, np.broadcast_to(v[:, 0, 0][:, None], Od.shape))


def pin_gqa_equals_expanded_mha():
    """P5: GQA/MQA equals MHA on K/V expanded with repeat_interleave over heads."""
    rng = np.random.default_rng(5)
    for Hkv in (1, 2, 4):
        q, k, v = _rand(rng, 2, 8, 7, 8), _rand(rng, 2, Hkv, 9, 8), _rand(rng, 2, Hkv, 9, 8)
        g = 8 // Hkv
        ke, ve = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
        for causal in (False, True):
            O, lse = OA.attention_forward(q, k, v, 0.4, causal)
            Oe, lsee = OA.attention_forward(q, ke, ve, 0.4, causal)
            np.testing.assert_array_equal(O, Oe)
            np.testing.assert_array_equal(lse, lsee)


def _brute(q, k, v, scale, causal, offset=0):
    """Independent evaluation: explicit loops, exp without max subtraction at 40 digits.

    A row with no visible key gets O = 0 and lse = -inf (the convention)."""
    mpmath.mp.dps = 40
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    O = np.zeros((B, Hq, Nq, D))
    lse = np.zeros((B, Hq, Nq))
    sc = mpmath.mpf(float(scale))
    for b in range(B):
        for h in range(Hq):
            kvh = (h * Hkv) // Hq
            for i in range(Nq):
                keys = [j for j in range(Nkv) if (not causal) or j <= i + offset]
                if not keys:
                    lse[b, h, i] = -np.inf
                    continue
                w = []
                for j in keys:
                    dot = mpmath.mpf(math.fsum(float(q[b, h, i, d]) * float(k[b, kvh, j, d]) for d in range(D)))
                    w.append(mpmath.exp(sc * dot))
                tot = mpmath.fsum(w)
                for d in range(D):
                    O[b, h, i, d] = float(mpmath.fsum(wj * mpmath.mpf(float(v[b, kvh, j, d])) for wj, j in zip(w, keys)) / tot)
                lse[b, h, i] = float(mpmath.log(tot))
    return O, lse


def pin_brute_force_tiny():
    """P6: agreement with the brute force on tiny shapes (odd N, g in {1,2,4})."""
    rng = np.random.default_rng(6)
    shapes = [(1, 1, 1, 1, 1, 1), (1, 2, 2, 5, 5, 3), (2, 4, 2, 7, 7, 4), (1, 4, 1, 9, 9, 8), (1, 4, 4, 3, 6, 2)]
    for (B, Hq, Hkv, Nq, Nkv, D) in shapes:
        q, k, v = _rand(rng, B, Hq, Nq, D), _rand(rng, B, Hkv, Nkv, D), _rand(rng, B, Hkv, Nkv, D)
        for causal in (False, True):
            if causal and Nq > Nkv:
                continue
            O, lse = OA.attention_forward(q, k, v, 0.7, causal)
            Ob, lseb = _brute(q, k, v, 0.7, causal)
            np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, lseb, rtol=1e-12, atol=1e-12)


def pin_brute_force_bottom_right():
    """P6b: bottom-right causal (offset Nkv - Nq) against the brute force, for
    Nq < Nkv, Nq == Nkv and Nq > Nkv (whose first Nq - Nkv rows see no key)."""
    rng = np.random.default_rng(61)
    shapes = [(1, 2, 1, 3, 8, 4), (1, 4, 2, 5, 5, 3), (2, 2, 2, 7, 4, 3), (1, 1, 1, 1, 6, 2)]
    for (B, Hq, Hkv, Nq, Nkv, D) in shapes:
        q, k, v = _rand(rng, B, Hq, Nq, D), _rand(rng, B, Hkv, Nkv, D), _rand(rng, B, Hkv, Nkv, D)
        off = Nkv - Nq
        O, lse = OA.attention_forward(q, k, v, 0.6, True, causal_offset=off)
        Ob, lseb = _brute(q, k, v, 0.6, True, offset=off)
        np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lseb, rtol=1e-12, atol=1e-12)
        if Nq > Nkv:
            assert np.all(O[:, :, :Nq - Nkv] == 0.0) and np.all(lse[:, :, :Nq - Nkv] == -np.inf)


def pin_bottom_right_is_the_tail_of_full_causal():
    """P6c: chunked prefill -- the last Nq rows of a top-left causal attention over
    N tokens equal a bottom-right causal attention of those Nq queries against all N keys."""
    rng = np.random.default_rng(62)
    B, Hq, Hkv, N, D = 2, 4, 2, 17, 6
    q, k, v = _rand(rng, B, Hq, N, D), _rand(rng, B, Hkv, N, D), _rand(rng, B, Hkv, N, D)
    O, lse = OA.attention_forward(q, k, v, 0.5, True)
    for Nq in (1, 5, 16):
        Ot, lset = OA.attention_forward(q[:, :, N - Nq:], k, v, 0.5, True, causal_offset=N - Nq)
        np.testing.assert_allclose(Ot, O[:, :, N - Nq:], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lset, lse[:, :, N - Nq:], rtol=0, atol=1e-13)


def pin_shift_invariance():
    """P7: adding one vector u to every key leaves O unchanged and shifts lse by scale*q.u."""
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 1, 2, 6, 8), _rand(rng, 1, 1, 6, 8), _rand(rng, 1, 1, 6, 8)
    u = _rand(rng, 8) * 3.0
    for causal in (False, True):
        O, lse = OA.attention_forward(q, k, v, 0.5, causal)
        O2, lse2 = OA.attention_forward(q, k + u, v, 0.5, causal)
        np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse2, lse + 0.5 * (q @ u), rtol=0, atol=1e-11)


def pin_permutation_invariance():
    """P8: without a causal mask, permuting key/value positions together changes nothing."""
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 1, 2, 5, 8), _rand(rng, 1, 2, 10, 8), _rand(rng, 1, 2, 10, 8)
    perm = rng.permutation(10)
    O, lse = OA.attention_forward(q, k, v, 0.6, False)
    O2, lse2 = OA.attention_forward(q, k[:, :, perm], v[:, :, perm], 0.6, False)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


def pin_linear_in_v():
    """P9: O(a V1 + b V2) = a O(V1) + b O(V2)."""
    rng = np.random.default_rng(9)
    q, k = _rand(rng, 1, 2, 6, 8), _rand(rng, 1, 1, 6, 8)
    v1, v2 = _rand(rng, 1, 1, 6, 8), _rand(rng, 1, 1, 6, 8)
    for causal in (False, True):
        O1, _ = OA.attention_forward(q, k, v1, 0.5, causal)
        O2, _ = OA.attention_forward(q, k, v2, 0.5, causal)
        O12, _ = OA.attention_forward(q, k, 2.0 * v1 - 3.0 * v2, 0.5, causal)
        np.testing.assert_allclose(O12, 2.0 * O1 - 3.0 * O2, rtol=0, atol=1e-12)


def pin_causal_row_equals_decode():
    """P10: causal prefill row i equals decode of query i over i + 1 cached keys."""
    rng = np.random.default_rng(10)
    B, Hq, Hkv, N, D = 1, 4, 2, 12, 8
    q, k, v = _rand(rng, B, Hq, N, D), _rand(rng, B, Hkv, N, D), _rand(rng, B, Hkv, N, D)
    O, lse = OA.attention_forward(q, k, v, 0.45, True)
    for i in range(N):
        Od, lsed = OA.decode(q[:, :, i], k, v, i + 1, 0.45)
        np.testing.assert_allclose(Od, O[:, :, i], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lsed, lse[:, :, i], rtol=0, atol=1e-13)


def pin_decode_varlen():
    """P10b: per-sequence lengths -- each batch element against the mpmath brute
    force over its own prefix; equal lengths reduce to the scalar decode; a
    length of 0 gives O = 0 and lse = -inf."""
    rng = np.random.default_rng(101)
    B, Hq, Hkv, S, D = 4, 4, 2, 9, 5
    q, kc, vc = _rand(rng, B, Hq, D), _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    lens = [3, 0, 9, 1]
    O, lse = OA.decode_varlen(q, kc, vc, lens, 0.55)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(O[b] == 0.0) and np.all(lse[b] == -np.inf)
            continue
        Ob, lseb = _brute(q[b:b + 1, :, None, :], kc[b:b + 1, :, :L], vc[b:b + 1, :, :L], 0.55, False)
        np.testing.assert_allclose(O[b], Ob[0, :, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], lseb[0, :, 0], rtol=1e-12, atol=1e-12)
    Oe, lsee = OA.decode_varlen(q, kc, vc, [6] * B, 0.55)
    Od, lsed = OA.decode(q, kc, vc, 6, 0.55)
    np.testing.assert_array_equal(Oe, Od)
    np.testing.assert_array_equal(lsee, lsed)


def pin_sliding_window_rows_are_slices():
    """P6e: with a sliding window each query row equals unmasked attention over
    the explicit key slice [p - left, p + right] (clipped), p = i + offset, for
    causal and two-sided windows in both alignments; window sides of -1 stay
    open and a window covering everything is the plain mask."""
    rng = np.random.default_rng(64)
    B, Hq, Hkv, D = 1, 4, 2, 5
    for (Nq, Nkv, off, causal, wl, wr) in [(9, 9, 0, True, 3, -1), (9, 9, 0, False, 2, 1), (5, 12, 7, True, 4, -1),
                                            (6, 10, 4, False, 0, 3), (7, 7, 0, False, -1, 2), (8, 5, -3, True, 1, -1)]:
        q, k, v = _rand(rng, B, Hq, Nq, D), _rand(rng, B, Hkv, Nkv, D), _rand(rng, B, Hkv, Nkv, D)
        O, lse = OA.attention_forward(q, k, v, 0.7, causal, causal_offset=off, window=(wl, wr))
        for i in range(Nq):
            p = i + off
            lo = 0 if wl < 0 else max(0, p - wl)
            hi = min(Nkv - 1, p if causal else (Nkv - 1 if wr < 0 else p + wr))
            if wr >= 0:
                hi = min(hi, p + wr)
            if hi < lo:
                assert np.all(O[:, :, i] == 0.0) and np.all(lse[:, :, i] == -np.inf)
                continue
            Os, ls = OA.attention_forward(q[:, :, i:i + 1], k[:, :, lo:hi + 1], v[:, :, lo:hi + 1], 0.7, False)
            np.testing.assert_allclose(O[:, :, i], Os[:, :, 0], rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[:, :, i], ls[:, :, 0], rtol=0, atol=1e-13)
    q, k, v = _rand(rng, 1, 2, 6, 4), _rand(rng, 1, 1, 6, 4), _rand(rng, 1, 1, 6, 4)
    Ow, lw = OA.attention_forward(q, k, v, 0.5, True, window=(6, -1))
    Oc, lc = OA.attention_forward(q, k, v, 0.5, True)
    np.testing.assert_array_equal(Ow, Oc)
    np.testing.assert_array_equal(lw, lc)


def pin_zero_width_window_is_the_diagonal_key():
    """P6f: window (0, 0) leaves each query exactly one key, j = i + offset:
    O is that key's V row and lse its scaled score (closed form)."""
    rng = np.random.default_rng(65)
    q, k, v = _rand(rng, 1, 2, 5, 4), _rand(rng, 1, 1, 8, 4), _rand(rng, 1, 1, 8, 4)
    O, lse = OA.attention_forward(q, k, v, 0.9, False, causal_offset=3, window=(0, 0))
    for i in range(5):
        np.testing.assert_array_equal(O[0, :, i], np.repeat(v[0, 0, i + 3][None], 2, axis=0))
        np.testing.assert_allclose(lse[0, :, i], 0.9 * (q[0, :, i] @ k[0, 0, i + 3]), rtol=0, atol=1e-14)


def pin_decode_window_is_the_last_slots():
    """P10e: decode with a window of w keeps the last w + 1 cached slots: it
    equals decode over the cache shifted to start at slot L - 1 - w, for the
    contiguous, per-sequence and paged forms."""
    rng = np.random.default_rng(104)
    B, Hq, Hkv, S, D, w = 3, 4, 2, 16, 3, 5
    q, kc, vc = _rand(rng, B, Hq, D), _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    Ow, lw = OA.decode(q, kc, vc, 13, 0.5, window_left=w)
    Os, ls = OA.decode(q, kc[:, :, 13 - 1 - w:], vc[:, :, 13 - 1 - w:], w + 1, 0.5)
    np.testing.assert_allclose(Ow, Os, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lw, ls, rtol=0, atol=1e-14)
    lens = [13, 3, 0]
    Ov, lv = OA.decode_varlen(q, kc, vc, lens, 0.5, window_left=w)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(Ov[b] == 0.0) and np.all(lv[b] == -np.inf)
            continue
        lo = max(0, L - 1 - w)
        Ob, lb = OA.decode(q[b:b + 1], kc[b:b + 1, :, lo:L], vc[b:b + 1, :, lo:L], L - lo, 0.5)
        np.testing.assert_allclose(Ov[b], Ob[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lv[b], lb[0], rtol=0, atol=1e-14)
    perm = rng.permutation(B * (S // 4))
    kp, tbl = _scatter_to_pages(kc, perm, 4)
    vp, _ = _scatter_to_pages(vc, perm, 4)
    Op, lp = OA.decode_paged(q, kp, vp, tbl, lens, 4, 0.5, window_left=w)
    np.testing.assert_array_equal(Op, Ov)
    np.testing.assert_array_equal(lp, lv)


_BWD_MASKS = [(False, 0, (-1, -1)), (True, 0, (-1, -1)), (True, 2, (-1, -1)), (False, 1, (2, 1)), (True, 0, (1, -1))]


def pin_backward_finite_differences():
    """P11a: the backward equals central finite differences of the forward
    (L = sum(O * G)) for every element of Q, K and V, with no mask, causal in
    both alignments and sliding windows, GQA group of 2."""
    rng = np.random.default_rng(111)
    B, Hq, Hkv, Nq, Nkv, D, sc = 1, 2, 1, 4, 6, 3, 0.8
    q, k, v, g = _rand(rng, B, Hq, Nq, D), _rand(rng, B, Hkv, Nkv, D), _rand(rng, B, Hkv, Nkv, D), _rand(rng, B, Hq, Nq, D)
    eps = 1e-6
    for causal, off, win in _BWD_MASKS:
        def loss(qq, kk, vv):
            O, _ = OA.attention_forward(qq, kk, vv, sc, causal, causal_offset=off, window=win)
            return float((O * g).sum())
        dq, dk, dv = OA.attention_backward(q, k, v, g, sc, causal, causal_offset=off, window=win)
        for x, dx, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = xp, xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            np.testing.assert_allclose(dx, num, rtol=0, atol=2e-8)


def pin_backward_matches_torch_autograd():
    """P11b: the backward equals torch.autograd through an explicit float64
    attention on the CPU (GQA by repeat_interleave, masks as -inf scores)."""
    import torch
    rng = np.random.default_rng(112)
    B, Hq, Hkv, Nq, Nkv, D, sc = 2, 4, 2, 7, 9, 5, 0.6
    q, k, v, g = _rand(rng, B, Hq, Nq, D), _rand(rng, B, Hkv, Nkv, D), _rand(rng, B, Hkv, Nkv, D), _rand(rng, B, Hq, Nq, D)
    for causal, off, win in [(True, 0, (-1, -1)), (True, 2, (3, -1)), (False, 0, (1, 2))]:
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        kk = tk.repeat_interleave(Hq // Hkv, dim=1)
        vv = tv.repeat_interleave(Hq // Hkv, dim=1)
        S = sc * tq @ kk.transpose(-1, -2)
        i = torch.arange(Nq)[:, None] + off
        j = torch.arange(Nkv)[None, :]
        keep = torch.ones(Nq, Nkv, dtype=torch.bool)
        if causal:
            keep &= j <= i
        if win[0] >= 0:
            keep &= j >= i - win[0]
        if win[1] >= 0:
            keep &= j <= i + win[1]
        S = S.masked_fill(~keep, float("-inf"))
        P = torch.softmax(S, dim=-1).nan_to_num(0.0)
        (P @ vv * torch.tensor(g)).sum().backward()
        dq, dk, dv = OA.attention_backward(q, k, v, g, sc, causal, causal_offset=off, window=win)
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def pin_backward_gqa_is_group_sum():
    """P11c: GQA dK / dV are the sums over each group's q heads of the MHA
    gradients on K / V repeated per head; dQ is unchanged; and dK summed over
    keys is zero (O does not change when one vector is added to every key)."""
    rng = np.random.default_rng(113)
    B, Hq, Hkv, N, D = 1, 6, 2, 8, 4
    q, k, v, g = _rand(rng, B, Hq, N, D), _rand(rng, B, Hkv, N, D), _rand(rng, B, Hkv, N, D), _rand(rng, B, Hq, N, D)
    dq, dk, dv = OA.attention_backward(q, k, v, g, 0.5, True)
    ke, ve = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    dqe, dke, dve = OA.attention_backward(q, ke, ve, g, 0.5, True)
    np.testing.assert_allclose(dq, dqe, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, dke.reshape(B, Hkv, Hq // Hkv, N, D).sum(axis=2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, dve.reshape(B, Hkv, Hq // Hkv, N, D).sum(axis=2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-12)


def pin_varlen_backward_finite_differences():
    """P11d: the packed backward equals central finite differences of the
    packed forward (L = sum(O * G)) for every element, with an empty query set,
    a sequence without keys, L_q != L_k, bottom-right causal and a window."""
    rng = np.random.default_rng(114)
    Hq, Hkv, D, sc = 2, 1, 3, 0.7
    lens = [(3, 4), (0, 2), (2, 0), (2, 3)]
    cq = np.concatenate([[0], np.cumsum([a for a, _ in lens])])
    ck = np.concatenate([[0], np.cumsum([b for _, b in lens])])
    q, k, v = _rand(rng, int(cq[-1]), Hq, D), _rand(rng, int(ck[-1]), Hkv, D), _rand(rng, int(ck[-1]), Hkv, D)
    g = _rand(rng, int(cq[-1]), Hq, D)
    eps = 1e-6
    for causal, br, win in ((True, True, (-1, -1)), (False, False, (1, 1))):
        def loss(qq, kk, vv):
            O, _ = OA.attention_varlen(qq, kk, vv, cq, ck, sc, causal, bottom_right=br, window=win)
            return float((O * g).sum())
        dq, dk, dv = OA.attention_varlen_backward(q, k, v, g, cq, ck, sc, causal, bottom_right=br, window=win)
        for x, dx, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                ap, am = [q, k, v], [q, k, v]
                ap[which], am[which] = xp, xm
                num[idx] = (loss(*ap) - loss(*am)) / (2 * eps)
            np.testing.assert_allclose(dx, num, rtol=0, atol=2e-8)


def _scatter_to_pages(cache, perm, page_size):
    """Independent scatter of contiguous (B, Hkv, S, D) caches into a page pool:
    page perm[b * (S // page_size) + j] holds slots [j * ps, (j + 1) * ps) of sequence b."""
    B, H, S, D = cache.shape
    npb = S // page_size
    blocks = cache.reshape(B, H, npb, page_size, D).transpose(0, 2, 1, 3, 4).reshape(B * npb, H, page_size, D)
    pool = np.full((len(perm) + 3, H, page_size, D), np.nan)  # spare pages stay NaN
    pool[perm] = blocks
    table = np.asarray(perm).reshape(B, npb)
    return pool, table


def pin_decode_paged():
    """P10c: a paged cache scattered from contiguous caches through a shuffled
    block table decodes exactly like the per-sequence-length decode of the
    contiguous caches, and each sequence matches the mpmath brute force; the
    spare pages (NaN) are never read."""
    rng = np.random.default_rng(102)
    B, Hq, Hkv, S, D, ps = 3, 4, 2, 12, 5, 4
    q, kc, vc = _rand(rng, B, Hq, D), _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    perm = rng.permutation(B * (S // ps))
    kp, tbl = _scatter_to_pages(kc, perm, ps)
    vp, _ = _scatter_to_pages(vc, perm, ps)
    lens = [7, 0, 12]
    O, lse = OA.decode_paged(q, kp, vp, tbl, lens, ps, 0.6)
    Ov, lsev = OA.decode_varlen(q, kc, vc, lens, 0.6)
    np.testing.assert_array_equal(O, Ov)
    np.testing.assert_array_equal(lse, lsev)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(O[b] == 0.0) and np.all(lse[b] == -np.inf)
            continue
        Ob, lseb = _brute(q[b:b + 1, :, None, :], kc[b:b + 1, :, :L], vc[b:b + 1, :, :L], 0.6, False)
        np.testing.assert_allclose(O[b], Ob[0, :, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], lseb[0, :, 0], rtol=1e-12, atol=1e-12)


def pin_cache_write_paged():
    """P10d: the paged writer equals the contiguous writer applied per sequence
    (at that sequence's position) and scattered through the same block table."""
    rng = np.random.default_rng(103)
    B, Hkv, S, D, ps, T = 3, 2, 16, 3, 4, 3
    kc, vc = _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    kn, vn = _rand(rng, B, Hkv, T, D), _rand(rng, B, Hkv, T, D)
    perm = rng.permutation(B * (S // ps))
    kp, tbl = _scatter_to_pages(kc, perm, ps)
    vp, _ = _scatter_to_pages(vc, perm, ps)
    pos = [0, 5, S - T]
    kp2, vp2 = OA.kv_cache_write_paged(kp, vp, kn, vn, tbl, pos, ps)
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(B):
        kc2[b:b + 1], vc2[b:b + 1] = OA.kv_cache_write(kc[b:b + 1], vc[b:b + 1], kn[b:b + 1], vn[b:b + 1], pos[b])
    ke, _ = _scatter_to_pages(kc2, perm, ps)
    ve, _ = _scatter_to_pages(vc2, perm, ps)
    np.testing.assert_array_equal(kp2, ke)
    np.testing.assert_array_equal(vp2, ve)


def pin_prefill_varlen():
    """P6d: packed sequences of different lengths -- each sequence against the
    mpmath brute force on its own rows only (no key of another sequence may
    contribute), for no mask, top-left and bottom-right causal.  Lengths cover
    empty query sets, empty key sets (O = 0, lse = -inf), L_q < L_k and L_q > L_k."""
    rng = np.random.default_rng(63)
    Hq, Hkv, D = 4, 2, 3
    lens = [(3, 3), (0, 2), (4, 0), (2, 6), (5, 2), (1, 1)]
    cq = np.concatenate([[0], np.cumsum([a for a, _ in lens])])
    ck = np.concatenate([[0], np.cumsum([b for _, b in lens])])
    q, k, v = _rand(rng, int(cq[-1]), Hq, D), _rand(rng, int(ck[-1]), Hkv, D), _rand(rng, int(ck[-1]), Hkv, D)
    for causal, br in ((False, False), (True, False), (True, True)):
        O, lse = OA.attention_varlen(q, k, v, cq, ck, 0.8, causal, bottom_right=br)
        assert O.shape == q.shape and lse.shape == (Hq, q.shape[0])
        for b, (Lq, Lk) in enumerate(lens):
            rq, rk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
            if Lq == 0:
                continue
            if Lk == 0:
                assert np.all(O[rq] == 0.0) and np.all(lse[:, rq] == -np.inf)
                continue
            qs, ks, vs = (x.transpose(1, 0, 2)[None] for x in (q[rq], k[rk], v[rk]))
            Ob, lseb = _brute(qs, ks, vs, 0.8, causal, offset=(Lk - Lq) if br else 0)
            np.testing.assert_allclose(O[rq], Ob[0].transpose(1, 0, 2), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[:, rq], lseb[0], rtol=1e-12, atol=1e-12)
    # sampled rows give the same values as the full evaluation (up to the
    # matmul's blocking over a different number of rows)
    rows = np.array([0, 2, 7, 9, 13, int(cq[-1]) - 1])
    Os, ls = OA.attention_varlen(q, k, v, cq, ck, 0.8, True, bottom_right=True, rows=rows)
    np.testing.assert_allclose(Os, O[rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(ls, lse[:, rows], rtol=0, atol=1e-14)


def pin_row_sampling_matches_full():
    """Evaluating a subset of rows gives the same values as the full evaluation."""
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 1, 2, 40, 8), _rand(rng, 1, 1, 40, 8), _rand(rng, 1, 1, 40, 8)
    rows = np.array([0, 3, 17, 39])
    for causal in (False, True):
        O, lse = OA.attention_forward(q, k, v, 0.5, causal, chunk=7)
        Os, lses = OA.attention_forward(q, k, v, 0.5, causal, rows=rows)
        np.testing.assert_array_equal(Os, O[:, :, rows])
        np.testing.assert_array_equal(lses, lse[:, :, rows])


def pin_cache_write_touches_only_its_slots():
    rng = np.random.default_rng(12)
    kc = rng.integers(0, 2**16, (2, 3, 10, 4), dtype=np.uint16)
    vc = rng.integers(0, 2**16, (2, 3, 10, 4), dtype=np.uint16)
    kn = rng.integers(0, 2**16, (2, 3, 3, 4), dtype=np.uint16)
    vn = rng.integers(0, 2**16, (2, 3, 3, 4), dtype=np.uint16)
    k2, v2 = OA.kv_cache_write(kc, vc, kn, vn, 6)
    np.testing.assert_array_equal(k2[:, :, 6:9], kn)
    np.testing.assert_array_equal(v2[:, :, 6:9], vn)
    np.testing.assert_array_equal(np.delete(k2, [6, 7, 8], axis=2), np.delete(kc, [6, 7, 8], axis=2))
    np.testing.assert_array_equal(np.delete(v2, [6, 7, 8], axis=2), np.delete(vc, [6, 7, 8], axis=2))


ALL_PINS = [
    pin_golden_prefill,
    pin_golden_decode,
    pin_golden_cache_write,
    pin_rows_sum_to_one,
    pin_probs_head_mapping,
    pin_causal_row0_is_v0,
    pin_equal_scores_give_mean,
    pin_single_key,
    pin_gqa_equals_expanded_mha,
    pin_brute_force_tiny,
    pin_brute_force_bottom_right,
    pin_bottom_right_is_the_tail_of_full_causal,
    pin_shift_invariance,
    pin_permutation_invariance,
    pin_linear_in_v,
    pin_causal_row_equals_decode,
    pin_decode_varlen,
    pin_prefill_varlen,
    pin_decode_paged,
    pin_cache_write_paged,
    pin_backward_finite_differences,
    pin_backward_matches_torch_autograd,
    pin_backward_gqa_is_group_sum,
    pin_varlen_backward_finite_differences,
    pin_sliding_window_rows_are_slices,
    pin_zero_width_window_is_the_diagonal_key,
    pin_decode_window_is_the_last_slots,
    pin_row_sampling_matches_full,
    pin_cache_write_touches_only_its_slots,
]


def pin_brute_force_tiny_config():
    """P6 on the full tiny prefill workload (B=1, Hq=2, Hkv=1, N=65, D=64, fp16, causal)."""
    from workloads import TINY, prefill_inputs
    q, k, v = (t.float().numpy().astype(np.float64) for t in prefill_inputs(TINY))
    rows = np.array([0, 1, 31, 32, 63, 64])
    O, lse = OA.attention_forward(q, k, v, TINY.softmax_scale, True, rows=rows)
    # brute force of selected rows: evaluate row-by-row with the causal prefix made explicit
    for idx, i in enumerate(rows):
        Oi, lsei = _brute(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], TINY.softmax_scale, False)
        np.testing.assert_allclose(O[:, :, idx], Oi[:, :, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, :, idx], lsei[:, :, 0], rtol=1e-12, atol=1e-12)


ALL_PINS.append(pin_brute_force_tiny_config)
