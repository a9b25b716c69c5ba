"""Planted mistakes in the oracle must each trip at least one pin.

Every mutation below is a plausible bug (a flipped comparison, a wrong head
mapping, a dropped term, an off-by-one).  Each is planted in the oracle module
on the CPU with monkeypatch; the test asserts that running the full pin set
against the mutated oracle fails.  This shows the pins constrain every part of
the oracle rather than only re-deriving it.
"""

import numpy as np
import pytest

import oracle.attention as OA
from oracle_pins import ALL_PINS

_orig_vis = OA.visibility
_orig_soft = OA._masked_softmax
_orig_scores = OA._scores
_orig_decode = OA.decode
_orig_write = OA.kv_cache_write
_orig_varlen = OA.decode_varlen
_orig_bounds = OA.sequence_bounds
_orig_vcoff = OA.varlen_causal_offset
_orig_pslot = OA.page_slot
_orig_bwd = OA.attention_backward


def _bwd_variant(drop_rowsum=False, dk_unscaled=False, gqa_overwrite=False, dq_uses_v=False):
    def bwd(q, k, v, do, scale, causal, causal_offset=0, window=(-1, -1)):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        B, Hq, Nq, D = q.shape
        Hkv, Nkv = k.shape[1], k.shape[2]
        vis = OA.visibility(np.arange(Nq), Nkv, causal, causal_offset, window[0], window[1])
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                g = OA.kv_head_of(h, Hq, Hkv)
                P, _ = OA._masked_softmax(OA._scores(q[b, h], k[b, g], scale), vis)
                dP = do[b, h] @ v[b, g].T
                dS = P * dP if drop_rowsum else P * (dP - (P * dP).sum(axis=1, keepdims=True))
                if gqa_overwrite:
                    dv[b, g] = P.T @ do[b, h]
                else:
                    dv[b, g] += P.T @ do[b, h]
                dq[b, h] = scale * (dS @ (v[b, g] if dq_uses_v else k[b, g]))
                dk[b, g] += (1.0 if dk_unscaled else scale) * (dS.T @ q[b, h])
        return dq, dk, dv
    return bwd


def _vis_strict(q_pos, Nkv, causal, offset=0, window_left=-1, window_right=-1):
    j = np.arange(Nkv)
    vis = _orig_vis(q_pos, Nkv, False, offset, window_left, window_right)
    if causal:
        vis &= j[None, :] < q_pos[:, None] + offset
    return vis


def _vis_no_causal(q_pos, Nkv, causal, offset=0, window_left=-1, window_right=-1):
    return _orig_vis(q_pos, Nkv, False, offset, window_left, window_right)


def _vis_off_by_one(q_pos, Nkv, causal, offset=0, window_left=-1, window_right=-1):
    return _orig_vis(q_pos + 1, Nkv, causal, offset, window_left, window_right)


def _vis_offset_ignored(q_pos, Nkv, causal, offset=0, window_left=-1, window_right=-1):
    return _orig_vis(q_pos, Nkv, causal, 0, window_left, window_right)


def _vis_offset_sign(q_pos, Nkv, causal, offset=0, window_left=-1, window_right=-1):
    return _orig_vis(q_pos, Nkv, causal, -offset, window_left, window_right)


def _vis_window_ignored(q_pos, Nkv, causal, offset=0, window_left=-1, window_right=-1):
    return _orig_vis(q_pos, Nkv, causal, offset)


def _vis_window_left_strict(q_pos, Nkv, causal, offset=0, window_left=-1, window_right=-1):
    return _orig_vis(q_pos, Nkv, causal, offset, window_left - 1 if window_left > 0 else window_left, window_right)


def _vis_window_sides_swapped(q_pos, Nkv, causal, offset=0, window_left=-1, window_right=-1):
    return _orig_vis(q_pos, Nkv, causal, offset, window_right, window_left)


def _kv_head_tiled(h, Hq, Hkv):
    return h % Hkv


def _scores_unscaled(q_rows, k, scale):
    return _orig_scores(q_rows, k, 1.0)


def _scores_scaled_twice(q_rows, k, scale):
    return _orig_scores(q_rows, k, scale * scale)


def _soft_lse_is_max(S, vis):
    P, lse = _orig_soft(S, vis)
    Sm = np.where(vis, S, -np.inf)
    return P, Sm.max(axis=1)


def _soft_unnormalised(S, vis):
    Sm = np.where(vis, S, -np.inf)
    m = Sm.max(axis=1)
    E = np.where(vis, np.exp(Sm - m[:, None]), 0.0)
    return E, m + np.log(E.sum(1))


def _soft_base2(S, vis):
    return _orig_soft(S * np.log2(np.e) * np.log(2.0) ** 2, vis)


def _soft_mask_ignored_in_sum(S, vis):
    Sm = np.where(vis, S, -np.inf)
    m = Sm.max(axis=1)
    E = np.exp(S - m[:, None])  # masked keys leak into the sum
    l = E.sum(1)
    return np.where(vis, E, 0.0) / l[:, None], m + np.log(l)


def _decode_reads_one_more(q, k_cache, v_cache, cache_len, scale):
    n = min(cache_len + 1, np.asarray(k_cache).shape[2])
    return _orig_decode(q, k_cache, v_cache, n, scale)


def _varlen_longest_for_all(q, k_cache, v_cache, cache_lens, scale):
    L = max(int(x) for x in cache_lens)
    return _orig_varlen(q, k_cache, v_cache, [L] * len(cache_lens), scale)


def _varlen_off_by_one(q, k_cache, v_cache, cache_lens, scale):
    S = np.asarray(k_cache).shape[2]
    return _orig_varlen(q, k_cache, v_cache, [min(int(x) + 1, S) for x in cache_lens], scale)


def _bounds_from_zero(cu_seqlens, b):
    # every sequence starts at packed row 0 (offsets read as lengths)
    _, e = _orig_bounds(cu_seqlens, b)
    return 0, e - _orig_bounds(cu_seqlens, b)[0]


def _bounds_one_past(cu_seqlens, b):
    s, e = _orig_bounds(cu_seqlens, b)
    n = int(np.asarray(cu_seqlens).reshape(-1)[-1])
    return s, min(e + 1, n) if e > s else e


def _vcoff_swapped(Lq, Lk, bottom_right):
    return _orig_vcoff(Lk, Lq, bottom_right)


def _vcoff_always_top_left(Lq, Lk, bottom_right):
    return 0


def _pslot_row_and_page_swapped(block_table, b, r, page_size):
    return int(np.asarray(block_table)[b, r % page_size]), r // page_size


def _pslot_next_sequence(block_table, b, r, page_size):
    tbl = np.asarray(block_table)
    return _orig_pslot(tbl, (b + 1) % tbl.shape[0], r, page_size)


def _pslot_row_off_by_one(block_table, b, r, page_size):
    p, i = _orig_pslot(block_table, b, r, page_size)
    return p, (i + 1) % page_size


def _write_shifted(k_cache, v_cache, k_new, v_new, pos):
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    T = np.asarray(k_new).shape[2]
    p = min(pos + 1, kc.shape[2] - T)
    kc[:, :, p:p + T] = k_new
    vc[:, :, p:p + T] = v_new
    return kc, vc


def _probs_heads_tiled(q, k, scale, causal, causal_offset=0):
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    B, Hq, Nq, _ = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    out = np.zeros((B, Hq, Nq, Nkv))
    vis = OA.visibility(np.arange(Nq), Nkv, causal, causal_offset)
    for b in range(B):
        for h in range(Hq):
            out[b, h], _ = OA._masked_softmax(OA._scores(q[b, h], k[b, h % Hkv], scale), vis)
    return out


MUTATIONS = {
    "causal_strict_lt": ("visibility", _vis_strict),
    "causal_ignored": ("visibility", _vis_no_causal),
    "causal_off_by_one": ("visibility", _vis_off_by_one),
    "causal_offset_ignored": ("visibility", _vis_offset_ignored),
    "causal_offset_sign": ("visibility", _vis_offset_sign),
    "window_ignored": ("visibility", _vis_window_ignored),
    "window_left_one_short": ("visibility", _vis_window_left_strict),
    "window_sides_swapped": ("visibility", _vis_window_sides_swapped),
    "gqa_tiled_heads": ("kv_head_of", _kv_head_tiled),
    "probs_heads_tiled": ("attention_probs", _probs_heads_tiled),
    "scale_dropped": ("_scores", _scores_unscaled),
    "scale_twice": ("_scores", _scores_scaled_twice),
    "lse_missing_log_l": ("_masked_softmax", _soft_lse_is_max),
    "p_not_normalised": ("_masked_softmax", _soft_unnormalised),
    "exp_wrong_base": ("_masked_softmax", _soft_base2),
    "masked_keys_in_sum": ("_masked_softmax", _soft_mask_ignored_in_sum),
    "decode_reads_past_cache_len": ("decode", _decode_reads_one_more),
    "cache_write_off_by_one": ("kv_cache_write", _write_shifted),
    "varlen_longest_for_all": ("decode_varlen", _varlen_longest_for_all),
    "varlen_reads_one_more": ("decode_varlen", _varlen_off_by_one),
    "paged_row_and_page_swapped": ("page_slot", _pslot_row_and_page_swapped),
    "paged_other_sequences_table": ("page_slot", _pslot_next_sequence),
    "paged_row_off_by_one": ("page_slot", _pslot_row_off_by_one),
    "bwd_softmax_jacobian_rowsum_dropped": ("attention_backward", _bwd_variant(drop_rowsum=True)),
    "bwd_dk_scale_dropped": ("attention_backward", _bwd_variant(dk_unscaled=True)),
    "bwd_gqa_dv_overwritten": ("attention_backward", _bwd_variant(gqa_overwrite=True)),
    "bwd_dq_uses_v": ("attention_backward", _bwd_variant(dq_uses_v=True)),
    "packed_offsets_as_lengths": ("sequence_bounds", _bounds_from_zero),
    "packed_row_past_sequence": ("sequence_bounds", _bounds_one_past),
    "packed_causal_offset_swapped": ("varlen_causal_offset", _vcoff_swapped),
    "packed_bottom_right_ignored": ("varlen_causal_offset", _vcoff_always_top_left),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(OA, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception:  # assertion or a crash both mean the mutation is visible
            caught.append(pin.__name__)
            break
    assert caught, f"mutation {name} passed every pin"
