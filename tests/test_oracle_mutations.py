"""Plant plausible mistakes in the CPU oracle and check that at least one pin catches each.

Every mutation below is a slip someone could make while writing the method down (dropped term,
wrong index or head, wrong tie rule, transposed operand, missing mask).  All of it runs on the CPU.
"""
import math

import numpy as np
import pytest

import oracle_pins
from oracle import hils_oracle as O


def _bf16_truncate(x):
    a = np.ascontiguousarray(x, dtype=np.float32)
    return (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).reshape(a.shape)


def _wrong_head_prefill_rows(inp, rows, chunk, topk, dtype, scale=None, _orig=O.prefill_rows):
    if "w_up" in inp:
        d = inp["q"].shape[-1]
        w_up = inp["w_up"].copy()
        w_up[d:2 * d] = inp["w_up"][:d]          # every head uses head 0's rows
        inp = dict(inp, w_up=w_up)
    return _orig(inp, rows, chunk, topk, dtype, scale)


def _row_with(score_query="q_tilde", attend_query="q", own_chunk=True):
    def hils_row(q_row, q_tilde, keys, values, lmk, i, chunk, topk, scale):
        c = i // chunk
        ncand = c + 1 if own_chunk else max(c, 1)
        sigma = O.landmark_scores(q_tilde if score_query == "q_tilde" else q_row, lmk[:ncand])
        idx = O.select_top_k(sigma, topk)
        sel = idx[idx >= 0]
        w = np.zeros(topk)
        w[: len(sel)] = O.inter_chunk_weights(sigma[sel], scale)
        o = O.attend_row(q_row if attend_query == "q" else q_tilde, keys, values, idx, w, i, chunk, scale)
        return o, idx, w, sigma
    return hils_row


def _topk_ties_high(sigma, k):
    s = np.asarray(sigma, dtype=np.float64)
    order = sorted(range(len(s)), key=lambda j: (-s[j], -j))[:k]
    out = np.full(k, -1)
    out[: len(order)] = sorted(order)
    return out


def _topk_smallest(sigma, k):
    s = np.asarray(sigma, dtype=np.float64)
    order = sorted(range(len(s)), key=lambda j: (s[j], j))[:k]
    out = np.full(k, -1)
    out[: len(order)] = sorted(order)
    return out


def _given_weights_over_padding(q_row, keys, values, idx, sigma_selected, i, chunk, scale):
    idx = np.asarray(idx)
    w = O.inter_chunk_weights(np.asarray(sigma_selected), scale)     # padded entries included
    return O.attend_row(q_row, keys, values, idx, w, i, chunk, scale)


def _given_sigma_reversed(q_row, keys, values, idx, sigma_selected, i, chunk, scale,
                          _o=O.attend_given_selection):
    idx = np.asarray(idx)
    sig = np.array(sigma_selected, dtype=np.float32)
    n = int((idx >= 0).sum())
    sig[:n] = sig[:n][::-1]
    return _o(q_row, keys, values, idx, sig, i, chunk, scale)


def _chunk_bwd_dv_unweighted(q, K, V, w_j, g, scale, _o=O.chunk_backward):
    dq, dK, dV, dw = _o(q, K, V, w_j, g, scale)
    return dq, dK, dV / max(w_j, 1e-300), dw


def _chunk_bwd_dk_unscaled(q, K, V, w_j, g, scale, _o=O.chunk_backward):
    dq, dK, dV, dw = _o(q, K, V, w_j, g, scale)
    return dq, dK / scale, dV, dw


def _chunk_bwd_no_softmax_centering(q, K, V, w_j, g, scale):
    q, K, V, g = (np.asarray(x, dtype=np.float64) for x in (q, K, V, g))
    a = scale * (K @ q)
    p = np.exp(a - a.max())
    p /= p.sum()
    dp = w_j * (V @ g)
    da = p * dp
    return scale * (da @ K), scale * np.outer(da, q), np.outer(w_j * p, g), float(g @ (p @ V))


def _local_not_forced(sigma, k):
    return O.select_top_k(sigma, k)


def _local_drops_wrong_one(sigma, k):
    s = np.asarray(sigma)
    own = s.shape[0] - 1
    top = O.select_top_k(s, k)
    if own in set(int(j) for j in top if j >= 0):
        return top
    chosen = sorted([int(j) for j in top if j >= 0][1:] + [own])     # drops the smallest index
    out = np.full(k, -1)
    out[: len(chosen)] = chosen
    return out


def _hope_half_split(x, positions, rope_base, train_len):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    pos = np.broadcast_to(np.asarray(positions, dtype=np.float64), x.shape[-2:-1])
    out = x.copy()
    for i in O.hope_rotated_pairs(d, rope_base, train_len):
        ang = pos * float(rope_base) ** (-2.0 * i / d)
        a, b = x[..., i], x[..., i + d // 2]
        out[..., i] = a * np.cos(ang) - b * np.sin(ang)
        out[..., i + d // 2] = a * np.sin(ang) + b * np.cos(ang)
    return out


def _hope_theta_exponent(x, positions, rope_base, train_len):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    pos = np.broadcast_to(np.asarray(positions, dtype=np.float64), x.shape[-2:-1])
    out = x.copy()
    for i in O.hope_rotated_pairs(d, rope_base, train_len):
        ang = pos * float(rope_base) ** (-1.0 * i / d)
        a, b = x[..., 2 * i], x[..., 2 * i + 1]
        out[..., 2 * i] = a * np.cos(ang) - b * np.sin(ang)
        out[..., 2 * i + 1] = a * np.sin(ang) + b * np.cos(ang)
    return out


def _hope_window_reversed(d, rope_base, train_len, _o=O.hope_rotated_pairs):
    inside = set(int(i) for i in _o(d, rope_base, train_len))
    return np.asarray([i for i in range(d // 2) if i not in inside], dtype=np.int64)


def _partial_landmark_over_chunk(k_cache, kv_len, chunk, dtype):
    # divides the chunk's key sum by C instead of by the keys present
    out = {}
    for (b, g), (j, lm) in O.__dict__["_orig_partial_landmark"](k_cache, kv_len, chunk, dtype).items():
        n = min(max(int(kv_len[b]), 1), k_cache.shape[2]) - j * chunk
        out[(b, g)] = (j, O.round_to_run_dtype(np.asarray(lm, np.float64) * n / chunk, dtype))
    return out


def _partial_landmark_wrong_chunk(k_cache, kv_len, chunk, dtype):
    # takes the chunk of position kv_len rather than of the newest key kv_len - 1
    return O.__dict__["_orig_partial_landmark"](k_cache, np.asarray(kv_len) + 1, chunk, dtype)


O._orig_partial_landmark = O.partial_landmark

MUTATIONS = {
    "partial_landmark_over_chunk": ("partial_landmark", _partial_landmark_over_chunk),
    "partial_landmark_wrong_chunk": ("partial_landmark", _partial_landmark_wrong_chunk),
    "hope_rotation_reversed": ("hope_rotate", lambda x, p, b, t, _o=O.hope_rotate: _o(x, -np.asarray(p), b, t)),
    "hope_half_split_pairs": ("hope_rotate", _hope_half_split),
    "hope_theta_exponent": ("hope_rotate", _hope_theta_exponent),
    "hope_window_reversed": ("hope_rotated_pairs", _hope_window_reversed),
    "forced_local_ignored": ("select_with_local", _local_not_forced),
    "forced_local_drops_wrong_chunk": ("select_with_local", _local_drops_wrong_one),
    "bwd_dsigma_not_centred": ("inter_chunk_backward", lambda w, dw, s: s * np.asarray(w) * np.asarray(dw)),
    "bwd_dsigma_unscaled": ("inter_chunk_backward",
                            lambda w, dw, s, _o=O.inter_chunk_backward: _o(w, dw, 1.0) if s != 1.0 else 2 * _o(w, dw, s)),
    "bwd_dv_unweighted": ("chunk_backward", _chunk_bwd_dv_unweighted),
    "bwd_dk_unscaled": ("chunk_backward", _chunk_bwd_dk_unscaled),
    "bwd_softmax_not_centred": ("chunk_backward", _chunk_bwd_no_softmax_centering),
    "dense_attends_next_key": ("_causal_end", lambda i: i + 2),
    "dense_misses_itself": ("_causal_end", lambda i: max(i, 1)),
    "dense_unscaled": ("dense_attention_row",
                       lambda q, K, V, s, _o=O.dense_attention_row: _o(q, K, V, 1.0)),
    "dense_keys_values_swapped": ("dense_attention_row",
                                  lambda q, K, V, s, _o=O.dense_attention_row: _o(q, V, K, s)),
    "given_selection_weights_over_padding": ("attend_given_selection", _given_weights_over_padding),
    "given_selection_sigma_reversed": ("attend_given_selection", _given_sigma_reversed),
    "qcal_dropped": ("calibrated_query", lambda q, h, wd, wu, dt: O.round_to_run_dtype(q, dt)),
    "qcal_wrong_head": ("prefill_rows", _wrong_head_prefill_rows),
    "qcal_sign_flipped": ("qcal_offset", lambda h, wd, wu, _o=O.qcal_offset: -_o(h, wd, wu)),
    "bf16_truncates": ("round_to_bf16", _bf16_truncate),
    "scores_use_raw_query": ("hils_row", _row_with(score_query="q")),
    "attention_uses_calibrated_query": ("hils_row", _row_with(attend_query="q_tilde")),
    "own_chunk_not_candidate": ("hils_row", _row_with(own_chunk=False)),
    "topk_ties_to_larger_index": ("select_top_k", _topk_ties_high),
    "topk_picks_smallest": ("select_top_k", _topk_smallest),
    "weights_unscaled": ("inter_chunk_weights", lambda s, scale, _o=O.inter_chunk_weights: _o(s, 1.0)),
    "weights_uniform": ("inter_chunk_weights", lambda s, scale: np.full(len(s), 1.0 / len(s))),
    "no_causal_truncation": ("_visible_range", lambda j, C, i: (j * C, j * C + C)),
    "query_misses_itself": ("_visible_range", lambda j, C, i: (j * C, max(j * C + 1, min(j * C + C, i)))),
    "intra_softmax_unscaled": ("intra_chunk_attention",
                               lambda q, K, V, s, _o=O.intra_chunk_attention: _o(q, K, V, 1.0)),
    "intra_keys_values_swapped": ("intra_chunk_attention",
                                  lambda q, K, V, s, _o=O.intra_chunk_attention: _o(q, V, K, s)),
    "fusion_drops_weights": ("fuse", lambda ws, outs, _o=O.fuse: _o([1.0] * len(ws), outs)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, fake = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fake)
    caught = []
    # the finite-difference pin is the slowest: it runs only if no other pin catches the mutation
    for pin in sorted(oracle_pins.ALL_PINS, key=lambda p: p.__name__ == "pin_backward_finite_differences"):
        try:
            pin()
        except Exception:
            caught.append(pin.__name__)
            break
    assert caught, f"no pin catches mutation {name}"
