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


MUTATIONS = {
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
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutation {name}"
