"""Pins of the CPU oracle to facts fixed outside it (mathematics, library routines, closed forms).

Each pin raises AssertionError when the oracle disagrees.  test_oracle_pins.py runs them; the
mutation test plants plausible mistakes in the oracle and checks that some pin catches each one.
Nothing here reuses the oracle's own arithmetic to build an expected value.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import scipy.special

from oracle import hils_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _small_inputs(seed=0, B=1, H=2, L=256, d=16, C=64, r=4, D=24, dtype="fp32", wstd=0.3):
    """Small random prefill inputs (fp32 values; bf16-exact when dtype == 'bf16')."""
    g = _rng(seed)
    rnd = lambda *s: g.standard_normal(s).astype(np.float32)
    inp = dict(q=rnd(B, H, L, d), k=rnd(B, H, L, d), v=rnd(B, H, L, d), lmk=rnd(B, H, L // C, d) * 0.5)
    if r:
        inp.update(h=rnd(B, L, D), w_down=rnd(r, D) * wstd, w_up=rnd(H * d, r) * wstd)
    if dtype == "bf16":
        import torch
        for key in list(inp):
            inp[key] = torch.from_numpy(inp[key]).to(torch.bfloat16).float().numpy()
    return inp


def _dense_causal(q, k, v, scale):
    """Textbook causal softmax attention in matrix form, float64 (scipy softmax)."""
    a = scale * (q.astype(np.float64) @ k.astype(np.float64).T)
    L = a.shape[0]
    a[np.triu_indices(L, 1)] = -np.inf
    return scipy.special.softmax(a, axis=1) @ v.astype(np.float64)


# ---------------------------------------------------------------------------------------------
# Rounding
# ---------------------------------------------------------------------------------------------

def pin_bf16_known_values():
    one = 1.0
    cases = {
        one: one,
        one + 2.0 ** -8: one,                       # halfway, lower neighbour has even mantissa
        one + 3 * 2.0 ** -8: one + 2.0 ** -6,       # halfway, upper neighbour has even mantissa
        one + 2.0 ** -8 + 2.0 ** -20: one + 2.0 ** -7,
        -(one + 2.0 ** -8): -one,
        3.0: 3.0,
        0.0: 0.0,
    }
    for x, want in cases.items():
        got = float(O.round_to_bf16(np.array([x], dtype=np.float32))[0])
        assert got == want, (x, got, want)


def pin_bf16_matches_torch():
    import torch
    x = (_rng(1).standard_normal(200000) * np.exp(_rng(2).uniform(-20, 20, 200000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = O.round_to_bf16(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------------------------------------
# Q-Cal
# ---------------------------------------------------------------------------------------------

def pin_qcal_reassociated():
    """delta_q = W_up W_down h computed as (W_up W_down) h in matrix form."""
    inp = _small_inputs(3)
    d = inp["q"].shape[-1]
    for head in range(2):
        wu = inp["w_up"][head * d:(head + 1) * d].astype(np.float64)
        M = wu @ inp["w_down"].astype(np.float64)
        for i in (0, 77, 255):
            want = M @ inp["h"][0, i].astype(np.float64)
            got = O.qcal_offset(inp["h"][0, i], inp["w_down"], inp["w_up"][head * d:(head + 1) * d])
            assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def pin_qcal_identity_cases():
    inp = _small_inputs(4)
    d = inp["q"].shape[-1]
    q = inp["q"][0, 1, 5]
    assert np.array_equal(O.calibrated_query(q, None, None, None, "fp32"), q)
    z = O.calibrated_query(q, inp["h"][0, 5], np.zeros_like(inp["w_down"]), inp["w_up"][d:2 * d], "fp32")
    assert np.array_equal(z, q)


def pin_qcal_head_rows_and_rounding():
    """Only head h's rows of W_up move head h's query; bf16 runs round q + delta_q once (torch RNE)."""
    import torch
    inp = _small_inputs(5, dtype="bf16")
    d = inp["q"].shape[-1]
    w_up = inp["w_up"].copy()
    w_up[:d] = 0.0                      # head 0 gets no offset
    res = O.prefill_rows(dict(inp, w_up=w_up), [(0, 0, 9), (0, 1, 9)], 64, 2, "bf16")
    assert np.array_equal(res[(0, 0, 9)]["q_tilde"], inp["q"][0, 0, 9])
    dq = (w_up[d:2 * d].astype(np.float64) @ (inp["w_down"].astype(np.float64) @ inp["h"][0, 9].astype(np.float64)))
    s32 = (inp["q"][0, 1, 9].astype(np.float64) + dq.astype(np.float32).astype(np.float64)).astype(np.float32)
    want = torch.from_numpy(s32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(res[(0, 1, 9)]["q_tilde"], want)
    assert not np.array_equal(want, inp["q"][0, 1, 9])


# ---------------------------------------------------------------------------------------------
# Landmark scores
# ---------------------------------------------------------------------------------------------

def pin_scores_exact_sum():
    """sigma_j equals the exactly rounded dot product (math.fsum) of q~ and lmk_j."""
    inp = _small_inputs(6, dtype="bf16")
    res = O.prefill_rows(inp, [(0, 1, 200)], 64, 2, "bf16")[(0, 1, 200)]
    qt = res["q_tilde"]
    for j in range(200 // 64 + 1):
        exact = math.fsum(float(a) * float(b) for a, b in zip(qt, inp["lmk"][0, 1, j]))
        assert res["sigma"][j] == np.float32(exact), (j, res["sigma"][j], exact)


def pin_scores_use_calibrated_query():
    inp = _small_inputs(7)
    res = O.prefill_rows(inp, [(0, 0, 130)], 64, 2, "fp32")[(0, 0, 130)]
    raw = np.array([math.fsum(float(a) * float(b) for a, b in zip(inp["q"][0, 0, 130], inp["lmk"][0, 0, j]))
                    for j in range(3)])
    assert np.max(np.abs(res["sigma"] - raw)) > 1e-3


# ---------------------------------------------------------------------------------------------
# Top-k
# ---------------------------------------------------------------------------------------------

def _dominates(s, x, y):
    return s[x] > s[y] or (s[x] == s[y] and x < y)


def pin_topk_bruteforce():
    """The selected set is the unique k-subset whose members all beat all non-members (ties to the
    smaller index), found by enumerating every subset."""
    g = _rng(8)
    for trial in range(300):
        n = int(g.integers(1, 8))
        k = int(g.integers(1, 9))
        s = g.integers(-3, 4, n).astype(np.float32)         # many ties
        got = O.select_top_k(s, k)
        keff = min(k, n)
        winners = [set(S) for S in itertools.combinations(range(n), keff)
                   if all(_dominates(s, x, y) for x in S for y in range(n) if y not in S)]
        assert len(winners) == 1
        assert list(got[:keff]) == sorted(winners[0]) and all(got[keff:] == -1), (s, k, got)


def pin_topk_matches_stable_sort():
    g = _rng(9)
    for trial in range(50):
        n = int(g.integers(1, 300))
        k = int(g.integers(1, 65))
        s = np.round(g.standard_normal(n), 1).astype(np.float32)
        order = np.argsort(-s.astype(np.float64), kind="stable")[:k]
        got = O.select_top_k(s, k)
        want = np.full(k, -1)
        want[:len(order)] = np.sort(order)
        assert np.array_equal(got, want)


# ---------------------------------------------------------------------------------------------
# Inter-chunk softmax
# ---------------------------------------------------------------------------------------------

def pin_weights_closed_form():
    s = 0.125
    w = O.inter_chunk_weights(np.array([3.0, 1.0], dtype=np.float32), s)
    assert abs(w[0] - 1.0 / (1.0 + math.exp(-s * 2.0))) < 1e-15
    assert abs(w.sum() - 1.0) < 1e-15
    g = _rng(10)
    z = g.standard_normal(40).astype(np.float32) * 10
    w = O.inter_chunk_weights(z, 0.3)
    assert abs(w.sum() - 1.0) < 1e-12
    assert np.allclose(w, scipy.special.softmax(0.3 * z.astype(np.float64)), rtol=1e-12, atol=0)


# ---------------------------------------------------------------------------------------------
# Whole-row properties
# ---------------------------------------------------------------------------------------------

def pin_single_chunk_is_dense_causal():
    """With one chunk (L = C) the method reduces to dense causal attention of the raw query."""
    inp = _small_inputs(11, L=64, d=16, C=64)
    s = 1.0 / 4.0
    o, idx, w = O.prefill(inp, 64, 3, "fp32")
    for h in range(2):
        want = _dense_causal(inp["q"][0, h], inp["k"][0, h], inp["v"][0, h], s)
        assert np.allclose(o[0, h], want, rtol=0, atol=1e-12), np.abs(o[0, h] - want).max()
        assert np.all(idx[0, h, :, 0] == 0) and np.all(idx[0, h, :, 1:] == -1)
        assert np.all(w[0, h, :, 0] == 1.0)


def pin_all_chunks_two_level_softmax():
    """k >= number of causal chunks: o_i = sum_j softmax_j(s sigma) softmax_t(a) V, matrix form."""
    inp = _small_inputs(12, L=256, d=8, C=32, r=3, D=10)
    C, L, d = 32, 256, 8
    s = 1.0 / math.sqrt(d)
    o, idx, w = O.prefill(inp, C, 8, "fp32")
    for h in range(2):
        q = inp["q"][0, h].astype(np.float64)
        wu = inp["w_up"][h * d:(h + 1) * d].astype(np.float64)
        dq = ((inp["h"][0].astype(np.float64) @ inp["w_down"].astype(np.float64).T) @ wu.T).astype(np.float32)
        qt = (q + dq.astype(np.float64)).astype(np.float32).astype(np.float64)
        sig = (qt @ inp["lmk"][0, h].astype(np.float64).T).astype(np.float32).astype(np.float64)
        a = s * (q @ inp["k"][0, h].astype(np.float64).T)
        for i in range(L):
            c = i // C
            wj = scipy.special.softmax(s * sig[i, :c + 1])
            acc = np.zeros(d)
            for j in range(c + 1):
                hi = min((j + 1) * C, i + 1)
                p = scipy.special.softmax(a[i, j * C:hi])
                acc += wj[j] * (p @ inp["v"][0, h, j * C:hi].astype(np.float64))
            assert np.allclose(o[0, h, i], acc, rtol=0, atol=1e-6), (h, i)


def pin_exact_chunk_mass_identity():
    """Landmarks set to log of each chunk's exact attention mass, with every chunk kept, turn the
    two-level factorisation into dense causal attention (the block-sparse-by-exact-mass view)."""
    g = _rng(13)
    L, d, C = 320, 16, 64
    s = 0.25
    q = g.standard_normal((L, d)).astype(np.float32)
    k = g.standard_normal((L, d)).astype(np.float32)
    v = g.standard_normal((L, d)).astype(np.float32)
    dense = _dense_causal(q, k, v, s)
    for i in (0, 63, 64, 100, 191, 250, 319):
        c = i // C
        a = s * (k[: i + 1].astype(np.float64) @ q[i].astype(np.float64))
        lse = np.array([scipy.special.logsumexp(a[j * C:min((j + 1) * C, i + 1)]) for j in range(c + 1)])
        qq = q[i].astype(np.float64)
        lmk = np.zeros((L // C, d), dtype=np.float32)
        lmk[: c + 1] = (np.outer(lse / s, qq) / qq.dot(qq)).astype(np.float32)
        inp = dict(q=q[None, None], k=k[None, None], v=v[None, None], lmk=lmk[None, None])
        r = O.prefill_rows(inp, [(0, 0, i)], C, c + 1, "fp32", scale=s)[(0, 0, i)]
        assert np.allclose(r["o"], dense[i], rtol=0, atol=2e-5), (i, np.abs(r["o"] - dense[i]).max())


def pin_causality():
    """Row i ignores keys, values and landmarks after it."""
    inp = _small_inputs(14, L=256, C=64)
    rows = [(0, 0, 70), (0, 1, 130), (0, 1, 255)]
    base = O.prefill_rows(inp, rows, 64, 2, "fp32")
    for (b, h, i) in rows:
        pert = {key: val.copy() for key, val in inp.items()}
        pert["k"][:, :, i + 1:] += 5.0
        pert["v"][:, :, i + 1:] -= 3.0
        pert["lmk"][:, :, i // 64 + 1:] *= -7.0
        r = O.prefill_rows(pert, [(b, h, i)], 64, 2, "fp32")[(b, h, i)]
        assert np.array_equal(r["o"], base[(b, h, i)]["o"]) and np.array_equal(r["idx"], base[(b, h, i)]["idx"])


def pin_own_chunk_visible_and_not_forced():
    g = _rng(15)
    L, d, C = 192, 8, 64
    q = np.ones((1, 1, L, d), np.float32)
    k = g.standard_normal((1, 1, L, d)).astype(np.float32)
    v = g.standard_normal((1, 1, L, d)).astype(np.float32)
    lmk = np.stack([np.full(d, 1.0), np.full(d, 2.0), np.full(d, -5.0)]).astype(np.float32)[None, None]
    inp = dict(q=q, k=k, v=v, lmk=lmk)
    r = O.prefill_rows(inp, [(0, 0, 150)], C, 2, "fp32", scale=0.5)[(0, 0, 150)]
    assert list(r["idx"]) == [0, 1]                                  # own chunk 2 scored lowest, not forced
    r = O.prefill_rows(inp, [(0, 0, 130)], C, 3, "fp32", scale=0.5)[(0, 0, 130)]
    assert list(r["idx"]) == [0, 1, 2]
    # the own chunk sees keys 128..130 only: compare its share with a 3-key softmax
    a = 0.5 * (k[0, 0, 128:131].astype(np.float64) @ q[0, 0, 130].astype(np.float64))
    o2 = scipy.special.softmax(a) @ v[0, 0, 128:131].astype(np.float64)
    o0 = scipy.special.softmax(0.5 * (k[0, 0, :64].astype(np.float64) @ np.ones(d))) @ v[0, 0, :64]
    o1 = scipy.special.softmax(0.5 * (k[0, 0, 64:128].astype(np.float64) @ np.ones(d))) @ v[0, 0, 64:128]
    wj = scipy.special.softmax(0.5 * np.array([8.0, 16.0, -40.0]))
    assert np.allclose(r["o"], wj[0] * o0 + wj[1] * o1 + wj[2] * o2, rtol=0, atol=1e-12)


def pin_key_shift_invariance_and_value_linearity():
    inp = _small_inputs(16, L=256, C=64)
    rows = [(0, 0, 200), (0, 1, 90)]
    base = O.prefill_rows(inp, rows, 64, 2, "fp32")
    shifted = {key: val.copy() for key, val in inp.items()}
    u = _rng(17).standard_normal(16).astype(np.float32)
    shifted["k"][0, :, 64:128] += u            # one vector added to every key of chunk 1
    r = O.prefill_rows(shifted, rows, 64, 2, "fp32")
    for row in rows:   # fp32 rounding of k + u perturbs the keys by ~1e-7 relative
        assert np.allclose(r[row]["o"], base[row]["o"], rtol=0, atol=1e-5)
    assert any(1 in set(base[row]["idx"]) for row in rows)
    v2 = _rng(18).standard_normal(inp["v"].shape).astype(np.float32)
    r2 = O.prefill_rows(dict(inp, v=v2), rows, 64, 2, "fp32")
    r3 = O.prefill_rows(dict(inp, v=(2.0 * inp["v"] - 3.0 * v2).astype(np.float32)), rows, 64, 2, "fp32")
    for row in rows:
        assert np.allclose(r3[row]["o"], 2.0 * base[row]["o"] - 3.0 * r2[row]["o"], rtol=0, atol=1e-5)


def pin_decode_matches_prefill_row():
    inp = _small_inputs(19, L=256, C=64, dtype="bf16")
    rows = [(0, 0, 0), (0, 1, 63), (0, 0, 64), (0, 1, 200), (0, 0, 255)]
    pre = O.prefill_rows(inp, rows, 64, 2, "bf16")
    for (b, h, i) in rows:
        dec_in = dict(q=inp["q"][:, :, i], k_cache=inp["k"], v_cache=inp["v"], lmk=inp["lmk"],
                      kv_len=np.array([i + 1], np.int32), h=inp["h"][:, i], w_down=inp["w_down"], w_up=inp["w_up"])
        dec = O.decode(dec_in, 64, 2, "bf16", pairs=[(b, h)])[(b, h)]
        assert np.array_equal(dec["idx"], pre[(b, h, i)]["idx"])
        assert np.array_equal(dec["o"], pre[(b, h, i)]["o"])


def pin_hand_worked_example():
    """Two chunks of two tokens, d = 1, worked by hand (tests/golden/hand_two_chunks.json)."""
    with open(os.path.join(GOLDEN, "hand_two_chunks.json")) as f:
        ex = json.load(f)
    arr = lambda key: np.array(ex["inputs"][key], dtype=np.float32)
    inp = dict(q=arr("q"), k=arr("k"), v=arr("v"), lmk=arr("lmk"))
    e = math.e
    # row 3 (chunk 1): scores sigma = (2, 1).
    # k = 1: chunk 0 only; keys (0, ln 3) -> p = (1/4, 3/4); o = 4/4 + 3*8/4 = 7.
    r = O.prefill_rows(inp, [(0, 0, 3)], 2, 1, "fp32", scale=1.0)[(0, 0, 3)]
    assert list(r["idx"]) == [0] and abs(r["o"][0] - 7.0) < 1e-6
    # k = 2: w = (e/(e+1), 1/(e+1)); chunk 1 keys (0, 0) -> o_1 = (v2 + v3)/2 = 11.
    r = O.prefill_rows(inp, [(0, 0, 3)], 2, 2, "fp32", scale=1.0)[(0, 0, 3)]
    assert list(r["idx"]) == [0, 1]
    assert abs(r["o"][0] - (e / (e + 1) * 7.0 + 1 / (e + 1) * 11.0)) < 1e-6
    # row 2 (first key of chunk 1) with k = 2: own chunk sees only v2 = 10.
    r = O.prefill_rows(inp, [(0, 0, 2)], 2, 2, "fp32", scale=1.0)[(0, 0, 2)]
    assert abs(r["o"][0] - (e / (e + 1) * 7.0 + 1 / (e + 1) * 10.0)) < 1e-6
    # row 1 (chunk 0): only chunk 0 is a candidate; sees both keys -> 7 again.
    r = O.prefill_rows(inp, [(0, 0, 1)], 2, 2, "fp32", scale=1.0)[(0, 0, 1)]
    assert list(r["idx"]) == [0, -1] and abs(r["o"][0] - 7.0) < 1e-6 and r["w"][1] == 0.0
    # row 0: one visible key -> v0 = 4.
    r = O.prefill_rows(inp, [(0, 0, 0)], 2, 1, "fp32", scale=1.0)[(0, 0, 0)]
    assert abs(r["o"][0] - 4.0) < 1e-12


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
