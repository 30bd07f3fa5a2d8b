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


def pin_exact_chunk_mass_other_chunk_sizes():
    """The exact-chunk-mass identity at chunk sizes 32 and 128, with a partial last chunk (the
    sequence is not a multiple of the chunk): the factorisation with every chunk kept and each
    landmark score equal to its chunk's log attention mass is dense causal attention."""
    g = _rng(21)
    L, d = 300, 16
    s = 0.25
    q = g.standard_normal((L, d)).astype(np.float32)
    k = g.standard_normal((L, d)).astype(np.float32)
    v = g.standard_normal((L, d)).astype(np.float32)
    dense = _dense_causal(q, k, v, s)
    for C in (32, 128):
        N = -(-L // C)
        for i in (0, C - 1, C, 150, 255, 256, L - 1):
            c = i // C
            a = s * (k[: i + 1].astype(np.float64) @ q[i].astype(np.float64))
            lse = np.array([scipy.special.logsumexp(a[j * C:min((j + 1) * C, i + 1)]) for j in range(c + 1)])
            qq = q[i].astype(np.float64)
            lmk = np.zeros((N, d), dtype=np.float32)
            lmk[: c + 1] = (np.outer(lse / s, qq) / qq.dot(qq)).astype(np.float32)
            inp = dict(q=q[None, None], k=k[None, None], v=v[None, None], lmk=lmk[None, None])
            r = O.prefill_rows(inp, [(0, 0, i)], C, c + 1, "fp32", scale=s)[(0, 0, i)]
            assert np.allclose(r["o"], dense[i], rtol=0, atol=2e-5), (C, i, np.abs(r["o"] - dense[i]).max())


def pin_decode_matches_prefill_row_other_chunk_sizes():
    """decode(kv_len = i + 1) equals prefill row i at chunk sizes 32 and 128, the cache ending
    inside a chunk."""
    for C, L in ((32, 200), (128, 300)):
        inp = _small_inputs(22, L=L, C=C, dtype="bf16")
        N = -(-L // C)
        import torch
        lmk = (_rng(23).standard_normal((1, 2, N, 16)) * 0.5).astype(np.float32)
        inp["lmk"] = torch.from_numpy(lmk).to(torch.bfloat16).float().numpy()
        rows = [(0, 0, 0), (0, 1, C - 1), (0, 0, C), (0, 1, L // 2), (0, 0, L - 1)]
        pre = O.prefill_rows(inp, rows, C, 3, "bf16")
        for (b, h, i) in rows:
            dec_in = dict(q=inp["q"][:, :, i], k_cache=inp["k"], v_cache=inp["v"], lmk=inp["lmk"],
                          kv_len=np.array([i + 1], np.int32), h=inp["h"][:, i], w_down=inp["w_down"],
                          w_up=inp["w_up"])
            dec = O.decode(dec_in, C, 3, "bf16", pairs=[(b, h)])[(b, h)]
            assert np.array_equal(dec["idx"], pre[(b, h, i)]["idx"]), (C, i)
            assert np.array_equal(dec["o"], pre[(b, h, i)]["o"]), (C, i)


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


# ---------------------------------------------------------------------------------------------
# Fusion over a supplied selection (used where the GPU's selection differs within the tie band)
# ---------------------------------------------------------------------------------------------

def pin_given_selection_matches_own_rows():
    """Given the oracle's own selection and its scores, the fusion reproduces the oracle's row
    output exactly, padded rows (fewer candidates than k) included."""
    inp = _small_inputs(20, L=320, d=16, C=64)
    rows = [(0, 0, 5), (0, 1, 64), (0, 0, 130), (0, 1, 200), (0, 0, 319)]
    res = O.prefill_rows(inp, rows, 64, 3, "fp32")
    for (b, h, i) in rows:
        r = res[(b, h, i)]
        sig = np.array([r["sigma"][j] if j >= 0 else 0.0 for j in r["idx"]], dtype=np.float32)
        got = O.attend_given_selection(inp["q"][b, h, i], inp["k"][b, h], inp["v"][b, h], r["idx"], sig, i, 64,
                                       1.0 / 4.0)
        assert np.array_equal(got, r["o"]), (i, np.abs(got - r["o"]).max())


def pin_given_selection_matrix_form():
    """Arbitrary (non-top-k) selections, padded with -1: the fusion equals the two-level sum
    written in matrix form, sum_j softmax(s sigma_G)_j * softmax(a over chunk j's visible keys) V."""
    g = _rng(21)
    L, d, C = 384, 8, 64
    s = 0.3
    q, k, v = (g.standard_normal((L, d)) for _ in range(3))
    a_all = s * (q @ k.T)
    for i, sel, nsel in ((383, [0, 2, 5], 3), (200, [1, 3, -1, -1], 2), (70, [1, -1], 1), (300, [4, 0, 2], 3)):
        sel = np.array(sel)
        valid = sel[sel >= 0]
        sig = np.zeros(len(sel), np.float32)
        sig[:nsel] = g.standard_normal(nsel).astype(np.float32) * 3
        wts = scipy.special.softmax(s * sig[:nsel].astype(np.float64))
        want = np.zeros(d)
        for wj, j in zip(wts, valid):
            hi = min((j + 1) * C, i + 1)
            want += wj * (scipy.special.softmax(a_all[i, j * C:hi]) @ v[j * C:hi])
        got = O.attend_given_selection(q[i], k, v, sel, sig, i, C, s)
        assert np.allclose(got, want, rtol=0, atol=1e-12), (i, sel, np.abs(got - want).max())


# ---------------------------------------------------------------------------------------------
# Dense (full) attention baseline
# ---------------------------------------------------------------------------------------------

def pin_dense_equals_one_chunk_hils():
    """With one chunk (L = C) HiLS is dense causal attention, through its own code path."""
    inp = _small_inputs(22, L=64, d=16, C=64, r=0)
    rows = [(0, h, i) for h in range(2) for i in (0, 1, 17, 40, 63)]
    dense = O.dense_causal_rows(inp, rows)
    hils = O.prefill_rows(inp, rows, 64, 1, "fp32")
    for row in rows:
        assert np.allclose(dense[row], hils[row]["o"], rtol=0, atol=1e-12), row


def pin_dense_exact_chunk_mass_hils():
    """HiLS over every chunk with each landmark set to its chunk's exact log attention mass equals
    dense causal attention (several chunks, the own chunk truncated)."""
    g = _rng(23)
    L, d, C, s = 320, 16, 64, 0.25
    q, k, v = (g.standard_normal((L, d)).astype(np.float32) for _ in range(3))
    inp = dict(q=q[None, None], k=k[None, None], v=v[None, None])
    for i in (0, 70, 191, 250, 319):
        c = i // C
        a = s * (k[: i + 1].astype(np.float64) @ q[i].astype(np.float64))
        lse = np.array([scipy.special.logsumexp(a[j * C:min((j + 1) * C, i + 1)]) for j in range(c + 1)])
        qq = q[i].astype(np.float64)
        lmk = np.zeros((L // C, d), dtype=np.float32)
        lmk[: c + 1] = (np.outer(lse / s, qq) / qq.dot(qq)).astype(np.float32)
        r = O.prefill_rows(dict(inp, lmk=lmk[None, None]), [(0, 0, i)], C, c + 1, "fp32", scale=s)[(0, 0, i)]
        want = O.dense_causal_rows(inp, [(0, 0, i)], scale=s)[(0, 0, i)]
        assert np.allclose(r["o"], want, rtol=0, atol=2e-5), (i, np.abs(r["o"] - want).max())


def pin_dense_equal_keys_mean():
    """All keys equal: the weights are uniform and row i returns the mean of v_0..v_i."""
    g = _rng(24)
    L, d = 200, 8
    k = np.tile(g.standard_normal(d), (L, 1))
    inp = dict(q=g.standard_normal((1, 1, L, d)), k=k[None, None], v=g.standard_normal((1, 1, L, d)))
    res = O.dense_causal_rows(inp, [(0, 0, i) for i in (0, 1, 99, 199)], scale=0.7)
    for (_, _, i), o in res.items():
        assert np.allclose(o, inp["v"][0, 0, : i + 1].mean(axis=0), rtol=0, atol=1e-12), i


def pin_dense_scale_sharpens_to_argmax():
    """A large scale sends all weight to the best visible key (one-hot limit)."""
    g = _rng(25)
    L, d = 96, 8
    q, k, v = (g.standard_normal((L, d)) for _ in range(3))
    inp = dict(q=q[None, None], k=k[None, None], v=v[None, None])
    for i in (5, 50, 95):
        best = int(np.argmax(k[: i + 1] @ q[i]))
        o = O.dense_causal_rows(inp, [(0, 0, i)], scale=1e4)[(0, 0, i)]
        assert np.allclose(o, v[best], rtol=0, atol=1e-9), i


def pin_dense_decode_matches_prefill_row():
    inp = _small_inputs(26, L=256, C=64, r=0)
    for (h, i) in ((0, 0), (1, 63), (0, 64), (1, 200), (0, 255)):
        dec_in = dict(q=inp["q"][:, :, i], k_cache=inp["k"], v_cache=inp["v"], kv_len=np.array([i + 1], np.int32))
        dec = O.dense_decode(dec_in, pairs=[(0, h)])[(0, h)]
        pre = O.dense_causal_rows(inp, [(0, h, i)])[(0, h, i)]
        assert np.array_equal(dec, pre), (h, i)
        hils = O.prefill_rows(inp, [(0, h, i)], 64, 4, "fp32")[(0, h, i)]
        assert (i >= 64) == (not np.allclose(dec, hils["o"], atol=1e-9)), (h, i)


# ---------------------------------------------------------------------------------------------
# Backward pass
# ---------------------------------------------------------------------------------------------

def _bwd_case(seed, B=1, H=2, L=16, d=4, C=4, r=2, D=6):
    g = _rng(seed)
    inp = dict(q=g.standard_normal((B, H, L, d)), k=g.standard_normal((B, H, L, d)),
               v=g.standard_normal((B, H, L, d)), lmk=g.standard_normal((B, H, L // C, d)))
    if r:
        inp.update(h=g.standard_normal((B, L, D)), w_down=0.5 * g.standard_normal((r, D)),
                   w_up=0.5 * g.standard_normal((H * d, r)))
    return inp, g.standard_normal((B, H, L, d))


def _loss(inp, dout, C, k, scale):
    o, idx, _ = O.prefill(inp, C, k, "fp64", scale=scale)
    return float(np.sum(o * dout)), idx


def pin_backward_finite_differences():
    """Every gradient entry against central differences of sum(dout * o) of the float64 forward
    (the selection stays the same under the perturbations, checked)."""
    C, k, s, eps = 4, 2, 0.6, 1e-5
    inp, dout = _bwd_case(27)
    grads = O.prefill_backward(inp, dout, C, k, "fp64", scale=s)
    _, idx0 = _loss(inp, dout, C, k, s)
    names = dict(q="dq", k="dk", v="dv", lmk="dlmk", h="dh", w_down="dw_down", w_up="dw_up")
    for name, gname in names.items():
        x = inp[name]
        num = np.zeros(x.shape)
        for pos in np.ndindex(*x.shape):
            old = x[pos]
            x[pos] = old + eps
            lp, ip = _loss(inp, dout, C, k, s)
            x[pos] = old - eps
            lm, im = _loss(inp, dout, C, k, s)
            x[pos] = old
            assert np.array_equal(ip, idx0) and np.array_equal(im, idx0), (name, pos)
            num[pos] = (lp - lm) / (2 * eps)
        scale_ = max(1.0, float(np.abs(num).max()))
        assert np.allclose(grads[gname], num, rtol=0, atol=1e-7 * scale_), \
            (name, float(np.abs(grads[gname] - num).max()))


def pin_backward_single_chunk_is_dense_gradient():
    """One chunk, k = 1, no Q-Cal: HiLS is dense causal attention, whose gradients have the
    textbook matrix form dV = P^T dO, dS = P * (dO V^T - rowsum(P * dO V^T)), dQ = s dS K,
    dK = s dS^T Q; the single inter-chunk weight is 1, so the landmark gets no gradient."""
    g = _rng(28)
    L, d, s = 64, 8, 0.4
    q, k, v, dout = (g.standard_normal((L, d)) for _ in range(4))
    inp = dict(q=q[None, None], k=k[None, None], v=v[None, None], lmk=g.standard_normal((1, 1, 1, d)))
    grads = O.prefill_backward(inp, dout[None, None], 64, 1, "fp64", scale=s)
    a = s * q @ k.T
    a[np.triu_indices(L, 1)] = -np.inf
    P = scipy.special.softmax(a, axis=1)
    dP = dout @ v.T
    dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
    assert np.allclose(grads["dv"][0, 0], P.T @ dout, rtol=0, atol=1e-12)
    assert np.allclose(grads["dq"][0, 0], s * dS @ k, rtol=0, atol=1e-12)
    assert np.allclose(grads["dk"][0, 0], s * dS.T @ q, rtol=0, atol=1e-12)
    assert np.all(grads["dlmk"] == 0.0)


def pin_backward_shift_invariances():
    """Adding one vector to every landmark shifts all of a row's scores equally (the weights do
    not change): the landmark gradients sum to zero.  Adding one vector to every key of a chunk
    shifts that chunk's visible scores equally: each chunk's key gradients sum to zero."""
    C, k = 4, 3
    inp, dout = _bwd_case(29, L=20, r=2)
    grads = O.prefill_backward(inp, dout, C, k, "fp64", scale=0.5)
    assert np.allclose(grads["dlmk"].sum(axis=2), 0.0, rtol=0, atol=1e-12)
    dk = grads["dk"].reshape(1, 2, 20 // C, C, -1).sum(axis=3)
    assert np.allclose(dk, 0.0, rtol=0, atol=1e-12)
    assert np.abs(grads["dlmk"]).max() > 1e-3 and np.abs(grads["dk"]).max() > 1e-3


# ---------------------------------------------------------------------------------------------
# Forced local chunk (a serving variant)
# ---------------------------------------------------------------------------------------------

def pin_forced_local_bruteforce():
    """The selection holds the own (last) chunk and the unique (k-1)-subset of the others that
    beats every other earlier chunk (ties to the smaller index), by enumeration."""
    g = _rng(30)
    for trial in range(300):
        n = int(g.integers(1, 8))
        k = int(g.integers(1, 9))
        s = g.integers(-3, 4, n).astype(np.float32)
        got = O.select_with_local(s, k)
        keff = min(k, n)
        m = keff - 1
        winners = [set(S) for S in itertools.combinations(range(n - 1), m)
                   if all(_dominates(s, x, y) for x in S for y in range(n - 1) if y not in S)]
        assert len(winners) == 1
        want = sorted(winners[0] | {n - 1})
        assert list(got[:keff]) == want and all(got[keff:] == -1), (s, k, got)


def pin_forced_local_rows():
    """Whole rows: with the own chunk scoring highest, forcing changes nothing; with it scoring
    lowest, the row keeps it and drops its k-th best earlier chunk, and the weights are the
    softmax over the forced set."""
    g = _rng(31)
    L, d, C, s = 256, 8, 64, 0.5
    q = np.ones((1, 1, L, d), np.float32)
    k = g.standard_normal((1, 1, L, d)).astype(np.float32)
    v = g.standard_normal((1, 1, L, d)).astype(np.float32)
    lmk = np.stack([np.full(d, 2.0), np.full(d, 1.0), np.full(d, 3.0), np.full(d, -4.0)]).astype(np.float32)
    inp = dict(q=q, k=k, v=v, lmk=lmk[None, None])
    a = O.prefill_rows(inp, [(0, 0, 150)], C, 2, "fp32", scale=s)[(0, 0, 150)]          # own chunk 2 best
    b = O.prefill_rows(inp, [(0, 0, 150)], C, 2, "fp32", scale=s, force_local=True)[(0, 0, 150)]
    assert list(a["idx"]) == [0, 2] and list(b["idx"]) == [0, 2] and np.array_equal(a["o"], b["o"])
    c = O.prefill_rows(inp, [(0, 0, 200)], C, 2, "fp32", scale=s)[(0, 0, 200)]          # own chunk 3 worst
    f = O.prefill_rows(inp, [(0, 0, 200)], C, 2, "fp32", scale=s, force_local=True)[(0, 0, 200)]
    assert list(c["idx"]) == [0, 2] and list(f["idx"]) == [2, 3]
    sig = np.array([3.0 * d, -4.0 * d])
    assert np.allclose(f["w"], scipy.special.softmax(s * sig), rtol=0, atol=1e-12)
    dec = O.decode(dict(q=q[:, :, 200], k_cache=k, v_cache=v, lmk=lmk[None, None], kv_len=np.array([201])),
                   C, 2, "fp32", scale=s, force_local=True)[(0, 0)]
    assert np.array_equal(dec["idx"], f["idx"]) and np.array_equal(dec["o"], f["o"])


# HoPE ([P3] "Engineering details", hierarchical positional encoding item; H1-H3)

def pin_hope_complex_rotation():
    """With base 16 and d = 8 the pair frequencies are 1, 1/2, 1/4, 1/8 exactly; with a window
    that holds every wavelength, pair i of a row at position p is the complex number x + iy
    multiplied by exp(i p theta_i) (cmath, not the oracle's cos/sin)."""
    import cmath
    g = _rng(41)
    x = g.standard_normal((3, 5, 8))
    pos = np.array([0, 1, 7, 1000, 65535])
    got = O.hope_rotate(x, pos, 16.0, 10 ** 6)
    for r in range(5):
        for i, theta in enumerate((1.0, 0.5, 0.25, 0.125)):
            for b in range(3):
                z = complex(x[b, r, 2 * i], x[b, r, 2 * i + 1]) * cmath.exp(1j * pos[r] * theta)
                assert abs(got[b, r, 2 * i] - z.real) < 1e-9 and abs(got[b, r, 2 * i + 1] - z.imag) < 1e-9, (r, i)


def pin_hope_relative_position():
    """For the rotated pairs the product of a rotated query and key depends only on the key's
    offset from the query; the unrotated pairs contribute the plain product."""
    g = _rng(42)
    d = 64
    q, k = g.standard_normal(d), g.standard_normal(d)
    base, win = 10000.0, 512
    rot = O.hope_rotated_pairs(d, base, win)
    assert 0 < len(rot) < d // 2
    ref = None
    for m in (0, 5, 77, 4096):
        qm = O.hope_rotate(q[None], [m], base, win)[0]
        kn = O.hope_rotate(k[None], [m + 9], base, win)[0]
        v = float(qm @ kn)
        ref = v if ref is None else ref
        assert abs(v - ref) < 1e-9 * max(1.0, abs(ref)), (m, v, ref)
    # dimensions left alone
    keep = np.ones(d, dtype=bool)
    for i in rot:
        keep[2 * i:2 * i + 2] = False
    qr = O.hope_rotate(q[None], [123], base, win)[0]
    assert np.array_equal(qr[keep], q[keep])


def pin_hope_window_split():
    """Base 16, d = 8: wavelengths 2 pi, 4 pi, 8 pi and 16 pi tokens.  A 13-token window rotates
    pairs 0 and 1 only, a 6-token window none (identity), a 51-token window all four; position 0
    is the identity; every pair keeps its length."""
    g = _rng(43)
    x = g.standard_normal((4, 8))
    pos = [1, 2, 3, 9]
    assert list(O.hope_rotated_pairs(8, 16.0, 13)) == [0, 1]
    assert list(O.hope_rotated_pairs(8, 16.0, 6)) == []
    assert list(O.hope_rotated_pairs(8, 16.0, 51)) == [0, 1, 2, 3]
    y = O.hope_rotate(x, pos, 16.0, 13)
    assert np.array_equal(y[:, 4:], x[:, 4:]) and not np.allclose(y[:, :4], x[:, :4])
    assert np.array_equal(O.hope_rotate(x, pos, 16.0, 6), x)
    assert np.allclose(O.hope_rotate(x, [0, 0, 0, 0], 16.0, 51), x, atol=0, rtol=0)
    z = O.hope_rotate(x, pos, 16.0, 51)
    for i in range(4):
        assert np.allclose(np.hypot(z[:, 2 * i], z[:, 2 * i + 1]), np.hypot(x[:, 2 * i], x[:, 2 * i + 1]), atol=1e-12)


def pin_partial_landmark_arithmetic_keys():
    """Keys in arithmetic progression (row t holds c + t u, small integers, exact in fp32): the
    landmark of the chunk holding the newest key is c + u (first + last) / 2 over that chunk's
    rows so far; one key gives the key itself, a full chunk its own mean, and kv_len is clamped."""
    B, Hk, Lmax, d = 6, 2, 300, 4
    u = np.array([1.0, -2.0, 0.5, 4.0])
    c = np.array([3.0, 0.0, -1.0, 2.0])
    t = np.arange(Lmax, dtype=np.float64)[:, None]
    k = np.broadcast_to((c + t * u)[None, None], (B, Hk, Lmax, d)).astype(np.float32).copy()
    k[:, 1] *= -1.0                                    # the second key/value head differs
    for C in (32, 64, 128):
        kv_len = np.array([1, C, C + 1, 2 * C + 7, Lmax, Lmax + 50], np.int32)
        res = O.partial_landmark(k, kv_len, C, "fp32")
        for b in range(B):
            n_keys = min(int(kv_len[b]), Lmax)
            j = (n_keys - 1) // C
            first, last = j * C, n_keys - 1
            for g in range(Hk):
                want = (c + u * (first + last) / 2.0) * (1.0 if g == 0 else -1.0)
                got_j, got = res[(b, g)]
                assert got_j == j, (C, b, got_j, j)
                assert np.array_equal(got, want.astype(np.float32)), (C, b, g, got, want)


def pin_partial_landmark_only_its_rows():
    """The landmark depends on rows jC .. kv_len-1 only, not on their order, and equal keys give
    that key exactly (bf16)."""
    g = _rng(31)
    B, Hk, Lmax, d, C = 3, 2, 200, 8, 64
    k = g.standard_normal((B, Hk, Lmax, d)).astype(np.float32)
    kv_len = np.array([70, 128, 200], np.int32)
    base = O.partial_landmark(k, kv_len, C, "fp32")
    pert = k.copy()
    for b in range(B):
        j = (int(kv_len[b]) - 1) // C
        pert[b, :, : j * C] += 3.0                     # earlier chunks
        pert[b, :, int(kv_len[b]):] -= 5.0             # rows past the newest key
        rows = np.arange(j * C, int(kv_len[b]))
        pert[b, :, rows] = k[b, :, rows[::-1]]        # the chunk's rows reversed
    got = O.partial_landmark(pert, kv_len, C, "fp32")
    for key in base:
        assert got[key][0] == base[key][0]
        assert np.allclose(got[key][1], base[key][1], rtol=0, atol=1e-6), key
    same = np.broadcast_to(np.array([1.5, -0.25, 3.0, 0.0078125, -7.0, 2.0, 0.5, 1.0], np.float32),
                           (B, Hk, Lmax, d)).copy()
    for (b, gh), (j, lm) in O.partial_landmark(same, kv_len, C, "bf16").items():
        assert np.array_equal(lm, same[0, 0, 0]), (b, gh)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
