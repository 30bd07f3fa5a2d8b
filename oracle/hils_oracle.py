"""HiLS attention forward pass: CPU oracle.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constants) and imports only
NumPy.

It is written for a reader to check against the pages by eye: one query row at
a time, in the order the method states its steps, float64 arithmetic.

What the method computes (sources are the pages' titles and sections):

  [P1] "HiLS-Attention" model page, "Model Description": block-sparse attention
       that ranks chunks by their exact attention mass would need the full QK
       product; HiLS instead scores compressed per-chunk keys to get a surrogate
       of that mass, selects the top-k chunks, and factorises attention into an
       inter-chunk softmax and an intra-chunk softmax.
  [P2] "HiLS Attention Extrapolates 64x at 90% Retrieval Accuracy": each query
       attends to every retrieved chunk independently and the per-chunk outputs
       are combined with the chunks' retrieval scores.
  [P3] "HiLS Attention: Tencent ... Sparse Attention" explainer,
       "Core idea: landmark tokens and hierarchical factorisation": one landmark
       token per chunk; level 1 is the query's attention over the landmarks
       (a distribution over chunks), level 2 is ordinary attention over the
       tokens inside the selected chunks.
       "Engineering details", Q-Cal item: a low-rank offset
       delta_q = W_up W_down h, with h the token's hidden state, adapts the
       query for chunk-level mass estimation.

Readings taken where the pages are silent:
  R1 one scale s (default 1/sqrt(d)) serves both softmax levels;
  R2 candidates of query i are the causal chunks j <= floor(i/C), its own chunk
     included and scored like the others (not forced in);
  R3 ties in the landmark score go to the smaller chunk index;
  R4 with fewer than k candidates every candidate is selected; idx is padded
     with -1 and w with 0; idx is listed in ascending chunk order;
  R5 W_down is [r, D], shared by the heads; W_up is [H*d, r]; rows
     h*d..h*d+d-1 of W_up give head h's offset;
  R6 the calibrated query q~ is used for chunk scoring only; the intra-chunk
     attention uses the raw q;
  R7 rounding points: delta_q and q + delta_q are formed and rounded to fp32,
     then q~ is rounded once to the run dtype (round-to-nearest-even to bf16 for
     bf16 runs); the landmark score sigma is rounded to fp32 before ranking and
     before the inter-chunk softmax (the kernel's precision decides the integer
     outcome, as both sides must take it in the same precision); everything else
     is float64 here;
  R8 the landmark token is not a key of the intra-chunk attention; the query's
     own chunk is causally truncated at the query;
  R9 decode: the new token's key/value are already in the cache; the query sits
     at position kv_len-1 and a partial last chunk is allowed.

HoPE ([P3] "Engineering details", hierarchical positional encoding item: rotary position
encoding on the dimensions inside the pre-training window, no position encoding beyond it):
  H1 the rotary encoding rotates dimension pairs (2i, 2i+1) by the angle pos * theta_i with
     theta_i = base^(-2i/d) (its original, interleaved form);
  H2 a pair is inside the pre-training window when its wavelength 2 pi / theta_i is at most the
     window's length in tokens; the other pairs are left as they are;
  H3 the caller applies it to q and k before the attention (prefill rows at positions pos0 + i,
     a decode query at kv_len - 1); landmarks and the Q-Cal offset see no position.

Landmark of the chunk still being filled during decode ([P3] "Core idea": a landmark token is
appended at the end of each chunk, so a chunk that has not reached C tokens has none yet):
  P1 its stand-in is the mean of the chunk's keys so far, rows jC .. kv_len-1 of the cache with
     j = floor((kv_len - 1) / C), rounded once to the run dtype; it is recomputed from the cache
     at every step (no running state), and the caller replaces it with the model's landmark once
     the chunk is complete.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional, Sequence

import numpy as np

__all__ = [
    "round_to_bf16", "round_to_run_dtype", "qcal_offset", "calibrated_query", "landmark_scores",
    "select_top_k", "select_with_local", "inter_chunk_weights", "intra_chunk_attention", "fuse", "prefill_rows",
    "prefill", "decode", "attend_given_selection", "dense_attention_row", "dense_causal_rows",
    "dense_decode", "chunk_backward", "inter_chunk_backward", "prefill_backward",
    "hope_rotated_pairs", "hope_rotate", "partial_landmark",
]


# ------------------------------------------------------------------------------------------
# Rounding (R7)
# ------------------------------------------------------------------------------------------

def round_to_bf16(x) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even); returns fp32 holding the result.

    bfloat16 keeps the top 16 bits of an fp32 word.  Round-to-nearest-even adds
    0x7FFF plus the lowest kept bit to the word and truncates.  Finite inputs only."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def round_to_run_dtype(x, dtype: str) -> np.ndarray:
    if dtype == "fp64":       # no rounding at all: the gradient checks' finite differences
        return np.asarray(x, dtype=np.float64)
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "fp32":
        return x32
    if dtype == "bf16":
        return round_to_bf16(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


# ------------------------------------------------------------------------------------------
# Step 1: Q-Cal ([P3] Engineering details, Q-Cal)
# ------------------------------------------------------------------------------------------

def qcal_offset(h_row: np.ndarray, w_down: np.ndarray, w_up_head: np.ndarray) -> np.ndarray:
    """delta_q = W_up[head rows] . (W_down . h), float64.  h_row [D], w_down [r,D], w_up_head [d,r]."""
    t = np.zeros(w_down.shape[0], dtype=np.float64)
    for a in range(w_down.shape[0]):
        t[a] = np.dot(w_down[a].astype(np.float64), h_row.astype(np.float64))
    dq = np.zeros(w_up_head.shape[0], dtype=np.float64)
    for e in range(w_up_head.shape[0]):
        dq[e] = np.dot(w_up_head[e].astype(np.float64), t)
    return dq


def calibrated_query(q_row: np.ndarray, h_row: Optional[np.ndarray], w_down: Optional[np.ndarray],
                     w_up_head: Optional[np.ndarray], dtype: str) -> np.ndarray:
    """q~ = round_dtype(fp32(q + fp32(delta_q)))  (R7).  Without Q-Cal (r = 0) q~ = q.
    dtype "fp64" keeps everything in float64."""
    if dtype == "fp64":
        q64 = np.asarray(q_row, dtype=np.float64)
        if w_down is None or w_down.shape[0] == 0:
            return q64
        return q64 + qcal_offset(h_row, w_down, w_up_head)
    q32 = np.asarray(q_row, dtype=np.float32)
    if w_down is None or w_down.shape[0] == 0:
        return round_to_run_dtype(q32, dtype)
    dq32 = qcal_offset(h_row, w_down, w_up_head).astype(np.float32)
    s32 = (q32.astype(np.float64) + dq32.astype(np.float64)).astype(np.float32)
    return round_to_run_dtype(s32, dtype)


# ------------------------------------------------------------------------------------------
# Step 2: inter-chunk scores over the landmarks ([P1] Model Description; [P3] Core idea, level 1)
# ------------------------------------------------------------------------------------------

def landmark_scores(q_tilde: np.ndarray, lmk_rows: np.ndarray) -> np.ndarray:
    """sigma_j = q~ . lmk_j for every given landmark row, float64 dot rounded to fp32 (R7); a
    float64 q~ (dtype "fp64") keeps float64 scores."""
    qt = np.asarray(q_tilde, dtype=np.float64)
    exact = np.asarray(q_tilde).dtype == np.float64
    out = np.empty(lmk_rows.shape[0], dtype=np.float64 if exact else np.float32)
    for j in range(lmk_rows.shape[0]):
        out[j] = np.dot(lmk_rows[j].astype(np.float64), qt)
    return out


# ------------------------------------------------------------------------------------------
# Step 3: top-k chunk selection ([P1] "selects top-k chunks"; R2-R4)
# ------------------------------------------------------------------------------------------

def select_top_k(sigma: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores (ties -> smaller index), ascending, padded with -1 to k.

    Repeatedly takes the best remaining candidate; np.argmax returns the first
    (smallest) index among equal maxima, which is the tie rule R3."""
    s = np.asarray(sigma).astype(np.float64)
    n = s.shape[0]
    taken = np.zeros(n, dtype=bool)
    chosen = []
    for _ in range(min(k, n)):
        masked = np.where(taken, -np.inf, s)
        j = int(np.argmax(masked))
        if taken[j]:          # only -inf left (cannot happen for finite scores)
            break
        taken[j] = True
        chosen.append(j)
    out = np.full(k, -1, dtype=np.int64)
    out[: len(chosen)] = sorted(chosen)
    return out


def select_with_local(sigma: np.ndarray, k: int) -> np.ndarray:
    """Variant with the query's own chunk forced in (a serving option; the pages do not force it,
    reading R2): the last candidate (the own chunk) is always selected, the other k - 1 slots are
    the top k - 1 of the earlier candidates (ties -> smaller index).  Ascending, -1 padded."""
    s = np.asarray(sigma)
    own = s.shape[0] - 1
    others = select_top_k(s[:own], k - 1) if k > 1 else np.zeros(0, dtype=np.int64)
    chosen = sorted([int(j) for j in others if j >= 0] + [own])
    out = np.full(k, -1, dtype=np.int64)
    out[: len(chosen)] = chosen
    return out


# ------------------------------------------------------------------------------------------
# Step 4: inter-chunk softmax over the selection ([P1] factorised inter-chunk softmax)
# ------------------------------------------------------------------------------------------

def inter_chunk_weights(sigma_selected: np.ndarray, scale: float) -> np.ndarray:
    """w_j = exp(s*sigma_j - max) / sum over the selection; float64."""
    z = scale * np.asarray(sigma_selected, dtype=np.float64)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


# ------------------------------------------------------------------------------------------
# Step 5: intra-chunk attention ([P3] Core idea, level 2; [P2] each chunk attended independently)
# ------------------------------------------------------------------------------------------

def intra_chunk_attention(q_row: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one (raw) query over one chunk's visible keys/values; float64 [d]."""
    q = np.asarray(q_row, dtype=np.float64)
    a = np.array([scale * np.dot(keys[t].astype(np.float64), q) for t in range(keys.shape[0])])
    a = a - a.max()
    p = np.exp(a)
    p = p / p.sum()
    o = np.zeros(values.shape[1], dtype=np.float64)
    for t in range(values.shape[0]):
        o += p[t] * values[t].astype(np.float64)
    return o


# ------------------------------------------------------------------------------------------
# Step 6: fusion by the chunk weights ([P2] outputs fused by retrieval scores)
# ------------------------------------------------------------------------------------------

def fuse(weights: Sequence[float], chunk_outputs: Sequence[np.ndarray]) -> np.ndarray:
    o = np.zeros_like(np.asarray(chunk_outputs[0], dtype=np.float64))
    for w, oj in zip(weights, chunk_outputs):
        o += w * np.asarray(oj, dtype=np.float64)
    return o


# ------------------------------------------------------------------------------------------
# One query row end to end
# ------------------------------------------------------------------------------------------

def _visible_range(j: int, chunk: int, i: int):
    """Keys of chunk j visible to query position i (R8): [jC, min(jC+C-1, i)]."""
    lo = j * chunk
    hi = min(lo + chunk, i + 1)
    return lo, hi


def attend_row(q_row, keys, values, idx, w, i, chunk, scale) -> np.ndarray:
    """Steps 5-6 for one row, given its selection idx (ascending, -1 padded) and weights w."""
    outs, ws = [], []
    for j, wj in zip(idx, w):
        if j < 0:
            continue
        lo, hi = _visible_range(int(j), chunk, i)
        outs.append(intra_chunk_attention(q_row, keys[lo:hi], values[lo:hi], scale))
        ws.append(wj)
    return fuse(ws, outs)


def hils_row(q_row, q_tilde, keys, values, lmk, i, chunk, topk, scale, force_local=False):
    """All steps for query position i.  keys/values [>= i+1, d], lmk [>= i//C + 1, d].
    force_local: the own chunk is always selected (select_with_local).

    Returns (o [d] float64, idx [k] int64, w [k] float64, sigma [c+1] fp32)."""
    c = i // chunk
    sigma = landmark_scores(q_tilde, lmk[: c + 1])
    idx = select_with_local(sigma, topk) if force_local else select_top_k(sigma, topk)
    sel = idx[idx >= 0]
    w = np.zeros(topk, dtype=np.float64)
    w[: len(sel)] = inter_chunk_weights(sigma[sel], scale)
    o = attend_row(q_row, keys, values, idx, w, i, chunk, scale)
    return o, idx, w, sigma


# ------------------------------------------------------------------------------------------
# Batched drivers (loops over batch, head and the requested rows)
# ------------------------------------------------------------------------------------------

def _w_up_head(w_up, head, d):
    return None if w_up is None else w_up[head * d:(head + 1) * d]


def prefill_rows(inp: Dict[str, np.ndarray], rows: Iterable[tuple], chunk: int, topk: int,
                 dtype: str, scale: Optional[float] = None, force_local: bool = False) -> Dict[tuple, dict]:
    """Prefill for selected (b, h, i) rows.  inp holds q,k,v [B,H,L,d], lmk [B,H,N,d] and,
    with Q-Cal, h [B,L,D], w_down [r,D], w_up [H*d,r] (fp32 arrays holding dtype-exact values).

    Returns {(b,h,i): dict(o, idx, w, sigma, q_tilde)}."""
    q, k, v, lmk = inp["q"], inp["k"], inp["v"], inp["lmk"]
    d = q.shape[-1]
    s = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    w_down = inp.get("w_down")
    if w_down is not None and w_down.shape[0] == 0:
        w_down = None
    out = {}
    for (b, h, i) in rows:
        hid = None if w_down is None else inp["h"][b, i]
        qt = calibrated_query(q[b, h, i], hid, w_down, _w_up_head(inp.get("w_up"), h, d), dtype)
        extra = {"force_local": True} if force_local else {}
        o, idx, w, sigma = hils_row(q[b, h, i], qt, k[b, h], v[b, h], lmk[b, h], i, chunk, topk, s, **extra)
        out[(b, h, i)] = dict(o=o, idx=idx, w=w, sigma=sigma, q_tilde=qt)
    return out


def prefill(inp: Dict[str, np.ndarray], chunk: int, topk: int, dtype: str,
            scale: Optional[float] = None):
    """Full prefill: returns o [B,H,L,d] float64, idx [B,H,L,k] int64, w [B,H,L,k] float64."""
    B, H, L, d = inp["q"].shape
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(L)]
    res = prefill_rows(inp, rows, chunk, topk, dtype, scale)
    o = np.zeros((B, H, L, d))
    idx = np.zeros((B, H, L, topk), dtype=np.int64)
    w = np.zeros((B, H, L, topk))
    for (b, h, i), r in res.items():
        o[b, h, i], idx[b, h, i], w[b, h, i] = r["o"], r["idx"], r["w"]
    return o, idx, w


def decode(inp: Dict[str, np.ndarray], chunk: int, topk: int, dtype: str,
           scale: Optional[float] = None, pairs: Optional[Iterable[tuple]] = None,
           force_local: bool = False) -> Dict[tuple, dict]:
    """Decode step (R9): q [B,H,d] at position kv_len[b]-1 over k_cache/v_cache [B,H,Lmax,d],
    lmk [B,H,ceil(Lmax/C),d], h [B,D].  Returns {(b,h): dict(o, idx, w, sigma, q_tilde)}."""
    q, kc, vc, lmk, kv_len = inp["q"], inp["k_cache"], inp["v_cache"], inp["lmk"], inp["kv_len"]
    B, H, d = q.shape
    s = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    w_down = inp.get("w_down")
    if w_down is not None and w_down.shape[0] == 0:
        w_down = None
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    out = {}
    for (b, h) in pairs:
        i = int(kv_len[b]) - 1
        hid = None if w_down is None else inp["h"][b]
        qt = calibrated_query(q[b, h], hid, w_down, _w_up_head(inp.get("w_up"), h, d), dtype)
        extra = {"force_local": True} if force_local else {}
        o, idx, w, sigma = hils_row(q[b, h], qt, kc[b, h], vc[b, h], lmk[b, h], i, chunk, topk, s, **extra)
        out[(b, h)] = dict(o=o, idx=idx, w=w, sigma=sigma, q_tilde=qt)
    return out


def attend_given_selection(q_row, keys, values, idx, sigma_selected, i, chunk, scale) -> np.ndarray:
    """Steps 4-6 on a supplied selection: idx (ascending, -1 padded) and the fp32 scores of the
    selected entries in the same order.  Used to check outputs where the selection differs from
    the oracle's own only inside the tie band."""
    idx = np.asarray(idx)
    valid = idx >= 0
    w = np.zeros(len(idx))
    w[valid] = inter_chunk_weights(np.asarray(sigma_selected)[valid], scale)
    return attend_row(q_row, keys, values, idx, w, i, chunk, scale)


# ------------------------------------------------------------------------------------------
# Full (dense) attention: the baseline HiLS is compared with ([P3] "Numerical results": prefill
# and per-decode-step latency against full attention on the same hardware; [P1] Model
# Description: the exact attention mass of a chunk comes from the full QK product)
# ------------------------------------------------------------------------------------------

def dense_attention_row(q_row, keys, values, scale) -> np.ndarray:
    """Softmax attention of one query over every given key, float64 [d]."""
    q = np.asarray(q_row, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    a = scale * (k @ q)
    p = np.exp(a - a.max())
    p = p / p.sum()
    return p @ np.asarray(values, dtype=np.float64)


def _causal_end(i: int) -> int:
    """Query position i sees keys 0..i."""
    return i + 1


def dense_causal_rows(inp: Dict[str, np.ndarray], rows: Iterable[tuple],
                      scale: Optional[float] = None) -> Dict[tuple, np.ndarray]:
    """Dense causal attention for selected (b, h, i) rows of q, k, v [B, H, L, d] (raw q, no
    Q-Cal).  Returns {(b, h, i): o [d] float64}."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    d = q.shape[-1]
    s = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    out = {}
    for (b, h, i) in rows:
        e = _causal_end(i)
        out[(b, h, i)] = dense_attention_row(q[b, h, i], k[b, h, :e], v[b, h, :e], s)
    return out


def dense_decode(inp: Dict[str, np.ndarray], scale: Optional[float] = None,
                 pairs: Optional[Iterable[tuple]] = None) -> Dict[tuple, np.ndarray]:
    """Dense attention of q [B, H, d] over the first kv_len[b] keys of k_cache / v_cache
    [B, H, Lmax, d] (the new token's key and value included).  Returns {(b, h): o [d]}."""
    q, kc, vc, kv_len = inp["q"], inp["k_cache"], inp["v_cache"], inp["kv_len"]
    B, H, d = q.shape
    s = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    out = {}
    for (b, h) in pairs:
        e = _causal_end(int(kv_len[b]) - 1)
        out[(b, h)] = dense_attention_row(q[b, h], kc[b, h, :e], vc[b, h, :e], s)
    return out


# ------------------------------------------------------------------------------------------
# Backward pass: gradients of a loss through the forward above.  The pages train the selection
# end to end: the landmark scores sit inside the forward attention, so the next-token loss sends
# gradients into the landmark keys ([P3] "Core idea": gradients flow into the landmark
# representations; [P2]: the chunk scores are learned from the language-modelling loss).
# Readings: the top-k choice is a fixed index set (not differentiable); the rounding of q~ to the
# run dtype passes gradients through unchanged; the loss is sum(dout * o) for a given dout.
# ------------------------------------------------------------------------------------------

def chunk_backward(q_row, keys, values, w_j, dout_row, scale):
    """One (row, chunk) term w_j * o_j with o_j = softmax(scale * K q) V over the chunk's visible
    keys.  Returns (dq [d], dK [n, d], dV [n, d], dw_j = dout . o_j), float64."""
    q = np.asarray(q_row, dtype=np.float64)
    K = np.asarray(keys, dtype=np.float64)
    V = np.asarray(values, dtype=np.float64)
    g = np.asarray(dout_row, dtype=np.float64)
    a = scale * (K @ q)
    p = np.exp(a - a.max())
    p = p / p.sum()
    o_j = p @ V
    dw = float(g @ o_j)                   # d(loss)/d(w_j)
    dp = w_j * (V @ g)                    # d(loss)/d(p_t) for the weighted term
    da = p * (dp - float(p @ dp))         # softmax backward
    dq = scale * (da @ K)
    dK = scale * np.outer(da, q)
    dV = np.outer(w_j * p, g)
    return dq, dK, dV, dw


def inter_chunk_backward(w, dw, scale):
    """d(loss)/d(sigma_j) for w = softmax(scale * sigma) over the selection, given dw_j."""
    w = np.asarray(w, dtype=np.float64)
    dw = np.asarray(dw, dtype=np.float64)
    return scale * w * (dw - float(w @ dw))


def prefill_backward(inp: Dict[str, np.ndarray], dout: np.ndarray, chunk: int, topk: int, dtype: str,
                     scale: Optional[float] = None, sel_idx: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradients of sum(dout * o) for the prefill of inp (as prefill_rows) with respect to q, k,
    v, lmk and, with Q-Cal, h, w_down and w_up.  The selection is the forward's own, or sel_idx
    [B,H,L,k] when given.  Returns float64 arrays keyed dq, dk, dv, dlmk (and dh, dw_down,
    dw_up with Q-Cal).  Also returns dsigma [B,H,L,k] (zero on padding)."""
    q, k, v, lmk = inp["q"], inp["k"], inp["v"], inp["lmk"]
    B, H, L, d = q.shape
    s = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    w_down = inp.get("w_down")
    qcal = w_down is not None and w_down.shape[0] > 0
    out = dict(dq=np.zeros(q.shape), dk=np.zeros(k.shape), dv=np.zeros(v.shape), dlmk=np.zeros(lmk.shape),
               dsigma=np.zeros((B, H, L, topk)))
    if qcal:
        r, D = w_down.shape
        w_up = inp["w_up"].astype(np.float64)
        out.update(dh=np.zeros((B, L, D)), dw_down=np.zeros((r, D)), dw_up=np.zeros((H * d, r)))
        dt = np.zeros((B, L, r))
    for b in range(B):
        for h in range(H):
            for i in range(L):
                # forward of row i (steps 1-4)
                hid = inp["h"][b, i] if qcal else None
                qt = calibrated_query(q[b, h, i], hid, w_down if qcal else None, _w_up_head(inp.get("w_up"), h, d),
                                      dtype)
                c = i // chunk
                sigma = landmark_scores(qt, lmk[b, h, : c + 1])
                idx = select_top_k(sigma, topk) if sel_idx is None else np.asarray(sel_idx[b, h, i])
                js = [int(j) for j in idx if j >= 0]
                w = inter_chunk_weights(np.asarray([sigma[j] for j in js]), s)
                # steps 5-6 backward, chunk by chunk
                dws = np.zeros(len(js))
                for n, j in enumerate(js):
                    lo, hi = _visible_range(j, chunk, i)
                    dq_j, dK, dV, dws[n] = chunk_backward(q[b, h, i], k[b, h, lo:hi], v[b, h, lo:hi], w[n],
                                                         dout[b, h, i], s)
                    out["dq"][b, h, i] += dq_j
                    out["dk"][b, h, lo:hi] += dK
                    out["dv"][b, h, lo:hi] += dV
                # step 4 backward, then step 2 (scores) and step 1 (Q-Cal)
                dsig = inter_chunk_backward(w, dws, s)
                out["dsigma"][b, h, i, : len(js)] = dsig
                dqt = np.zeros(d)
                for n, j in enumerate(js):
                    dqt += dsig[n] * lmk[b, h, j].astype(np.float64)
                    out["dlmk"][b, h, j] += dsig[n] * np.asarray(qt, dtype=np.float64)
                out["dq"][b, h, i] += dqt             # q~ = q + delta_q: rounding passes gradients
                if qcal:
                    t = w_down.astype(np.float64) @ inp["h"][b, i].astype(np.float64)
                    out["dw_up"][h * d:(h + 1) * d] += np.outer(dqt, t)
                    dt[b, i] += w_up[h * d:(h + 1) * d].T @ dqt
    if qcal:
        for b in range(B):
            for i in range(L):
                out["dw_down"] += np.outer(dt[b, i], inp["h"][b, i].astype(np.float64))
                out["dh"][b, i] = w_down.astype(np.float64).T @ dt[b, i]
    return out


# ------------------------------------------------------------------------------------------
# HoPE ([P3] "Engineering details", hierarchical positional encoding item; H1-H3)
# ------------------------------------------------------------------------------------------

def hope_rotated_pairs(d: int, rope_base: float, train_len: int) -> np.ndarray:
    """Indices i of the dimension pairs (2i, 2i+1) that carry the rotary encoding: those whose
    wavelength 2 pi / theta_i, theta_i = base^(-2i/d), fits in the pre-training window (H1, H2)."""
    out = []
    for i in range(d // 2):
        theta = float(rope_base) ** (-2.0 * i / d)
        if 2.0 * math.pi / theta <= train_len:
            out.append(i)
    return np.asarray(out, dtype=np.int64)


def hope_rotate(x: np.ndarray, positions, rope_base: float, train_len: int) -> np.ndarray:
    """x [..., n, d]: row r (position positions[r]) with each pair of hope_rotated_pairs turned by
    the angle pos * theta_i (float64); the other pairs unchanged."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    pos = np.broadcast_to(np.asarray(positions, dtype=np.float64), x.shape[-2:-1])
    out = x.copy()
    for i in hope_rotated_pairs(d, rope_base, train_len):
        theta = float(rope_base) ** (-2.0 * i / d)
        ang = pos * theta
        c, s_ = np.cos(ang), np.sin(ang)
        a, b = x[..., 2 * i], x[..., 2 * i + 1]
        out[..., 2 * i] = a * c - b * s_
        out[..., 2 * i + 1] = a * s_ + b * c
    return out


# ------------------------------------------------------------------------------------------
# Landmark of the chunk still being filled (P1)
# ------------------------------------------------------------------------------------------
def partial_landmark(k_cache: np.ndarray, kv_len, chunk: int, dtype: str) -> Dict[tuple, tuple]:
    """k_cache [B, Hk, Lmax, d], kv_len [B].  For every (sequence b, key/value head g): the chunk
    j = floor((kv_len[b] - 1) / C) that holds the newest key, and the mean of its keys so far
    (rows jC .. kv_len[b] - 1, float64), rounded once to the run dtype (P1).  kv_len is clamped to
    [1, Lmax].  Returns {(b, g): (j, landmark [d])}."""
    B, Hk, Lmax, _ = k_cache.shape
    out = {}
    for b in range(B):
        n_keys = min(max(int(kv_len[b]), 1), Lmax)
        j = (n_keys - 1) // chunk
        for g in range(Hk):
            rows = np.asarray(k_cache[b, g, j * chunk:n_keys], dtype=np.float64)
            out[(b, g)] = (j, round_to_run_dtype(rows.sum(axis=0) / rows.shape[0], dtype))
    return out
