"""Seeded synthetic inputs for the HiLS attention forward pass.

This module only draws inputs: Gaussian tensors, normalised random walks,
chunk-mean landmark keys and planted "needle" landmarks.  It holds none of the
attention method's arithmetic and imports neither the HIP library nor the
oracle, so that the CPU oracle and the GPU path can both be fed from it.

The workloads stand in for the pages' own long-context evaluations (RULER,
LongBench and perplexity runs of a trained 7B model), which need weights and
datasets that are not available: every tensor here is random with the shapes
of those runs.

Recipe (per tensor a fixed sub-seed ``seed*1000 + SUBSEED[name]``):
  * q, k, v ~ N(0, 1), rounded to the run dtype;
  * landmark key of chunk j = mean of the chunk's (dtype-rounded) keys
    + 0.1 * N(0, 1), rounded to the run dtype;
  * Q-Cal weights W_down [r, D], W_up [H*d, r] ~ N(0, 0.02^2);
  * hidden state h ~ N(0, 1), or a random walk (below);
  * "walk" queries: q_0 = sqrt(d) * u/|u|, q_t = sqrt(d) * normalise(q_{t-1} + 0.05 * eps_t),
    one walk per (batch, head); "walk" hidden states: the same with sqrt(D);
  * decode needles: per (sequence, head) 4 distinct chunks whose landmark is
    replaced by |lmk_j| * (0.9 * q_hat + sqrt(0.19) * u_perp), u_perp a random
    unit vector orthogonal to q_hat (cosine 0.9 with the raw query).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np

SUBSEED = dict(q=1, k=2, v=3, lmk_noise=4, h=5, w_down=6, w_up=7, needle=8)
WALK_STEP_STD = 0.05
LMK_NOISE_STD = 0.1
QCAL_WEIGHT_STD = 0.02
NEEDLE_COSINE = 0.9


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    chunk: int
    topk: int
    dtype: str          # "bf16" or "fp32"
    qcal_rank: int      # r (0 = no Q-Cal)
    hidden: int         # D
    q_mode: str = "iid"  # "iid" or "walk"
    h_mode: str = "iid"  # "iid" or "walk"
    q_tile: int = 64
    seed: int = 0

    @property
    def n_chunks(self) -> int:
        return self.seq_len // self.chunk


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    heads: int
    max_kv_len: int
    head_dim: int
    chunk: int
    topk: int
    dtype: str
    qcal_rank: int
    hidden: int
    kv_len: Sequence[int]   # one length per sequence, 1 <= kv_len[b] <= max_kv_len
    needles: int = 0
    seed: int = 0

    @property
    def n_chunks(self) -> int:
        return -(-self.max_kv_len // self.chunk)


# The five workloads: a tiny fp32 case, a 345M-scale 32K prefill, a 7B-shape
# 128K prefill, a 7B-shape 512K decode step and a 512K prefill in two query regimes.
CONFIGS: Dict[str, object] = {
    "tiny_fp32": PrefillConfig("tiny_fp32", 1, 2, 2048, 64, 64, 4, "fp32", 8, 128),
    "prefill_32k": PrefillConfig("prefill_32k", 1, 16, 32768, 64, 64, 16, "bf16", 16, 1024),
    "prefill_128k": PrefillConfig("prefill_128k", 1, 32, 131072, 128, 64, 32, "bf16", 32, 4096,
                                  q_mode="walk", h_mode="walk"),
    "decode_512k": DecodeConfig("decode_512k", 8, 32, 524288, 128, 64, 64, "bf16", 32, 4096,
                                kv_len=(524288,) * 8, needles=4),
    "prefill_512k_walk": PrefillConfig("prefill_512k_walk", 1, 32, 524288, 128, 64, 64, "bf16", 32, 4096,
                                       q_mode="walk", h_mode="walk"),
    "prefill_512k_iid": PrefillConfig("prefill_512k_iid", 1, 32, 524288, 128, 64, 64, "bf16", 32, 4096,
                                      q_mode="iid", h_mode="iid"),
}


def subseed(seed: int, name: str) -> int:
    return seed * 1000 + SUBSEED[name]


def round_to_dtype_np(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float data to the run dtype (bf16 via torch's CPU conversion) and return fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp32":
        return x
    if dtype != "bf16":
        raise ValueError(dtype)
    import torch
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()


def random_walk(rng: np.random.Generator, n_walks: int, steps: int, dim: int, norm: float,
                step_std: float = WALK_STEP_STD, block: int = 4096) -> np.ndarray:
    """Normalised Gaussian random walks, shape [n_walks, steps, dim], fp32."""
    out = np.empty((n_walks, steps, dim), dtype=np.float32)
    x = rng.standard_normal((n_walks, dim))
    x *= norm / np.linalg.norm(x, axis=1, keepdims=True)
    t = 0
    while t < steps:
        nb = min(block, steps - t)
        eps = rng.standard_normal((nb, n_walks, dim)) * step_std
        for s in range(nb):
            if t + s > 0:
                x = x + eps[s]
                x *= norm / np.linalg.norm(x, axis=1, keepdims=True)
            out[:, t + s] = x
        t += nb
    return out


def chunk_mean_landmarks_np(k: np.ndarray, chunk: int, noise: np.ndarray) -> np.ndarray:
    """Landmark per chunk: mean of that chunk's keys plus noise. k [..., L, d] -> [..., ceil(L/C), d]."""
    *lead, L, d = k.shape
    n = -(-L // chunk)
    pad = n * chunk - L
    sums = np.zeros((*lead, n, d), dtype=np.float64)
    counts = np.full(n, chunk, dtype=np.float64)
    if pad:
        counts[-1] = chunk - pad
    full = (L // chunk) * chunk
    sums[..., : L // chunk, :] = k[..., :full, :].reshape(*lead, L // chunk, chunk, d).sum(axis=-2)
    if pad:
        sums[..., -1, :] = k[..., full:, :].sum(axis=-2)
    return (sums / counts[:, None] + noise).astype(np.float32)


def make_prefill_inputs_np(cfg: PrefillConfig) -> Dict[str, np.ndarray]:
    """Host (NumPy PCG64) inputs for a prefill config; fp32 arrays holding dtype-exact values."""
    B, H, L, d, C, r, D = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.chunk, cfg.qcal_rank, cfg.hidden
    rng = lambda name: np.random.default_rng(subseed(cfg.seed, name))
    if cfg.q_mode == "walk":
        q = random_walk(rng("q"), B * H, L, d, math.sqrt(d)).reshape(B, H, L, d)
    else:
        q = rng("q").standard_normal((B, H, L, d), dtype=np.float32)
    k = rng("k").standard_normal((B, H, L, d), dtype=np.float32)
    v = rng("v").standard_normal((B, H, L, d), dtype=np.float32)
    q, k, v = (round_to_dtype_np(t, cfg.dtype) for t in (q, k, v))
    noise = rng("lmk_noise").standard_normal((B, H, -(-L // C), d)) * LMK_NOISE_STD
    lmk = round_to_dtype_np(chunk_mean_landmarks_np(k, C, noise), cfg.dtype)
    out = dict(q=q, k=k, v=v, lmk=lmk)
    if r > 0:
        if cfg.h_mode == "walk":
            h = random_walk(rng("h"), B, L, D, math.sqrt(D)).reshape(B, L, D)
        else:
            h = rng("h").standard_normal((B, L, D), dtype=np.float32)
        out["h"] = round_to_dtype_np(h, cfg.dtype)
        out["w_down"] = round_to_dtype_np(rng("w_down").standard_normal((r, D)) * QCAL_WEIGHT_STD, cfg.dtype)
        out["w_up"] = round_to_dtype_np(rng("w_up").standard_normal((H * d, r)) * QCAL_WEIGHT_STD, cfg.dtype)
    return out


def plant_needles_np(rng: np.random.Generator, lmk: np.ndarray, q: np.ndarray, kv_len: Sequence[int],
                     chunk: int, n_needles: int) -> np.ndarray:
    """Return per-(b,h) needle chunk ids [B,H,n] and modify lmk [B,H,N,d] in place (fp32 values).

    The needle landmark keeps its norm and gets cosine NEEDLE_COSINE with q[b,h]."""
    B, H, N, d = lmk.shape
    ids = np.zeros((B, H, n_needles), dtype=np.int64)
    for b in range(B):
        nb = -(-int(kv_len[b]) // chunk)
        m = min(n_needles, nb)
        for hh in range(H):
            sel = np.sort(rng.choice(nb, size=m, replace=False))
            ids[b, hh, :m] = sel
            ids[b, hh, m:] = -1
            qhat = q[b, hh].astype(np.float64)
            qhat /= np.linalg.norm(qhat)
            for j in sel:
                u = rng.standard_normal(d)
                u -= u.dot(qhat) * qhat
                u /= np.linalg.norm(u)
                nrm = np.linalg.norm(lmk[b, hh, j].astype(np.float64))
                lmk[b, hh, j] = (nrm * (NEEDLE_COSINE * qhat + math.sqrt(1 - NEEDLE_COSINE ** 2) * u)).astype(np.float32)
    return ids


def make_decode_inputs_np(cfg: DecodeConfig) -> Dict[str, np.ndarray]:
    """Host inputs for a (small) decode config; fp32 arrays holding dtype-exact values."""
    B, H, Lm, d, C, r, D = cfg.batch, cfg.heads, cfg.max_kv_len, cfg.head_dim, cfg.chunk, cfg.qcal_rank, cfg.hidden
    rng = lambda name: np.random.default_rng(subseed(cfg.seed, name))
    q = round_to_dtype_np(rng("q").standard_normal((B, H, d), dtype=np.float32), cfg.dtype)
    k = round_to_dtype_np(rng("k").standard_normal((B, H, Lm, d), dtype=np.float32), cfg.dtype)
    v = round_to_dtype_np(rng("v").standard_normal((B, H, Lm, d), dtype=np.float32), cfg.dtype)
    noise = rng("lmk_noise").standard_normal((B, H, cfg.n_chunks, d)) * LMK_NOISE_STD
    lmk = chunk_mean_landmarks_np(k, C, noise)
    needle_ids = None
    if cfg.needles:
        needle_ids = plant_needles_np(rng("needle"), lmk, q, cfg.kv_len, C, cfg.needles)
    out = dict(q=q, k_cache=k, v_cache=v, lmk=round_to_dtype_np(lmk, cfg.dtype),
               kv_len=np.asarray(cfg.kv_len, dtype=np.int32))
    if needle_ids is not None:
        out["needle_ids"] = needle_ids
    if r > 0:
        out["h"] = round_to_dtype_np(rng("h").standard_normal((B, D), dtype=np.float32), cfg.dtype)
        out["w_down"] = round_to_dtype_np(rng("w_down").standard_normal((r, D)) * QCAL_WEIGHT_STD, cfg.dtype)
        out["w_up"] = round_to_dtype_np(rng("w_up").standard_normal((H * d, r)) * QCAL_WEIGHT_STD, cfg.dtype)
    return out


# ----------------------------------------------------------------------------------------------
# Device generators (torch).  Values differ from the host generators but are seeded the same way.
# ----------------------------------------------------------------------------------------------

def _torch_dtype(name: str):
    import torch
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def _randn_dev(gen, shape, device, dtype, slab: int = 1 << 28):
    """N(0,1) in `dtype`, drawn in fp32 slabs along dim 0 to bound temporary memory."""
    import torch
    out = torch.empty(shape, device=device, dtype=dtype)
    flat = out.view(shape[0], -1)
    rows = max(1, slab // max(1, flat.shape[1]))
    for s in range(0, shape[0], rows):
        e = min(shape[0], s + rows)
        flat[s:e] = torch.randn((e - s, flat.shape[1]), generator=gen, device=device, dtype=torch.float32).to(dtype)
    return out


def _landmarks_dev(gen, k, chunk: int, dtype):
    """Chunk-mean landmarks of k [B,H,L,d] (L multiple of chunk) plus 0.1*N(0,1), on the device."""
    import torch
    B, H, L, d = k.shape
    N = L // chunk
    lmk = torch.empty((B, H, N, d), device=k.device, dtype=dtype)
    for b in range(B):
        for h0 in range(0, H, 4):
            h1 = min(H, h0 + 4)
            m = k[b, h0:h1].view(h1 - h0, N, chunk, d).to(torch.float32).mean(dim=2)
            m += LMK_NOISE_STD * torch.randn(m.shape, generator=gen, device=k.device, dtype=torch.float32)
            lmk[b, h0:h1] = m.to(dtype)
    return lmk


def chunk_landmarks_dev(k, chunk: int, seed: int = 0):
    """Landmarks of a device key cache [B,H,L,d] (L a multiple of chunk) for another chunk size, by
    the workloads' recipe (chunk means plus noise, no needles), in k's dtype."""
    import torch
    gen = torch.Generator(device=k.device)
    gen.manual_seed(subseed(seed, "lmk_noise"))
    return _landmarks_dev(gen, k, chunk, k.dtype)


def make_prefill_inputs_torch(cfg: PrefillConfig, device="cuda", q_mode: Optional[str] = None,
                              h_mode: Optional[str] = None):
    """Device inputs for a prefill config (torch tensors in the run dtype)."""
    import torch
    dt = _torch_dtype(cfg.dtype)
    B, H, L, d, C, r, D = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.chunk, cfg.qcal_rank, cfg.hidden
    q_mode = q_mode or cfg.q_mode
    h_mode = h_mode or cfg.h_mode
    gen = lambda name: torch.Generator(device=device).manual_seed(subseed(cfg.seed, name))
    if q_mode == "walk":
        walk = random_walk(np.random.default_rng(subseed(cfg.seed, "q")), B * H, L, d, math.sqrt(d))
        q = torch.from_numpy(walk).view(B, H, L, d).to(device=device, dtype=dt)
        del walk
    else:
        q = _randn_dev(gen("q"), (B, H, L, d), device, dt)
    k = _randn_dev(gen("k"), (B, H, L, d), device, dt)
    v = _randn_dev(gen("v"), (B, H, L, d), device, dt)
    lmk = _landmarks_dev(gen("lmk_noise"), k, C, dt)
    out = dict(q=q, k=k, v=v, lmk=lmk)
    if r > 0:
        if h_mode == "walk":
            walk = random_walk(np.random.default_rng(subseed(cfg.seed, "h")), B, L, D, math.sqrt(D))
            out["h"] = torch.from_numpy(walk).view(B, L, D).to(device=device, dtype=dt)
            del walk
        else:
            out["h"] = _randn_dev(gen("h"), (B, L, D), device, dt)
        out["w_down"] = (QCAL_WEIGHT_STD * torch.randn((r, D), generator=gen("w_down"), device=device)).to(dt)
        out["w_up"] = (QCAL_WEIGHT_STD * torch.randn((H * d, r), generator=gen("w_up"), device=device)).to(dt)
    return out


def make_decode_inputs_torch(cfg: DecodeConfig, device="cuda"):
    """Device inputs for a decode config.  The cache length is rounded up to whole chunks for the
    landmark recipe; needles are drawn on the host and written into the device landmarks."""
    import torch
    dt = _torch_dtype(cfg.dtype)
    B, H, Lm, d, C, r, D = cfg.batch, cfg.heads, cfg.max_kv_len, cfg.head_dim, cfg.chunk, cfg.qcal_rank, cfg.hidden
    if Lm % C:
        raise ValueError("device decode generator needs max_kv_len to be a multiple of the chunk size")
    gen = lambda name: torch.Generator(device=device).manual_seed(subseed(cfg.seed, name))
    q = _randn_dev(gen("q"), (B, H, d), device, dt)
    k = _randn_dev(gen("k"), (B, H, Lm, d), device, dt)
    v = _randn_dev(gen("v"), (B, H, Lm, d), device, dt)
    lmk = _landmarks_dev(gen("lmk_noise"), k, C, dt)
    out = dict(q=q, k_cache=k, v_cache=v, lmk=lmk,
               kv_len=torch.tensor(list(cfg.kv_len), dtype=torch.int32, device=device))
    if cfg.needles:
        rng = np.random.default_rng(subseed(cfg.seed, "needle"))
        qh = q.float().cpu().numpy()
        ids = np.zeros((B, H, cfg.needles), dtype=np.int64)
        for b in range(B):
            nb = -(-int(cfg.kv_len[b]) // C)
            for hh in range(H):
                sel = np.sort(rng.choice(nb, size=cfg.needles, replace=False))
                ids[b, hh] = sel
                rows = lmk[b, hh, torch.from_numpy(sel).to(device)].float().cpu().numpy().astype(np.float64)
                qhat = qh[b, hh].astype(np.float64)
                qhat /= np.linalg.norm(qhat)
                new = np.empty_like(rows)
                for t in range(len(sel)):
                    u = rng.standard_normal(d)
                    u -= u.dot(qhat) * qhat
                    u /= np.linalg.norm(u)
                    new[t] = np.linalg.norm(rows[t]) * (NEEDLE_COSINE * qhat + math.sqrt(1 - NEEDLE_COSINE ** 2) * u)
                lmk[b, hh, torch.from_numpy(sel).to(device)] = torch.from_numpy(new.astype(np.float32)).to(device, dt)
        out["needle_ids"] = ids
    if r > 0:
        out["h"] = _randn_dev(gen("h"), (B, D), device, dt)
        out["w_down"] = (QCAL_WEIGHT_STD * torch.randn((r, D), generator=gen("w_down"), device=device)).to(dt)
        out["w_up"] = (QCAL_WEIGHT_STD * torch.randn((H * d, r), generator=gen("w_up"), device=device)).to(dt)
    return out
