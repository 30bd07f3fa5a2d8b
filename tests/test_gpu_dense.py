"""The dense causal attention baseline (prefill and decode) on the GPU through the C ABI, against
the oracle's dense attention, element by element."""
import math

import numpy as np
import pytest

from chunk_wise_sparse_amd import synth
from oracle import hils_oracle as O
from parity import TOL_O

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    return torch


def _dt(dtype):
    torch = _torch()
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]


def _round(x, dtype):
    return synth.round_to_dtype_np(x, dtype)


def _check(got, want, dtype, what):
    diff = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    mx, mean = TOL_O[dtype]
    print(f"[parity] {what}: max|do| {diff.max():.3g} mean|do| {diff.mean():.3g}", flush=True)
    assert diff.max() <= mx and diff.mean() <= mean, (what, diff.max(), diff.mean())


def _prefill_case(B, H, Hkv, L, d, dtype, seed):
    g = np.random.default_rng(seed)
    q = _round(g.standard_normal((B, H, L, d), dtype=np.float32), dtype)
    k = _round(g.standard_normal((B, Hkv, L, d), dtype=np.float32), dtype)
    v = _round(g.standard_normal((B, Hkv, L, d), dtype=np.float32), dtype)
    return q, k, v


@pytest.mark.parametrize("B,H,Hkv,L,d,dtype", [
    (1, 2, 2, 640, 64, "fp32"),        # L % 128 != 0: four-wave groups
    (1, 1, 1, 512, 128, "fp32"),
    (2, 4, 2, 1024, 128, "bf16"),      # grouped-query heads
    (1, 2, 2, 2048, 64, "bf16"),
    (1, 1, 1, 64, 128, "bf16"),        # one chunk
])
def test_dense_prefill_all_rows(lib, B, H, Hkv, L, d, dtype):
    from chunk_wise_sparse_amd import hils
    import oracle_pool  # noqa: F401  (rows are few enough for one process here)
    torch = _torch()
    print(f"[case] dense prefill B={B} H={H} Hkv={Hkv} L={L} d={d} {dtype}", flush=True)
    q, k, v = _prefill_case(B, H, Hkv, L, d, dtype, seed=L + d)
    dt = _dt(dtype)
    o = hils.dense_prefill(*(torch.from_numpy(x).to("cuda", dt) for x in (q, k, v)))
    torch.cuda.synchronize()
    G = H // Hkv
    inp = dict(q=q, k=np.repeat(k, G, axis=1), v=np.repeat(v, G, axis=1))
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(L)]
    ref = O.dense_causal_rows(inp, rows)
    got = o.float().cpu().numpy()
    _check(np.stack([got[r] for r in rows]), np.stack([ref[r] for r in rows]), dtype, f"dense prefill L={L} {dtype}")


def test_dense_prefill_32k_sampled(lib):
    """The 32K workload's shape (H = 16, d = 64, bf16): sampled rows of every head."""
    from chunk_wise_sparse_amd import hils
    torch = _torch()
    cfg = synth.CONFIGS["prefill_32k"]
    print(f"[case] dense prefill {cfg.name}", flush=True)
    dev = synth.make_prefill_inputs_torch(cfg, "cuda")
    o = hils.dense_prefill(dev["q"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    g = np.random.default_rng(3)
    rows = [(0, h, int(i)) for h in range(cfg.heads) for i in
            np.concatenate([[0, 63, 64, cfg.seq_len - 1], g.integers(0, cfg.seq_len, 12)])]
    inp = {key: dev[key].float().cpu().numpy() for key in ("q", "k", "v")}
    ref = O.dense_causal_rows(inp, rows)
    got = o.float().cpu().numpy()
    _check(np.stack([got[r] for r in rows]), np.stack([ref[r] for r in rows]), "bf16", "dense prefill 32K")


@pytest.mark.parametrize("B,H,Hkv,Lmax,d,dtype,lens", [
    (2, 2, 2, 1500, 64, "fp32", (1500, 1)),
    (3, 4, 2, 5000, 128, "fp32", (5000, 65, 4097)),
    (4, 8, 8, 3000, 128, "bf16", (3000, 64, 1, 2047)),
    (2, 4, 1, 20000, 64, "bf16", (20000, 12345)),
])
def test_dense_decode(lib, B, H, Hkv, Lmax, d, dtype, lens):
    from chunk_wise_sparse_amd import hils
    torch = _torch()
    print(f"[case] dense decode B={B} H={H} Hkv={Hkv} Lmax={Lmax} d={d} {dtype} kv_len={lens}", flush=True)
    g = np.random.default_rng(Lmax)
    q = _round(g.standard_normal((B, H, d), dtype=np.float32), dtype)
    kc = _round(g.standard_normal((B, Hkv, Lmax, d), dtype=np.float32), dtype)
    vc = _round(g.standard_normal((B, Hkv, Lmax, d), dtype=np.float32), dtype)
    dt = _dt(dtype)
    kv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o = hils.dense_decode(torch.from_numpy(q).to("cuda", dt), torch.from_numpy(kc).to("cuda", dt),
                          torch.from_numpy(vc).to("cuda", dt), kv)
    torch.cuda.synchronize()
    G = H // Hkv
    inp = dict(q=q, k_cache=np.repeat(kc, G, axis=1), v_cache=np.repeat(vc, G, axis=1),
               kv_len=np.asarray(lens, np.int32))
    ref = O.dense_decode(inp)
    got = o.float().cpu().numpy()
    pairs = sorted(ref)
    _check(np.stack([got[p] for p in pairs]), np.stack([ref[p] for p in pairs]), dtype, f"dense decode {lens}")


def test_dense_decode_matches_dense_prefill_rows(lib):
    """decode(kv_len = i + 1) of a cache holding a prefill's keys equals that prefill's row i."""
    from chunk_wise_sparse_amd import hils
    torch = _torch()
    q, k, v = _prefill_case(1, 2, 2, 1024, 128, "fp32", seed=9)
    dev = [torch.from_numpy(x).to("cuda") for x in (q, k, v)]
    o = hils.dense_prefill(*dev)
    for i in (0, 63, 64, 500, 1023):
        od = hils.dense_decode(dev[0][:, :, i].contiguous(), dev[1], dev[2],
                               torch.tensor([i + 1], dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert (od - o[:, :, i]).abs().max().item() <= 1e-5, i
