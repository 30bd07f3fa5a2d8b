"""The landmark of the chunk still being filled (hils_partial_landmark) against the oracle: the mean
of the chunk's keys so far written into that chunk's row, every other landmark row untouched, for
ragged and clamped kv_len, bf16 and fp32, d = 64 and 128, chunks of 32, 64 and 128 keys; then a
decode step over the updated landmarks against the oracle's decode with the oracle's landmark."""
import numpy as np
import pytest

from chunk_wise_sparse_amd import synth
from oracle import hils_oracle as O
import test_gpu_decode as TD

pytestmark = pytest.mark.gpu

CASES = [
    # (B, Hk, Lmax, d, C, dtype, kv_len)
    (6, 3, 1000, 128, 64, "bf16", (1, 64, 65, 999, 1000, 5000)),
    (4, 2, 777, 64, 32, "fp32", (31, 32, 33, 777)),
    (5, 4, 3000, 128, 128, "bf16", (1, 127, 128, 129, 2999)),
    (3, 1, 300, 64, 128, "bf16", (300, 256, 257)),
    (2, 8, 4096, 64, 64, "fp32", (4096, 4033)),
]


def _tol(dtype, want):
    # fp32 sums in a fixed order against the float64 mean, both rounded once to the dtype
    return (2.0 ** -7) * np.abs(want) + 1e-7 if dtype == "bf16" else 1e-5 * np.abs(want) + 1e-6


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_Hk{c[1]}_L{c[2]}_d{c[3]}_C{c[4]}_{c[5]}")
def test_partial_landmark_matches_oracle(lib, case):
    from chunk_wise_sparse_amd import hils
    torch = TD._torch()
    B, Hk, Lmax, d, C, dtype, kv = case
    print(f"[case] partial landmark {case}", flush=True)
    g = np.random.default_rng(B * 1000 + Lmax)
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    N = -(-Lmax // C)
    k = torch.from_numpy(g.standard_normal((B, Hk, Lmax, d)).astype(np.float32)).to("cuda", dt)
    lmk = torch.from_numpy(g.standard_normal((B, Hk, N, d)).astype(np.float32)).to("cuda", dt)
    before = lmk.clone()
    kv_len = torch.tensor(kv, dtype=torch.int32, device="cuda")
    hils.partial_landmark(k, lmk, kv_len, chunk=C)
    torch.cuda.synchronize()
    ref = O.partial_landmark(k.float().cpu().numpy(), np.asarray(kv), C, dtype)
    got, prev = lmk.float().cpu().numpy(), before.float().cpu().numpy()
    for (b, gh), (j, want) in ref.items():
        rows = [r for r in range(N) if r != j]
        assert np.array_equal(got[b, gh, rows], prev[b, gh, rows]), (b, gh)
        err = np.abs(got[b, gh, j] - want)
        assert np.all(err <= _tol(dtype, want)), (b, gh, j, err.max())
    # the same call again gives the same bits
    again = before.clone()
    hils.partial_landmark(k, again, kv_len, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(again, lmk)


def test_decode_after_partial_landmark(lib):
    """Steps of a decode: each new key stored, the partial chunk's landmark rewritten, then the
    step; the oracle decodes with its own landmark row on the same caches."""
    from chunk_wise_sparse_amd import hils
    torch = TD._torch()
    cfg = synth.DecodeConfig("partial_lmk_steps", 2, 4, 2000, 128, 64, 8, "bf16", 16, 256, kv_len=(1500, 700))
    inp = synth.make_decode_inputs_np(cfg)
    dev = TD._to_dev(inp, cfg.dtype)
    for step in range(3):
        kv = [cfg.kv_len[b] + step for b in range(cfg.batch)]
        dev["kv_len"] = torch.tensor(kv, dtype=torch.int32, device="cuda")
        hils.partial_landmark(dev["k_cache"], dev["lmk"], dev["kv_len"], chunk=cfg.chunk)
        o, idx, w = TD._run(dev, cfg)
        torch.cuda.synchronize()
        ref_lmk = O.partial_landmark(inp["k_cache"], np.asarray(kv), cfg.chunk, cfg.dtype)
        sub = dict(inp, kv_len=np.asarray(kv, np.int32), lmk=dev["lmk"].float().cpu().numpy())
        for (b, gh), (j, want) in ref_lmk.items():
            assert np.all(np.abs(sub["lmk"][b, gh, j] - want) <= _tol("bf16", want)), (step, b, gh)
        pairs = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
        TD._compare(sub, cfg, o, idx, w, pairs)
