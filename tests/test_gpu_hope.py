"""HoPE rotation on the GPU through the C ABI against the oracle's float64 rotation.

Bars: fp32 within 1e-5 absolute (cosine and sine rounded to fp32, one fp32 product sum per
element, inputs of unit scale); bf16 within one bf16 step of the larger of the element and 1
(2^-8: the fp32 result is rounded once to bf16); pairs outside the window bitwise unchanged.
"""
import numpy as np
import pytest

from oracle import hils_oracle as O

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    return torch


CASES = [
    # (dtype, B, H, L, d, base, window, pos0, positions)
    ("fp32", 2, 3, 200, 128, 10000.0, 4096, 5, None),
    ("bf16", 2, 3, 200, 128, 10000.0, 4096, 0, None),
    ("fp32", 1, 2, 77, 64, 500000.0, 8192, 0, None),
    ("bf16", 1, 4, 33, 64, 10000.0, 64, 131000, None),
    ("fp32", 3, 2, 1, 128, 10000.0, 4096, 0, [0, 1000, 524287]),     # decode queries
    ("bf16", 3, 2, 40, 128, 10000.0, 2048, 0, [7, 65536, 524200]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_B{c[1]}H{c[2]}L{c[3]}d{c[4]}_w{c[6]}")
def test_hope_matches_oracle(lib, case):
    from chunk_wise_sparse_amd import hils
    torch = _torch()
    dtype, B, H, L, d, base, win, pos0, positions = case
    print(f"[case] hope {case}", flush=True)
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    x = torch.from_numpy(np.random.default_rng(5).standard_normal((B, H, L, d)).astype(np.float32)).to(tdt)
    x_in = x.float().numpy().astype(np.float64)
    xd = x.to("cuda")
    pt = None if positions is None else torch.tensor(positions, dtype=torch.int32, device="cuda")
    hils.hope_rotate(xd, rope_base=base, train_len=win, pos0=pos0, positions=pt)
    torch.cuda.synchronize()
    got = xd.float().cpu().numpy().astype(np.float64)
    want = np.empty_like(x_in)
    for b in range(B):
        start = pos0 if positions is None else positions[b]
        want[b] = O.hope_rotate(x_in[b], np.arange(L) + start, base, win)
    rot = O.hope_rotated_pairs(d, base, win)
    assert 0 < len(rot) <= d // 2
    keep = np.ones(d, dtype=bool)
    for i in rot:
        keep[2 * i:2 * i + 2] = False
    assert np.array_equal(got[..., keep], x_in[..., keep]), "pairs outside the window changed"
    err = np.abs(got - want)
    if dtype == "fp32":
        assert err.max() <= 1e-5, err.max()
    else:
        assert np.all(err <= 2.0 ** -8 * np.maximum(np.abs(want), 1.0)), err.max()
    print(f"[parity] hope {dtype} d={d}: {len(rot)} of {d // 2} pairs rotated, max err {err.max():.3g}", flush=True)
