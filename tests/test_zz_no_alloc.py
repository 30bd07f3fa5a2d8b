"""hils_decode_fwd_noalloc (the library's static scratch, no workspace argument) against
hils_decode_fwd with a caller workspace: calls in a row on one GPU, the second smaller than the
first, the third at chunks of 128 keys, each bitwise equal to the workspace entry point (same
kernels), and the first also against the oracle."""
import numpy as np
import pytest

from chunk_wise_sparse_amd import synth
from oracle import hils_oracle as O

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    return torch


def _dev(inp, dtype):
    torch = _torch()
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    return {k: (torch.from_numpy(v).to("cuda") if k == "kv_len" else
                torch.from_numpy(np.ascontiguousarray(v)).to("cuda", dt))
            for k, v in inp.items() if k != "needle_ids"}


def _both(cfg):
    from chunk_wise_sparse_amd import hils
    torch = _torch()
    inp = synth.make_decode_inputs_np(cfg)
    d = _dev(inp, cfg.dtype)
    args = (d["q"], d["k_cache"], d["v_cache"], d["lmk"], d["kv_len"], d.get("h"), d.get("w_down"), d.get("w_up"))
    ref = hils.decode(*args, topk=cfg.topk, chunk=cfg.chunk, return_selection=True)
    got = hils.decode(*args, topk=cfg.topk, chunk=cfg.chunk, return_selection=True, no_alloc=True)
    torch.cuda.synchronize()
    return inp, ref, got


CASES = [
    # 256 (sequence, head) pairs in bf16: the fused one-kernel step; ragged lengths
    synth.DecodeConfig("noalloc_fused", 4, 64, 3000, 128, 64, 64, "bf16", 32, 512, kv_len=(3000, 1, 65, 2047)),
    # a smaller second call: fp32, four pairs, the multi-kernel path
    synth.DecodeConfig("noalloc_small", 2, 2, 1500, 64, 64, 8, "fp32", 8, 128, kv_len=(1500, 700)),
    # a third call at chunks of 128 keys: the scan, the selection and the split attention
    synth.DecodeConfig("noalloc_c128", 2, 4, 5000, 128, 128, 16, "bf16", 16, 256, kv_len=(5000, 333)),
]


def test_noalloc_matches_workspace_entry_two_calls(lib):
    torch = _torch()
    for n, cfg in enumerate(CASES):
        print(f"[case] no-alloc decode call {n}: {cfg}", flush=True)
        inp, ref, got = _both(cfg)
        for a, b, name in zip(got, ref, ("o", "idx", "w")):
            assert torch.equal(a, b), f"call {n}: {name} differs from hils_decode_fwd"
        if n == 0:
            pairs = [(0, 0), (1, 5), (2, 63), (3, 17)]
            res = O.decode(inp, cfg.chunk, cfg.topk, cfg.dtype, pairs=pairs)
            o, idx = got[0].float().cpu().numpy(), got[1].cpu().numpy()
            for (b, h) in pairs:
                assert np.array_equal(idx[b, h], res[(b, h)]["idx"]), (b, h)
                assert np.abs(o[b, h] - res[(b, h)]["o"]).max() <= 2e-2, (b, h)

