"""Backward pass of the prefill on the GPU through the C ABI, every gradient element against the
oracle's float64 backward over the same selection.

Tolerances (relative to the largest magnitude of each reference gradient):
  fp32: max |g - g_ref| <= 1e-4 * max |g_ref|;
  bf16: max |g - g_ref| <= 2e-2 * max |g_ref| and rms(g - g_ref) <= 1e-2 * rms(g_ref).
bf16 rounds the chunk softmax p and ds to bf16 (relative 2^-9 each) before the MFMA products and
every gradient once more on output, so a few 2^-9 of the largest term bounds the error.
"""
import numpy as np
import pytest

from chunk_wise_sparse_amd import synth
from oracle import hils_oracle as O

pytestmark = pytest.mark.gpu

TOL = {"fp32": (1e-4, None), "bf16": (2e-2, 1e-2)}


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    return torch


CASES = [
    (synth.PrefillConfig("bwd_fp32_d64", 1, 2, 640, 64, 64, 4, "fp32", 8, 128), 0),
    (synth.PrefillConfig("bwd_fp32_d128_noqcal", 1, 1, 512, 128, 64, 3, "fp32", 0, 0), 0),
    (synth.PrefillConfig("bwd_bf16_d128", 2, 2, 1024, 128, 64, 8, "bf16", 16, 256, q_mode="walk"), 0),
    (synth.PrefillConfig("bwd_bf16_d64_allchunks", 1, 1, 2048, 64, 64, 64, "bf16", 4, 128), 0),
    (synth.PrefillConfig("bwd_bf16_gqa", 1, 4, 512, 128, 64, 4, "bf16", 8, 128), 2),
    (synth.PrefillConfig("bwd_fp32_gqa_L576", 1, 2, 576, 64, 64, 5, "fp32", 0, 0), 1),
    # 64 chunks, k = 32: the selection's two-pass regime and long per-chunk lists
    (synth.PrefillConfig("bwd_bf16_4k_k32", 1, 2, 4096, 128, 64, 32, "bf16", 32, 512, q_mode="walk",
                         h_mode="walk"), 0),
    # Q-Cal rank above 32 (two 32-code blocks), H d and hidden not multiples of 512, and split-K
    # splits of 1046 and 1044 tokens (ragged 16-token groups)
    (synth.PrefillConfig("bwd_bf16_r36_ragged", 1, 3, 3136, 64, 64, 8, "bf16", 36, 384), 0),
    (synth.PrefillConfig("bwd_fp32_r40", 1, 2, 1152, 128, 64, 6, "fp32", 40, 256), 0),
]


@pytest.mark.parametrize("cfg,kv_heads", CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_backward_matches_oracle(lib, cfg, kv_heads):
    from chunk_wise_sparse_amd import hils
    torch = _torch()
    print(f"[case] backward {cfg} kv_heads={kv_heads}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    G = cfg.heads // kv_heads if kv_heads else 1
    if G > 1:        # key/value heads: every G-th head's tensors, repeated for the oracle
        for key in ("k", "v", "lmk"):
            inp[key] = np.ascontiguousarray(np.repeat(inp[key][:, ::G], G, axis=1))
    dout = synth.round_to_dtype_np(np.random.default_rng(99).standard_normal(inp["q"].shape), cfg.dtype)
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32}[cfg.dtype]
    dev = {key: torch.from_numpy(np.ascontiguousarray(val)).to("cuda", dt) for key, val in inp.items()}
    for key in ("k", "v", "lmk"):
        dev[key] = dev[key][:, ::G].contiguous()
    dout_d = torch.from_numpy(dout).to("cuda", dt)
    o, idx, w = hils.prefill(dev["q"], dev["k"], dev["v"], dev["lmk"], dev.get("h"), dev.get("w_down"),
                             dev.get("w_up"), topk=cfg.topk, return_selection=True)
    grads = hils.prefill_bwd(dev["q"], dev["k"], dev["v"], dev["lmk"], dev.get("h"), dev.get("w_down"),
                             dev.get("w_up"), idx, w, dout_d, topk=cfg.topk)
    again = hils.prefill_bwd(dev["q"], dev["k"], dev["v"], dev["lmk"], dev.get("h"), dev.get("w_down"),
                             dev.get("w_up"), idx, w, dout_d, topk=cfg.topk)
    torch.cuda.synchronize()
    for name in grads:                        # fixed summation order: bitwise reproducible
        assert torch.equal(grads[name], again[name]), name
    ref = O.prefill_backward(inp, dout, cfg.chunk, cfg.topk, cfg.dtype, sel_idx=idx.cpu().numpy())
    if G > 1:        # gradients of shared key/value heads are the sums over their query heads
        for key in ("dk", "dv", "dlmk"):
            r = ref[key]
            ref[key] = r.reshape(r.shape[0], r.shape[1] // G, G, *r.shape[2:]).sum(axis=2)
    mx_tol, rms_tol = TOL[cfg.dtype]
    for name, g in grads.items():
        got = g.float().cpu().numpy().astype(np.float64)
        want = ref[name]
        assert got.shape == want.shape, (name, got.shape, want.shape)
        scale = float(np.abs(want).max())
        err = np.abs(got - want)
        rel_max = float(err.max()) / max(scale, 1e-30)
        rel_rms = float(np.sqrt((err ** 2).mean() / max((want ** 2).mean(), 1e-60)))
        print(f"[parity] {cfg.name} {name}: max|g| {scale:.3g} rel max {rel_max:.3g} rel rms {rel_rms:.3g}",
              flush=True)
        assert scale > 0, name
        assert rel_max <= mx_tol, (name, rel_max)
        if rms_tol is not None:
            assert rel_rms <= rms_tol, (name, rel_rms)
