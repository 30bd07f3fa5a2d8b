"""Paged keys/values in prefill: the keys and values scattered over shuffled one-chunk pages of a
pool (with spare pages) give bitwise the same selection and output as the contiguous layout, in
every attention path and at chunks of 32, 64 and 128 keys, and match the oracle."""
import numpy as np
import pytest

from chunk_wise_sparse_amd import synth
from test_gpu_prefill import _compare, _torch

pytestmark = pytest.mark.gpu


def _paged(k, v, seed, C=64):
    """Pools [pages, Hkv, C, d] holding k, v [B, Hkv, L, d] chunk by chunk, and the block table."""
    torch = _torch()
    B, Hk, L, d = k.shape
    N = L // C
    g = np.random.default_rng(seed)
    pages = B * N + 7                          # spare pages hold noise
    perm = g.permutation(pages)[: B * N]
    table = torch.from_numpy(perm.reshape(B, N).astype(np.int32)).to(k.device)
    kp = torch.randn((pages, Hk, C, d), device=k.device).to(k.dtype)
    vp = torch.randn((pages, Hk, C, d), device=k.device).to(k.dtype)
    for b in range(B):
        for j in range(N):
            kp[perm[b * N + j]] = k[b, :, C * j:C * j + C]
            vp[perm[b * N + j]] = v[b, :, C * j:C * j + C]
    return kp, vp, table


@pytest.mark.parametrize("cfg,kv_heads,mode", [
    (synth.PrefillConfig("paged_bf16_k8", 2, 2, 1024, 128, 64, 8, "bf16", 16, 256), 0, 0),
    (synth.PrefillConfig("paged_bf16_k48_gqa", 1, 4, 2048, 64, 64, 48, "bf16", 8, 128), 2, 0),
    (synth.PrefillConfig("paged_fp32", 1, 2, 640, 64, 64, 4, "fp32", 8, 128), 0, 0),
    (synth.PrefillConfig("paged_chunk_major", 1, 2, 2048, 128, 64, 16, "bf16", 16, 256), 0, 1),
    # chunks of 128 and 32 keys: pages of C rows under the chunk-major kernels
    (synth.PrefillConfig("paged_c128_bf16", 2, 2, 2048, 128, 128, 8, "bf16", 16, 256), 0, 0),
    (synth.PrefillConfig("paged_c32_bf16_gqa", 1, 4, 1536, 64, 32, 12, "bf16", 8, 128), 2, 0),
], ids=lambda x: getattr(x, "name", str(x)))
def test_prefill_paged_matches_contiguous(lib, cfg, kv_heads, mode):
    from chunk_wise_sparse_amd import hils
    torch = _torch()
    print(f"[case] paged prefill {cfg} kv_heads={kv_heads} mode={mode}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    G = cfg.heads // kv_heads if kv_heads else 1
    if G > 1:
        for key in ("k", "v", "lmk"):
            inp[key] = np.ascontiguousarray(np.repeat(inp[key][:, ::G], G, axis=1))
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32}[cfg.dtype]
    dev = {key: torch.from_numpy(np.ascontiguousarray(val)).to("cuda", dt) for key, val in inp.items()}
    for key in ("k", "v", "lmk"):
        dev[key] = dev[key][:, ::G].contiguous()
    kp, vp, table = _paged(dev["k"], dev["v"], seed=cfg.seq_len, C=cfg.chunk)
    ref = hils.prefill(dev["q"], dev["k"], dev["v"], dev["lmk"], dev.get("h"), dev.get("w_down"), dev.get("w_up"),
                       topk=cfg.topk, chunk=cfg.chunk, return_selection=True, attn_mode=mode)
    got = hils.prefill(dev["q"], kp, vp, dev["lmk"], dev.get("h"), dev.get("w_down"), dev.get("w_up"),
                       topk=cfg.topk, chunk=cfg.chunk, return_selection=True, attn_mode=mode, block_table=table)
    torch.cuda.synchronize()
    for a, b, name in zip(got, ref, ("o", "idx", "w")):
        assert torch.equal(a, b), name
    rows = [(b, h, i) for b in range(cfg.batch) for h in range(cfg.heads) for i in range(0, cfg.seq_len, 3)]
    _compare(inp, cfg, *got, rows)
