"""Grouped-query attention (kv_heads < heads) through the C ABI.  The GPU gets H/G key/value (and
landmark) heads; the oracle gets the same heads repeated G times, which is what grouped-query
attention computes (query head h reads key/value head h / G)."""
import numpy as np
import pytest

from chunk_wise_sparse_amd import hils, synth
import test_gpu_decode as TD
import test_gpu_prefill as TP
from parity import sample_rows

pytestmark = pytest.mark.gpu


def _split(inp, G, keys):
    """(inputs with H/G key/value heads, inputs with those heads repeated G times)."""
    sub, full = dict(inp), dict(inp)
    for key in keys:
        hk = inp[key].shape[1] // G
        sub[key] = np.ascontiguousarray(inp[key][:, :hk])
        full[key] = np.ascontiguousarray(np.repeat(sub[key], G, axis=1))
    return sub, full


PREFILL = [
    (synth.PrefillConfig("gqa_bf16_d128_g4", 1, 8, 2048, 128, 64, 8, "bf16", 16, 256), 4, hils.ATTN_UNION),
    (synth.PrefillConfig("gqa_bf16_d128_g4_cm", 1, 8, 2048, 128, 64, 8, "bf16", 16, 256), 4, hils.ATTN_CHUNK_MAJOR),
    (synth.PrefillConfig("gqa_bf16_k40_g2", 1, 4, 4096, 128, 64, 40, "bf16", 8, 128), 2, hils.ATTN_UNION),
    (synth.PrefillConfig("gqa_bf16_d64_576_g4", 2, 4, 576, 64, 64, 4, "bf16", 0, 0), 4, hils.ATTN_UNION),
    (synth.PrefillConfig("gqa_fp32_d64_g2", 1, 4, 1024, 64, 64, 4, "fp32", 8, 128), 2, hils.ATTN_UNION),
]


@pytest.mark.parametrize("cfg,G,mode", PREFILL, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_prefill_gqa_all_rows(lib, cfg, G, mode):
    print(f"[case] prefill gqa G={G} mode={mode} {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    sub, full = _split(inp, G, ("k", "v", "lmk"))
    o, idx, w = TP._run(lib, TP._to_dev(sub, cfg.dtype), cfg, attn_mode=mode)
    TP._torch().cuda.synchronize()
    rows = [(b, h, i) for b in range(cfg.batch) for h in range(cfg.heads) for i in range(cfg.seq_len)]
    if cfg.seq_len * cfg.heads * cfg.batch > 12000:
        rows = sample_rows(cfg.batch, cfg.heads, cfg.seq_len, 256, seed=31)
    TP._compare(full, cfg, o, idx, w, rows)


DECODE = [
    (synth.DecodeConfig("gqa_dec_bf16_g4", 2, 8, 3000, 128, 64, 16, "bf16", 16, 256, kv_len=(3000, 1234)), 4),
    (synth.DecodeConfig("gqa_dec_fp32_g2", 2, 4, 2000, 64, 64, 4, "fp32", 8, 128, kv_len=(2000, 65)), 2),
    # 256 (sequence, head) pairs: the fused single-kernel step
    (synth.DecodeConfig("gqa_dec_fused_g4", 8, 32, 4096, 128, 64, 16, "bf16", 16, 256,
                        kv_len=(4096, 4000, 3333, 2048, 1500, 777, 130, 64)), 4),
]


@pytest.mark.parametrize("cfg,G", DECODE, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_decode_gqa(lib, cfg, G):
    print(f"[case] decode gqa G={G} {cfg}", flush=True)
    inp = synth.make_decode_inputs_np(cfg)
    sub, full = _split(inp, G, ("k_cache", "v_cache", "lmk"))
    o, idx, w = TD._run(TD._to_dev(sub, cfg.dtype), cfg)
    TD._torch().cuda.synchronize()
    pairs = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    if len(pairs) > 64:
        rng = np.random.default_rng(37)
        pairs = [pairs[i] for i in sorted(rng.choice(len(pairs), 48, replace=False))]
    TD._compare(full, cfg, o, idx, w, pairs)
