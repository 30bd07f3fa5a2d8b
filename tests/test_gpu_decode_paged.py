"""Paged key/value caches for decode (block_table): the same step on the same cache contents laid
out as shuffled pages must give bitwise the same selection and output as the contiguous cache,
and match the oracle."""
import numpy as np
import pytest

from chunk_wise_sparse_amd import hils, synth
import test_gpu_decode as TD
from test_gpu_gqa import _split

pytestmark = pytest.mark.gpu


def _paginate(kc, vc, n_chunks, spare, seed, C=64):
    """Pools [pages, Hk, C, d] holding every (sequence, chunk) of kc / vc [B, Hk, Lmax, d] at a
    random page (plus `spare` unused pages), and the block table [B, n_chunks]."""
    B, Hk, Lm, d = kc.shape
    pages = B * n_chunks + spare
    perm = np.random.default_rng(seed).permutation(pages)[:B * n_chunks].reshape(B, n_chunks)
    kp = np.zeros((pages, Hk, C, d), np.float32)
    vp = np.zeros((pages, Hk, C, d), np.float32)
    for b in range(B):
        for j in range(n_chunks):
            rows = min(C, Lm - C * j)
            kp[perm[b, j], :, :rows] = kc[b, :, C * j:C * j + rows]
            vp[perm[b, j], :, :rows] = vc[b, :, C * j:C * j + rows]
    return kp, vp, perm.astype(np.int32)


CASES = [
    (synth.DecodeConfig("paged_bf16", 3, 4, 3000, 128, 64, 8, "bf16", 16, 256, kv_len=(3000, 1999, 64)), 1),
    (synth.DecodeConfig("paged_fp32_gqa", 2, 4, 1500, 64, 64, 4, "fp32", 8, 128, kv_len=(1500, 700)), 2),
    # 256 (sequence, head) pairs: the fused single-kernel step, with grouped-query heads
    (synth.DecodeConfig("paged_fused_gqa", 8, 32, 4096, 128, 64, 16, "bf16", 16, 256,
                        kv_len=(4096, 4000, 3333, 2048, 1500, 777, 130, 64)), 4),
    # chunks of 128 and 32 keys: pages of C rows under the split attention
    (synth.DecodeConfig("paged_c128_bf16", 3, 4, 3000, 128, 128, 8, "bf16", 16, 256, kv_len=(3000, 1999, 129)), 1),
    (synth.DecodeConfig("paged_c32_fp32_gqa", 2, 4, 1500, 64, 32, 4, "fp32", 8, 128, kv_len=(1500, 700)), 2),
    (synth.DecodeConfig("paged_c32_bf16_many", 8, 32, 2000, 128, 32, 16, "bf16", 16, 256,
                        kv_len=(2000, 1999, 1000, 33, 32, 31, 1, 1500)), 1),
]


@pytest.mark.parametrize("cfg,G", CASES, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_decode_paged_matches_contiguous(lib, cfg, G):
    print(f"[case] paged decode G={G} {cfg}", flush=True)
    torch = TD._torch()
    inp = synth.make_decode_inputs_np(cfg)
    sub, full = _split(inp, G, ("k_cache", "v_cache", "lmk")) if G > 1 else (inp, inp)
    dev = TD._to_dev(sub, cfg.dtype)
    o_c, idx_c, w_c = hils.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["lmk"], dev["kv_len"], dev.get("h"),
                                  dev.get("w_down"), dev.get("w_up"), topk=cfg.topk, chunk=cfg.chunk,
                                  return_selection=True)
    n_chunks = -(-cfg.max_kv_len // cfg.chunk)
    kp, vp, table = _paginate(sub["k_cache"], sub["v_cache"], n_chunks, spare=5, seed=41, C=cfg.chunk)
    dt = dev["q"].dtype
    kpd = torch.from_numpy(kp).to("cuda", dt)
    vpd = torch.from_numpy(vp).to("cuda", dt)
    tbl = torch.from_numpy(table).to("cuda")
    o_p, idx_p, w_p = hils.decode(dev["q"], kpd, vpd, dev["lmk"], dev["kv_len"], dev.get("h"), dev.get("w_down"),
                                  dev.get("w_up"), topk=cfg.topk, chunk=cfg.chunk, return_selection=True,
                                  block_table=tbl, max_kv_len=cfg.max_kv_len)
    torch.cuda.synchronize()
    assert torch.equal(idx_c, idx_p) and torch.equal(w_c, w_p)
    assert torch.equal(o_c, o_p)
    pairs = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    if len(pairs) > 64:
        rng = np.random.default_rng(43)
        pairs = [pairs[i] for i in sorted(rng.choice(len(pairs), 32, replace=False))]
    TD._compare(full, cfg, o_p, idx_p, w_p, pairs)
