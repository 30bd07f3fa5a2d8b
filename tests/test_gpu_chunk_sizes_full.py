"""Chunk sizes 32 and 128 at full size, in the launch configuration bench.py times: the 32K prefill
workload at C = 32 and 128 (sampled rows of every head against the oracle), and the decode batch of
the 512K workload at C = 128 and of its first 256K tokens at C = 32 (landmarks made for the chunk
size by the workloads' recipe; sampled (sequence, head) pairs against the oracle)."""
import dataclasses

import numpy as np
import pytest

from chunk_wise_sparse_amd import synth
from parity import sample_rows
import test_gpu_decode as TD
import test_gpu_prefill as TP

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("C", [32, 128])
def test_prefill_32k_chunk_size_sampled(lib, C):
    torch = TP._torch()
    cfg = dataclasses.replace(synth.CONFIGS["prefill_32k"], chunk=C, name=f"prefill_32k_chunk{C}")
    print(f"[case] full size {cfg}", flush=True)
    dev = synth.make_prefill_inputs_torch(cfg, "cuda")
    o, idx, w = TP._run(lib, dev, cfg, chunk=C)
    torch.cuda.synchronize()
    rows = sample_rows(cfg.batch, cfg.heads, cfg.seq_len, 40, seed=13, chunk=C)
    inp = {key: dev[key].float().cpu().numpy() for key in ("q", "k", "v", "lmk")}
    pos = sorted({r[2] for r in rows})
    h_full = np.zeros((cfg.batch, cfg.seq_len, cfg.hidden), dtype=np.float32)
    h_full[:, pos] = dev["h"][:, pos].float().cpu().numpy()
    inp["h"] = h_full
    inp["w_down"] = dev["w_down"].float().cpu().numpy()
    inp["w_up"] = dev["w_up"].float().cpu().numpy()
    TP._compare(inp, cfg, o, idx, w, rows)


def test_decode_chunk_sizes_sampled(lib):
    from chunk_wise_sparse_amd import hils
    torch = TP._torch()
    base = synth.CONFIGS["decode_512k"]
    print(f"[case] full size {base}", flush=True)
    D = synth.make_decode_inputs_torch(base, "cuda")
    for C, L in ((128, base.max_kv_len), (32, base.max_kv_len // 2)):
        cfg = dataclasses.replace(base, chunk=C, max_kv_len=L, kv_len=(L,) * base.batch, needles=0,
                                  name=f"decode_chunk{C}")
        print(f"[case] chunk {C}, kv_len {L}", flush=True)
        kc = D["k_cache"] if L == base.max_kv_len else D["k_cache"][:, :, :L].contiguous()
        vc = D["v_cache"] if L == base.max_kv_len else D["v_cache"][:, :, :L].contiguous()
        lmk = synth.chunk_landmarks_dev(kc, C, base.seed)
        kvl = torch.full_like(D["kv_len"], L)
        o, idx, w = hils.decode(D["q"], kc, vc, lmk, kvl, D["h"], D["w_down"], D["w_up"], topk=cfg.topk,
                                chunk=C, return_selection=True)
        torch.cuda.synchronize()
        # 8 pairs: every sequence, one head each, spread over the heads
        pairs = [(b, (7 * b + C) % cfg.heads) for b in range(cfg.batch)]
        d = kc.shape[-1]
        for (b, h) in pairs:
            sub = {"q": D["q"][b:b + 1, h:h + 1].float().cpu().numpy(),
                   "h": D["h"][b:b + 1].float().cpu().numpy(),
                   "w_down": D["w_down"].float().cpu().numpy(),
                   "w_up": D["w_up"][h * d:(h + 1) * d].float().cpu().numpy(),
                   "kv_len": np.asarray([L], np.int32),
                   "lmk": lmk[b:b + 1, h:h + 1].float().cpu().numpy(),
                   "k_cache": kc[b:b + 1, h:h + 1].float().cpu().numpy(),
                   "v_cache": vc[b:b + 1, h:h + 1].float().cpu().numpy()}
            TD._compare(sub, cfg, o[b:b + 1, h:h + 1], idx[b:b + 1, h:h + 1], w[b:b + 1, h:h + 1], [(0, 0)])
        del kc, vc, lmk, o, idx, w
        torch.cuda.empty_cache()
