"""The forced-local-chunk option (the query's own chunk always selected) in prefill and decode,
through the C ABI, against the oracle's forced selection; the own chunk ranks first for the
near-tie band, its real score feeds the weights."""
import math

import numpy as np
import pytest

from chunk_wise_sparse_amd import synth
from oracle import hils_oracle as O
from parity import assert_within, check_rows
from test_gpu_prefill import _to_dev, _torch
import test_gpu_decode as TD

pytestmark = pytest.mark.gpu


def _ranked(res, own):
    for key, r in res.items():
        rs = np.array(r["sigma"], dtype=np.float64)
        rs[own(key)] = np.inf
        r["rank_sigma"] = rs
    return res


@pytest.mark.parametrize("cfg", [
    synth.PrefillConfig("local_bf16_k8", 1, 2, 4096, 128, 64, 8, "bf16", 16, 256, q_mode="walk"),
    synth.PrefillConfig("local_bf16_k48", 1, 2, 4096, 64, 64, 48, "bf16", 8, 128),
    synth.PrefillConfig("local_fp32_k4", 1, 2, 2048, 64, 64, 4, "fp32", 8, 128),
    synth.PrefillConfig("local_bf16_k1", 1, 2, 1024, 128, 64, 1, "bf16", 0, 0),
], ids=lambda c: c.name)
def test_prefill_force_local(lib, cfg):
    from chunk_wise_sparse_amd import hils
    import oracle_pool
    torch = _torch()
    print(f"[case] prefill force_local {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    dev = _to_dev(inp, cfg.dtype)
    o, idx, w = hils.prefill(dev["q"], dev["k"], dev["v"], dev["lmk"], dev.get("h"), dev.get("w_down"),
                             dev.get("w_up"), topk=cfg.topk, return_selection=True, force_local=True)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    for i in range(cfg.seq_len):               # the own chunk is in every row
        assert np.all(np.any(idx_np[:, :, i] == i // 64, axis=-1)), i
    rows = [(0, h, i) for h in range(cfg.heads) for i in range(0, cfg.seq_len, 3)]
    res = _ranked(oracle_pool.prefill_rows(inp, rows, cfg.chunk, cfg.topk, cfg.dtype, force_local=True),
                  lambda key: key[2] // 64)
    o_np, w_np = o.float().cpu().numpy(), w.cpu().numpy()
    stats = check_rows(res, {r: o_np[r] for r in res}, {r: idx_np[r] for r in res}, {r: w_np[r] for r in res},
                       cfg.dtype, lambda key: (inp["q"][key], inp["k"][key[0], key[1]], inp["v"][key[0], key[1]]),
                       cfg.chunk, 1.0 / math.sqrt(cfg.head_dim))
    print(f"[parity] {cfg.name}: {stats}", flush=True)
    assert_within(stats, cfg.dtype)


@pytest.mark.parametrize("cfg", [
    synth.DecodeConfig("local_fp32_ragged", 3, 2, 3000, 64, 64, 4, "fp32", 8, 128, kv_len=(3000, 700, 65)),
    synth.DecodeConfig("local_bf16_pairs256", 4, 64, 3000, 128, 64, 16, "bf16", 16, 256, kv_len=(3000, 1, 2047, 130)),
    synth.DecodeConfig("local_bf16_long", 1, 2, 600000, 64, 64, 64, "bf16", 8, 128, kv_len=(599937,), needles=4),
], ids=lambda c: c.name)
def test_decode_force_local(lib, cfg):
    from chunk_wise_sparse_amd import hils
    torch = _torch()
    print(f"[case] decode force_local {cfg}", flush=True)
    inp = synth.make_decode_inputs_np(cfg)
    dev = TD._to_dev(inp, cfg.dtype)
    o, idx, w = hils.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["lmk"], dev["kv_len"], dev.get("h"),
                            dev.get("w_down"), dev.get("w_up"), topk=cfg.topk, return_selection=True,
                            force_local=True)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)][:64]
    res = O.decode(inp, cfg.chunk, cfg.topk, cfg.dtype, pairs=pairs, force_local=True)
    res = _ranked(res, lambda key: (int(inp["kv_len"][key[0]]) - 1) // 64)
    o_np, idx_np, w_np = o.float().cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    for (b, h) in pairs:
        assert (int(inp["kv_len"][b]) - 1) // 64 in set(idx_np[b, h]), (b, h)
    stats = check_rows(res, {p: o_np[p] for p in res}, {p: idx_np[p] for p in res}, {p: w_np[p] for p in res},
                       cfg.dtype, lambda p: (inp["q"][p], inp["k_cache"][p], inp["v_cache"][p]), cfg.chunk,
                       1.0 / math.sqrt(cfg.head_dim), row_pos=lambda p: int(inp["kv_len"][p[0]]) - 1)
    print(f"[parity] {cfg.name}: {stats}", flush=True)
    assert_within(stats, cfg.dtype)
