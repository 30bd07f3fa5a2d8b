"""Chunk sizes 32 and 128 in prefill and decode, through the C ABI, against the oracle: every row
of small prefills (ragged last chunk, GQA, forced local chunk), and ragged decode batches.  bf16
prefills select with the MFMA kernel when the sequence is whole 64-query tiles (else in the
generic kernel; the forced local chunk amends the MFMA selection in a post-pass, and the generic
selection takes it directly) and attend in the chunk-major MFMA kernels (several
work items per chunk, partial last chunks read with clamped rows); fp32 prefills run the
generic kernel.  Decode steps at these sizes take the 64-key path's landmark scan and selection
and a split attention over C-key chunks."""
import math

import numpy as np
import pytest

from chunk_wise_sparse_amd import synth
from oracle import hils_oracle as O
from parity import assert_within, check_rows, sample_rows
import test_gpu_decode as TD
import test_gpu_prefill as TP
from test_gpu_gqa import _split

pytestmark = pytest.mark.gpu


def _ranked(res, own):
    for key, r in res.items():
        rs = np.array(r["sigma"], dtype=np.float64)
        rs[own(key)] = np.inf
        r["rank_sigma"] = rs
    return res


PREFILL = [
    # (config, kv-head group size G, forced local chunk)
    (synth.PrefillConfig("c32_bf16_d128_L1000", 1, 2, 1000, 128, 32, 8, "bf16", 16, 256), 1, False),
    (synth.PrefillConfig("c32_bf16_d64_k64", 1, 2, 4096, 64, 32, 64, "bf16", 8, 128), 1, False),
    (synth.PrefillConfig("c32_fp32_d64_noqcal", 2, 2, 333, 64, 32, 3, "fp32", 0, 0), 1, False),
    (synth.PrefillConfig("c128_fp32_d64_L777", 1, 2, 777, 64, 128, 4, "fp32", 8, 128), 1, False),
    (synth.PrefillConfig("c128_bf16_d128_walk", 1, 2, 4096, 128, 128, 8, "bf16", 32, 512, q_mode="walk"),
     1, False),
    (synth.PrefillConfig("c128_bf16_d128_g4", 1, 8, 2048, 128, 128, 4, "bf16", 16, 256), 4, False),
    (synth.PrefillConfig("c32_bf16_d128_local", 1, 2, 2048, 128, 32, 8, "bf16", 16, 256), 1, True),
    (synth.PrefillConfig("c128_fp32_d64_local", 1, 2, 1500, 64, 128, 3, "fp32", 8, 128), 1, True),
    # the 32K workload's shape (d = 64, k = 16, r = 16) at a ragged length: chunks chosen by
    # hundreds of rows (several chunk-major work items each)
    (synth.PrefillConfig("c32_bf16_d64_k16_L3333", 1, 4, 3333, 64, 32, 16, "bf16", 16, 256), 1, False),
    (synth.PrefillConfig("c128_bf16_d64_k16_L5000", 2, 2, 5000, 64, 128, 16, "bf16", 16, 256), 1, False),
    (synth.PrefillConfig("c128_bf16_d128_k64_L9000", 1, 1, 9000, 128, 128, 64, "bf16", 0, 0), 1, False),
    # whole 64-query tiles: the MFMA selection (tiles scored against their last row's candidates,
    # the first half of a C = 32 tile masking one more landmark), with and without its bound pass
    (synth.PrefillConfig("c32_bf16_d64_k16_L8192", 1, 2, 8192, 64, 32, 16, "bf16", 16, 256), 1, False),
    (synth.PrefillConfig("c32_bf16_d128_k32_walk", 1, 2, 4096, 128, 32, 32, "bf16", 32, 512, q_mode="walk"),
     1, False),
    (synth.PrefillConfig("c128_bf16_d128_k16_r12_L16384", 1, 1, 16384, 128, 128, 16, "bf16", 12, 256), 1, False),
    (synth.PrefillConfig("c128_bf16_d64_L2368", 1, 2, 2368, 64, 128, 8, "bf16", 8, 128), 1, False),
    (synth.PrefillConfig("c32_bf16_d64_k40_L2368", 1, 2, 2368, 64, 32, 40, "bf16", 8, 128), 1, False),
    (synth.PrefillConfig("c32_bf16_d128_g2_L3072", 1, 4, 3072, 128, 32, 8, "bf16", 16, 256), 2, False),
    # forced local chunk: the MFMA selection amended by the post-pass, and (ragged) the generic one
    (synth.PrefillConfig("c128_bf16_d64_local_L4096", 1, 2, 4096, 64, 128, 4, "bf16", 8, 128), 1, True),
    (synth.PrefillConfig("c32_bf16_d64_local_L999", 1, 2, 999, 64, 32, 6, "bf16", 8, 128), 1, True),
    # one 64-query tile: a single partial 128-key chunk, and two 32-key chunks with k = 1
    (synth.PrefillConfig("c128_bf16_d128_L64", 2, 2, 64, 128, 128, 4, "bf16", 8, 128), 1, False),
    (synth.PrefillConfig("c32_bf16_d64_L64_k1", 1, 3, 64, 64, 32, 1, "bf16", 8, 128), 1, False),
]


@pytest.mark.parametrize("cfg,G,local", PREFILL, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_prefill_chunk_size(lib, cfg, G, local):
    import oracle_pool
    print(f"[case] prefill chunk={cfg.chunk} G={G} local={local} {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    sub, full = _split(inp, G, ("k", "v", "lmk")) if G > 1 else (inp, inp)
    o, idx, w = TP._run(lib, TP._to_dev(sub, cfg.dtype), cfg, chunk=cfg.chunk, force_local=local)
    TP._torch().cuda.synchronize()
    C = cfg.chunk
    idx_np = idx.cpu().numpy()
    for i in range(cfg.seq_len):
        sel = idx_np[:, :, i]
        nsel = min(cfg.topk, i // C + 1)
        assert np.all((sel[..., :nsel] >= 0) & (sel[..., :nsel] <= i // C)), i
        assert np.all(sel[..., nsel:] == -1), i
        if local:
            assert np.all(np.any(sel == i // C, axis=-1)), i
    rows = [(b, h, i) for b in range(cfg.batch) for h in range(cfg.heads) for i in range(cfg.seq_len)]
    if len(rows) > 6000:
        rows = sample_rows(cfg.batch, cfg.heads, cfg.seq_len, 1024, seed=41)
    if not local:
        TP._compare(full, cfg, o, idx, w, rows)
        return
    res = _ranked(oracle_pool.prefill_rows(full, rows, C, cfg.topk, cfg.dtype, force_local=True),
                  lambda key: key[2] // C)
    o_np, w_np = o.float().cpu().numpy(), w.cpu().numpy()
    stats = check_rows(res, {r: o_np[r] for r in res}, {r: idx_np[r] for r in res}, {r: w_np[r] for r in res},
                       cfg.dtype, lambda key: (full["q"][key], full["k"][key[0], key[1]], full["v"][key[0], key[1]]),
                       C, 1.0 / math.sqrt(cfg.head_dim))
    print(f"[parity] {cfg.name}: {stats}", flush=True)
    assert_within(stats, cfg.dtype)


DECODE = [
    (synth.DecodeConfig("c32_dec_fp32_ragged", 3, 2, 3000, 64, 32, 4, "fp32", 8, 128, kv_len=(3000, 1500, 1)),
     1, False),
    (synth.DecodeConfig("c32_dec_bf16_d128_k64", 2, 4, 8000, 128, 32, 64, "bf16", 32, 512, kv_len=(8000, 2049)),
     1, False),
    (synth.DecodeConfig("c128_dec_bf16_needles", 2, 4, 30000, 64, 128, 16, "bf16", 16, 256,
                        kv_len=(30000, 29937), needles=4), 1, False),
    (synth.DecodeConfig("c128_dec_bf16_g4", 2, 8, 5000, 128, 128, 8, "bf16", 16, 256, kv_len=(5000, 129)), 4, False),
    (synth.DecodeConfig("c32_dec_bf16_local", 3, 2, 4000, 128, 32, 8, "bf16", 16, 256, kv_len=(4000, 31, 33)),
     1, True),
    (synth.DecodeConfig("c128_dec_fp32_local", 2, 2, 3000, 64, 128, 4, "fp32", 0, 0, kv_len=(3000, 700)), 1, True),
    # more than 8192 chunks: dense scores and the radix selection instead of candidate lists
    (synth.DecodeConfig("c32_dec_bf16_dense_scores", 2, 2, 300000, 64, 32, 16, "bf16", 8, 128,
                        kv_len=(300000, 262177)), 1, False),
    # fp32 past 8192 chunks (dense scores, radix selection)
    (synth.DecodeConfig("c32_dec_fp32_dense_scores", 1, 2, 290000, 64, 32, 8, "fp32", 8, 128,
                        kv_len=(289999,)), 1, False),
    # one key in the last chunk, a cache of exactly one chunk, and k above the candidates
    (synth.DecodeConfig("c128_dec_bf16_short", 3, 2, 1000, 128, 128, 12, "bf16", 16, 256, kv_len=(897, 128, 1)),
     1, False),
]


@pytest.mark.parametrize("cfg,G,local", DECODE, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_decode_chunk_size(lib, cfg, G, local):
    from chunk_wise_sparse_amd import hils
    print(f"[case] decode chunk={cfg.chunk} G={G} local={local} {cfg}", flush=True)
    inp = synth.make_decode_inputs_np(cfg)
    sub, full = _split(inp, G, ("k_cache", "v_cache", "lmk")) if G > 1 else (inp, inp)
    dev = TD._to_dev(sub, cfg.dtype)
    o, idx, w = hils.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["lmk"], dev["kv_len"], dev.get("h"),
                            dev.get("w_down"), dev.get("w_up"), topk=cfg.topk, chunk=cfg.chunk,
                            return_selection=True, force_local=local)
    TD._torch().cuda.synchronize()
    C = cfg.chunk
    pairs = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    res = O.decode(full, C, cfg.topk, cfg.dtype, pairs=pairs, force_local=local)
    if local:
        res = _ranked(res, lambda key: (int(inp["kv_len"][key[0]]) - 1) // C)
    o_np, idx_np, w_np = o.float().cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    for (b, h) in pairs:
        own = (int(inp["kv_len"][b]) - 1) // C
        nsel = min(cfg.topk, own + 1)
        assert np.all(idx_np[b, h, nsel:] == -1), (b, h)
        if local:
            assert own in set(idx_np[b, h]), (b, h)
    stats = check_rows(res, {p: o_np[p] for p in res}, {p: idx_np[p] for p in res}, {p: w_np[p] for p in res},
                       cfg.dtype, lambda p: (full["q"][p], full["k_cache"][p], full["v_cache"][p]), C,
                       1.0 / math.sqrt(cfg.head_dim), row_pos=lambda p: int(inp["kv_len"][p[0]]) - 1)
    print(f"[parity] {cfg.name}: {stats['n_rows']} (b,h), max|do| {stats['max_abs']:.3g}, "
          f"max|dw| {stats['max_w']:.3g}, near-tie swaps {stats['n_diff_sel']}", flush=True)
    assert_within(stats, cfg.dtype)


@pytest.mark.parametrize("C", [32, 128])
def test_prefill_chunk_size_ignores_mode_and_q_tile(lib, C):
    """attn_mode and q_tile leave chunk sizes 32 and 128 on their one path: bitwise equal results."""
    from chunk_wise_sparse_amd import hils
    cfg = synth.PrefillConfig(f"c{C}_modes", 1, 2, 2048, 128, C, 8, "bf16", 16, 256)
    print(f"[case] modes chunk={C} {cfg}", flush=True)
    dev = TP._to_dev(synth.make_prefill_inputs_np(cfg), cfg.dtype)
    ref = TP._run(lib, dev, cfg, chunk=C)
    for kw in (dict(attn_mode=hils.ATTN_UNION), dict(attn_mode=hils.ATTN_AUTO), dict(q_tile=16)):
        got = TP._run(lib, dev, cfg, chunk=C, **kw)
        TP._torch().cuda.synchronize()
        for a, b in zip(ref, got):
            assert TP._torch().equal(a, b), kw


@pytest.mark.parametrize("C", [32, 128])
def test_chunk_size_selection_in_workspace(lib, C):
    """With the selection kept in the workspace (no idx / w outputs) prefill and decode give
    bitwise the same output as with the selection returned."""
    from chunk_wise_sparse_amd import hils
    torch = TP._torch()
    cfg = synth.PrefillConfig(f"c{C}_ws", 1, 2, 2048, 64, C, 8, "bf16", 16, 256)
    print(f"[case] selection in workspace, chunk={C}", flush=True)
    dev = TP._to_dev(synth.make_prefill_inputs_np(cfg), cfg.dtype)
    o_sel, _, _ = TP._run(lib, dev, cfg, chunk=C)
    o_ws = hils.prefill(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["h"], dev["w_down"], dev["w_up"],
                        topk=cfg.topk, chunk=C)
    dcfg = synth.DecodeConfig(f"c{C}_dec_ws", 2, 4, 3000, 128, C, 8, "bf16", 16, 256, kv_len=(3000, 777))
    dd = TD._to_dev(synth.make_decode_inputs_np(dcfg), dcfg.dtype)
    args = (dd["q"], dd["k_cache"], dd["v_cache"], dd["lmk"], dd["kv_len"], dd["h"], dd["w_down"], dd["w_up"])
    od_sel, _, _ = hils.decode(*args, topk=dcfg.topk, chunk=C, return_selection=True)
    od_ws = hils.decode(*args, topk=dcfg.topk, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o_sel, o_ws)
    assert torch.equal(od_sel, od_ws)
