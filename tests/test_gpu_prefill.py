"""Prefill on the GPU through the C ABI, element by element against the CPU oracle."""
import math

import numpy as np
import pytest

from chunk_wise_sparse_amd import synth
from oracle import hils_oracle as O
import oracle_pool
from parity import assert_within, check_rows, sample_rows

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    return torch


def _to_dev(inp, dtype):
    torch = _torch()
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda", dt) for k, v in inp.items()}


def _run(lib, dev, cfg, **kw):
    from chunk_wise_sparse_amd import hils
    return hils.prefill(dev["q"], dev["k"], dev["v"], dev["lmk"], dev.get("h"), dev.get("w_down"),
                        dev.get("w_up"), topk=cfg.topk, return_selection=True, **kw)


def _compare(inp, cfg, o, idx, w, rows, scale=None):
    s = (1.0 / math.sqrt(cfg.head_dim)) if scale is None else scale
    res = oracle_pool.prefill_rows(inp, rows, cfg.chunk, cfg.topk, cfg.dtype, scale=scale)
    rset = sorted(res)
    bi = np.array([r[0] for r in rset]); hi = np.array([r[1] for r in rset]); ii = np.array([r[2] for r in rset])
    import torch
    o_np = o.float()[bi, hi, ii].cpu().numpy()
    idx_np = idx[bi, hi, ii].cpu().numpy()
    w_np = w[bi, hi, ii].cpu().numpy()
    gpu_o = {key: o_np[t] for t, key in enumerate(rset)}
    gpu_idx = {key: idx_np[t] for t, key in enumerate(rset)}
    gpu_w = {key: w_np[t] for t, key in enumerate(rset)}
    stats = check_rows(res, gpu_o, gpu_idx, gpu_w, cfg.dtype,
                       lambda key: (inp["q"][key[0], key[1], key[2]], inp["k"][key[0], key[1]], inp["v"][key[0], key[1]]),
                       cfg.chunk, s)
    print(f"[parity] {cfg.name}: {stats['n_rows']} rows, max|do| {stats['max_abs']:.3g}, "
          f"mean|do| {stats['mean_abs']:.3g}, max|dw| {stats['max_w']:.3g}, near-tie swaps {stats['n_diff_sel']}",
          flush=True)
    assert_within(stats, cfg.dtype)
    return stats


SMALL = [
    synth.CONFIGS["tiny_fp32"],
    synth.PrefillConfig("bf16_d128_k8", 2, 2, 1024, 128, 64, 8, "bf16", 16, 256),
    synth.PrefillConfig("bf16_d64_allchunks", 1, 2, 2048, 64, 64, 64, "bf16", 4, 128),
    synth.PrefillConfig("bf16_d128_noqcal", 1, 3, 640, 128, 64, 3, "bf16", 0, 0),
    synth.PrefillConfig("fp32_d128_k1", 1, 1, 512, 128, 64, 1, "fp32", 64, 128),
    # the selection's Q-Cal forms at d = 128: rank above 32 (four 16-wide steps) and a rank that
    # is not a multiple of 8 (element-wise loads)
    synth.PrefillConfig("bf16_d128_r40", 1, 2, 2048, 128, 64, 16, "bf16", 40, 256),
    synth.PrefillConfig("bf16_d128_r12_k40", 1, 2, 2048, 128, 64, 40, "bf16", 12, 256),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_prefill_all_rows(lib, cfg):
    print(f"[case] prefill all rows {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    dev = _to_dev(inp, cfg.dtype)
    o, idx, w = _run(lib, dev, cfg)
    _torch().cuda.synchronize()
    rows = [(b, h, i) for b in range(cfg.batch) for h in range(cfg.heads) for i in range(cfg.seq_len)]
    _compare(inp, cfg, o, idx, w, rows)


def test_prefill_two_pass_selection(lib):
    """More than 128 candidate chunks: the lower-bound pass and the buffered exact top-k."""
    cfg = synth.PrefillConfig("bf16_16k_k32", 1, 2, 16384, 128, 64, 32, "bf16", 32, 512)
    print(f"[case] {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    o, idx, w = _run(lib, _to_dev(inp, cfg.dtype), cfg)
    _compare(inp, cfg, o, idx, w, sample_rows(1, 2, cfg.seq_len, 160, seed=1))


def test_prefill_ragged_tile_groups(lib):
    """203 chunks: the last group of eight 64-query tiles has five idle waves, and the long
    tiles take the lower-bound pass; rows of the first three chunks (the short group) are all
    checked."""
    cfg = synth.PrefillConfig("bf16_203chunks_k32", 1, 2, 64 * 203, 128, 64, 32, "bf16", 16, 256)
    print(f"[case] {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    o, idx, w = _run(lib, _to_dev(inp, cfg.dtype), cfg)
    rows = sample_rows(1, 2, cfg.seq_len, 96, seed=6)
    rows = sorted(set(rows) | {(0, h, i) for h in range(2) for i in range(0, 3 * 64, 5)})
    _compare(inp, cfg, o, idx, w, rows)


def test_prefill_two_pass_k64(lib):
    cfg = synth.PrefillConfig("bf16_16k_k64", 1, 1, 16384, 64, 64, 64, "bf16", 8, 128)
    print(f"[case] {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    o, idx, w = _run(lib, _to_dev(inp, cfg.dtype), cfg)
    _compare(inp, cfg, o, idx, w, sample_rows(1, 1, cfg.seq_len, 200, seed=2))


def test_prefill_ties_overflow(lib):
    """Every landmark identical: all scores tie, so every chunk passes the bound, the buffer
    overflows and is cut, and the selection must be the k smallest chunk indices."""
    cfg = synth.PrefillConfig("ties", 1, 2, 12288, 128, 64, 16, "bf16", 0, 0)
    print(f"[case] {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    inp["lmk"][:] = inp["lmk"][:, :, :1]
    o, idx, w = _run(lib, _to_dev(inp, cfg.dtype), cfg)
    idx_np = idx.cpu().numpy()
    for i in (0, 63, 64, 1023, 1024, 5000, 12287):
        keff = min(16, i // 64 + 1)
        assert list(idx_np[0, 0, i, :keff]) == list(range(keff)), (i, idx_np[0, 0, i])
    _compare(inp, cfg, o, idx, w, sample_rows(1, 2, cfg.seq_len, 64, seed=3))


def test_prefill_grouped_ties(lib):
    """Landmarks drawn from three distinct rows: large groups of exactly equal scores."""
    cfg = synth.PrefillConfig("group_ties", 1, 2, 10240, 64, 64, 24, "fp32", 8, 128)
    print(f"[case] {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    g = np.random.default_rng(5)
    pick = g.integers(0, 3, size=inp["lmk"].shape[2])
    inp["lmk"] = np.ascontiguousarray(inp["lmk"][:, :, pick])
    o, idx, w = _run(lib, _to_dev(inp, cfg.dtype), cfg)
    _compare(inp, cfg, o, idx, w, sample_rows(1, 2, cfg.seq_len, 96, seed=4))


def test_prefill_deterministic(lib):
    cfg = SMALL[1]
    inp = synth.make_prefill_inputs_np(cfg)
    dev = _to_dev(inp, cfg.dtype)
    a = _run(lib, dev, cfg)
    b = _run(lib, dev, cfg)
    torch = _torch()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_prefill_without_selection_output(lib):
    """idx/w kept in the workspace gives the same o."""
    from chunk_wise_sparse_amd import hils
    cfg = SMALL[1]
    dev = _to_dev(synth.make_prefill_inputs_np(cfg), cfg.dtype)
    o1, _, _ = _run(lib, dev, cfg)
    o2 = hils.prefill(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["h"], dev["w_down"], dev["w_up"], topk=cfg.topk)
    assert _torch().equal(o1, o2)


@pytest.mark.parametrize("name,per_head", [("prefill_32k", 48), ("prefill_128k", 64)])
def test_prefill_full_size_sampled(lib, name, per_head):
    """Full-size workloads in the launch configuration the benchmark times; sampled rows."""
    torch = _torch()
    cfg = synth.CONFIGS[name]
    print(f"[case] full size {cfg}", flush=True)
    dev = synth.make_prefill_inputs_torch(cfg, "cuda")
    o, idx, w = _run(lib, dev, cfg)
    torch.cuda.synchronize()
    rows = sample_rows(cfg.batch, cfg.heads, cfg.seq_len, per_head, seed=7)
    inp = {key: dev[key].float().cpu().numpy() for key in ("q", "k", "v", "lmk")}
    if cfg.qcal_rank:
        pos = sorted({r[2] for r in rows})
        h_full = np.zeros((cfg.batch, cfg.seq_len, cfg.hidden), dtype=np.float32)
        h_full[:, pos] = dev["h"][:, pos].float().cpu().numpy()
        inp["h"] = h_full
        inp["w_down"] = dev["w_down"].float().cpu().numpy()
        inp["w_up"] = dev["w_up"].float().cpu().numpy()
    _compare(inp, cfg, o, idx, w, rows)


@pytest.mark.parametrize("name", ["prefill_512k_walk", "prefill_512k_iid"])
def test_prefill_512k_sampled(lib, name):
    """The 512K-token prefill (k = 64) in the benchmark's launch configuration: 8 fixed and 32
    random rows of each of eight heads against the oracle (only those heads are copied back)."""
    torch = _torch()
    cfg = synth.CONFIGS[name]
    print(f"[case] full size {cfg}", flush=True)
    dev = synth.make_prefill_inputs_torch(cfg, "cuda")
    o, idx, w = _run(lib, dev, cfg)
    torch.cuda.synchronize()
    heads = [0, 4, 9, 13, 18, 22, 27, cfg.heads - 1]
    d = cfg.head_dim
    rows = sample_rows(1, len(heads), cfg.seq_len, 32, seed=11)
    sub = {key: dev[key][:, heads].float().cpu().numpy() for key in ("q", "k", "v", "lmk")}
    pos = sorted({r[2] for r in rows})
    h_sub = np.zeros((1, cfg.seq_len, cfg.hidden), dtype=np.float32)
    h_sub[:, pos] = dev["h"][:, pos].float().cpu().numpy()
    sub["h"] = h_sub
    sub["w_down"] = dev["w_down"].float().cpu().numpy()
    sub["w_up"] = np.concatenate([dev["w_up"][hh * d:(hh + 1) * d].float().cpu().numpy() for hh in heads])
    sub_cfg = synth.PrefillConfig(cfg.name, 1, len(heads), cfg.seq_len, d, cfg.chunk, cfg.topk, cfg.dtype,
                                  cfg.qcal_rank, cfg.hidden)
    _compare(sub, sub_cfg, o[:, heads], idx[:, heads], w[:, heads], rows)


# fp32 dispatch branches: the two-block kernel with 4 waves and 64 list entries (d = 64 with
# k > 32 or L % 256 != 0), with 2 waves (d = 64 with L % 128 != 0; d = 128 always), and the
# generic selection kernel's k > 32 form.  Every row is compared.
FP32_BRANCHES = [
    synth.PrefillConfig("fp32_d64_k40", 1, 1, 3072, 64, 64, 40, "fp32", 8, 128),
    synth.PrefillConfig("fp32_d64_k64", 1, 1, 4608, 64, 64, 64, "fp32", 8, 128),
    synth.PrefillConfig("fp32_d128_k40", 1, 1, 3072, 128, 64, 40, "fp32", 8, 128),
    synth.PrefillConfig("fp32_d128_k64", 1, 1, 4608, 128, 64, 64, "fp32", 0, 0),
    synth.PrefillConfig("fp32_d64_L640", 1, 2, 640, 64, 64, 4, "fp32", 8, 128),
    synth.PrefillConfig("fp32_d64_L1152", 1, 2, 1152, 64, 64, 8, "fp32", 8, 128),
    synth.PrefillConfig("fp32_d64_L576", 1, 2, 576, 64, 64, 4, "fp32", 8, 128),
    synth.PrefillConfig("fp32_d64_L704", 2, 1, 704, 64, 64, 3, "fp32", 0, 0),
]


@pytest.mark.parametrize("cfg", FP32_BRANCHES, ids=lambda c: c.name)
def test_prefill_fp32_branches_all_rows(lib, cfg):
    print(f"[case] prefill all rows {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    o, idx, w = _run(lib, _to_dev(inp, cfg.dtype), cfg)
    _torch().cuda.synchronize()
    rows = [(b, h, i) for b in range(cfg.batch) for h in range(cfg.heads) for i in range(cfg.seq_len)]
    _compare(inp, cfg, o, idx, w, rows)


@pytest.mark.parametrize("cfg", [
    synth.PrefillConfig("qtile_bf16_k16", 1, 2, 4096, 128, 64, 16, "bf16", 16, 256, q_mode="walk"),
    synth.PrefillConfig("qtile_bf16_k48", 1, 2, 4096, 64, 64, 48, "bf16", 8, 128),
    synth.PrefillConfig("qtile_bf16_L576", 1, 1, 576, 128, 64, 4, "bf16", 0, 0),
    synth.PrefillConfig("qtile_fp32", 1, 1, 2048, 64, 64, 8, "fp32", 8, 128),
], ids=lambda c: c.name)
def test_prefill_q_tile_bitwise(lib, cfg):
    """The union group size (q_tile = 16, 32, 64, 128) changes which rows share a staged chunk,
    not any row's result: outputs and selections are bitwise identical.  One run is also checked
    against the oracle on every row."""
    torch = _torch()
    print(f"[case] q_tile sweep {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    dev = _to_dev(inp, cfg.dtype)
    runs = {qt: _run(lib, dev, cfg, q_tile=qt) for qt in (16, 32, 64, 128, 0)}
    torch.cuda.synchronize()
    ref = runs[128]
    for qt, r in runs.items():
        for x, y in zip(r, ref):
            assert torch.equal(x, y), f"q_tile {qt} differs from q_tile 128"
    rows = [(b, h, i) for b in range(cfg.batch) for h in range(cfg.heads) for i in range(cfg.seq_len)]
    _compare(inp, cfg, *runs[16], rows)


@pytest.mark.parametrize("cfg", [
    synth.PrefillConfig("partial_bf16_L1000", 1, 2, 1000, 128, 64, 4, "bf16", 16, 256),
    synth.PrefillConfig("partial_bf16_L2047_k48", 1, 2, 2047, 64, 64, 48, "bf16", 8, 128, q_mode="walk"),
    synth.PrefillConfig("partial_fp32_L777", 2, 1, 777, 64, 64, 5, "fp32", 8, 128),
    synth.PrefillConfig("partial_bf16_L33", 1, 2, 33, 128, 64, 2, "bf16", 0, 0),
], ids=lambda c: c.name)
def test_prefill_partial_last_chunk(lib, cfg):
    """seq_len not a multiple of the chunk: every row against the oracle, the selection written
    out or kept in the workspace (same o), and the union group size changing nothing."""
    from chunk_wise_sparse_amd import hils
    torch = _torch()
    print(f"[case] partial last chunk {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    dev = _to_dev(inp, cfg.dtype)
    o, idx, w = _run(lib, dev, cfg)
    o2 = hils.prefill(dev["q"], dev["k"], dev["v"], dev["lmk"], dev.get("h"), dev.get("w_down"), dev.get("w_up"),
                      topk=cfg.topk, q_tile=32)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    rows = [(b, h, i) for b in range(cfg.batch) for h in range(cfg.heads) for i in range(cfg.seq_len)]
    _compare(inp, cfg, o, idx, w, rows)
