"""Decode on the GPU through the C ABI against the CPU oracle; decode/prefill consistency."""
import math

import numpy as np
import pytest

from chunk_wise_sparse_amd import synth
from oracle import hils_oracle as O
from parity import assert_within, check_rows

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    return torch


def _to_dev(inp, dtype):
    torch = _torch()
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    out = {}
    for k, v in inp.items():
        if k == "needle_ids":
            continue
        if k == "kv_len":
            out[k] = torch.from_numpy(np.asarray(v, dtype=np.int32)).to("cuda")
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v)).to("cuda", dt)
    return out


def _run(dev, cfg):
    from chunk_wise_sparse_amd import hils
    return hils.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["lmk"], dev["kv_len"], dev.get("h"),
                       dev.get("w_down"), dev.get("w_up"), topk=cfg.topk, return_selection=True)


def _compare(inp, cfg, o, idx, w, pairs):
    s = 1.0 / math.sqrt(cfg.head_dim)
    res = O.decode(inp, cfg.chunk, cfg.topk, cfg.dtype, pairs=pairs)
    o_np, idx_np, w_np = o.float().cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    stats = check_rows(res, {p: o_np[p] for p in res}, {p: idx_np[p] for p in res}, {p: w_np[p] for p in res},
                       cfg.dtype, lambda p: (inp["q"][p], inp["k_cache"][p], inp["v_cache"][p]), cfg.chunk, s,
                       row_pos=lambda p: int(inp["kv_len"][p[0]]) - 1)
    print(f"[parity] {cfg.name}: {stats['n_rows']} (b,h), max|do| {stats['max_abs']:.3g}, "
          f"mean|do| {stats['mean_abs']:.3g}, max|dw| {stats['max_w']:.3g}, near-tie swaps {stats['n_diff_sel']}",
          flush=True)
    assert_within(stats, cfg.dtype)


SMALL = [
    synth.DecodeConfig("tiny_fp32_ragged", 3, 2, 1000, 64, 64, 4, "fp32", 8, 128, kv_len=(1000, 77, 1)),
    synth.DecodeConfig("bf16_d128_k64", 4, 3, 6000, 128, 64, 64, "bf16", 32, 512, kv_len=(6000, 4097, 64, 130)),
    synth.DecodeConfig("bf16_d64_needles", 2, 4, 30000, 64, 64, 16, "bf16", 16, 256, kv_len=(30000, 29937),
                       needles=4),
    synth.DecodeConfig("fp32_d128_noqcal", 2, 2, 9000, 128, 64, 7, "fp32", 0, 0, kv_len=(9000, 8999)),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_decode_all_pairs(lib, cfg):
    print(f"[case] decode {cfg}", flush=True)
    inp = synth.make_decode_inputs_np(cfg)
    o, idx, w = _run(_to_dev(inp, cfg.dtype), cfg)
    _torch().cuda.synchronize()
    pairs = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    _compare(inp, cfg, o, idx, w, pairs)
    if cfg.needles:
        got = idx.cpu().numpy()
        for b, h in pairs:
            assert set(inp["needle_ids"][b, h]) <= set(got[b, h]), (b, h)


def test_decode_matches_prefill_rows(lib):
    """decode with kv_len = i + 1 reproduces prefill row i (both on the GPU)."""
    torch = _torch()
    from chunk_wise_sparse_amd import hils
    cfg = synth.PrefillConfig("dp", 1, 2, 4096, 128, 64, 8, "bf16", 16, 256)
    inp = synth.make_prefill_inputs_np(cfg)
    dt = torch.bfloat16
    dev = {k: torch.from_numpy(v).to("cuda", dt) for k, v in inp.items()}
    o, idx, w = hils.prefill(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["h"], dev["w_down"], dev["w_up"],
                             topk=cfg.topk, return_selection=True)
    for i in (0, 63, 64, 1000, 4095):
        od, idd, wd = hils.decode(dev["q"][:, :, i].contiguous(), dev["k"], dev["v"], dev["lmk"],
                                  torch.tensor([i + 1], dtype=torch.int32, device="cuda"), dev["h"][:, i].contiguous(),
                                  dev["w_down"], dev["w_up"], topk=cfg.topk, return_selection=True)
        assert torch.equal(idd, idx[:, :, i]), i
        assert torch.allclose(wd, w[:, :, i], atol=1e-6, rtol=0), i
        assert (od.float() - o[:, :, i].float()).abs().max().item() <= 1.6e-2, i


def test_decode_full_size_sampled(lib):
    """The 512K-token decode step (8 sequences x 32 heads) in the benchmark's launch configuration:
    needle recall on every (sequence, head), oracle parity on 32 pairs."""
    torch = _torch()
    cfg = synth.CONFIGS["decode_512k"]
    print(f"[case] full size {cfg}", flush=True)
    dev = synth.make_decode_inputs_torch(cfg, "cuda")
    o, idx, w = _run(dev, cfg)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    needles = dev["needle_ids"]
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            assert set(needles[b, h]) <= set(got[b, h]), (b, h)
    # 32 pairs: every sequence, four heads each, spread over the heads
    pairs = [(b, (5 * b + 9 * t) % cfg.heads) for b in range(cfg.batch) for t in range(4)]
    inp = {"q": dev["q"].float().cpu().numpy(), "lmk": None, "kv_len": np.asarray(cfg.kv_len, np.int32),
           "h": dev["h"].float().cpu().numpy(), "w_down": dev["w_down"].float().cpu().numpy(),
           "w_up": dev["w_up"].float().cpu().numpy()}
    B, H, Lm, d = dev["k_cache"].shape
    for (b, h) in pairs:
        sub = dict(inp)
        sub["q"] = inp["q"][b:b + 1, h:h + 1]
        sub["h"] = inp["h"][b:b + 1]
        sub["w_up"] = inp["w_up"][h * d:(h + 1) * d]
        sub["kv_len"] = inp["kv_len"][b:b + 1]
        sub["lmk"] = dev["lmk"][b:b + 1, h:h + 1].float().cpu().numpy()
        sub["k_cache"] = dev["k_cache"][b:b + 1, h:h + 1].float().cpu().numpy()
        sub["v_cache"] = dev["v_cache"][b:b + 1, h:h + 1].float().cpu().numpy()
        _compare(sub, cfg, o[b:b + 1, h:h + 1], idx[b:b + 1, h:h + 1], w[b:b + 1, h:h + 1], [(0, 0)])


# With bf16 and at least 256 (sequence, head) pairs the step runs as one fused kernel (one workgroup
# per pair): ragged caches there exercise empty slots and partial last chunks in it.
WHOLE = [
    synth.DecodeConfig("bf16_whole_ragged_d128", 4, 64, 3000, 128, 64, 64, "bf16", 32, 512,
                       kv_len=(3000, 1, 65, 2047)),
    synth.DecodeConfig("bf16_whole_ragged_d64", 8, 32, 1500, 64, 64, 16, "bf16", 16, 256,
                       kv_len=(1500, 64, 1, 777, 1024, 1100, 3, 1499)),
    # Q-Cal rank not a multiple of the 8-element vectors (element-wise W_up reads), and no Q-Cal
    synth.DecodeConfig("bf16_whole_rank12", 2, 128, 2000, 128, 64, 16, "bf16", 12, 256, kv_len=(2000, 700)),
    synth.DecodeConfig("bf16_whole_noqcal", 4, 64, 1000, 64, 64, 8, "bf16", 0, 0, kv_len=(1000, 1, 64, 999)),
]


@pytest.mark.parametrize("cfg", WHOLE, ids=lambda c: c.name)
def test_decode_whole_pair_ragged(lib, cfg):
    print(f"[case] decode {cfg}", flush=True)
    inp = synth.make_decode_inputs_np(cfg)
    o, idx, w = _run(_to_dev(inp, cfg.dtype), cfg)
    _torch().cuda.synchronize()
    pairs = [(b, h) for b in range(cfg.batch) for h in range(0, cfg.heads, 5)]
    _compare(inp, cfg, o, idx, w, pairs)


def _tied_landmarks(inp, cfg, kind):
    """Overwrite the landmarks so that many chunks carry bit-identical rows (hence bit-identical
    scores on both sides).  Scores of q-aligned rows c*q are about c*|q|^2, far above those of
    the N(0,1) rows.
      all_equal  - every chunk the same row: n equal scores (more candidates than the compaction
                   buffer holds: the block-wide path), expected selection 0..k-1;
      top_heavy  - 70% of chunks carry q itself: hundreds of ties at the k-th score;
      boundary   - 60 chunks carry q, 30 carry 0.8 q: the k-th score is tied among 30 chunks and
                   the 4 smallest of them are taken."""
    rng = np.random.default_rng(1234)
    lmk = inp["lmk"]
    B, H, N, d = lmk.shape
    for b in range(B):
        n = -(-int(cfg.kv_len[b]) // cfg.chunk)
        for h in range(H):
            q = inp["q"][b, h]
            if kind == "all_equal":
                lmk[b, h, :n] = synth.round_to_dtype_np(rng.standard_normal(d).astype(np.float32), cfg.dtype)
            elif kind == "top_heavy":
                sel = rng.random(n) < 0.7
                lmk[b, h, :n][sel] = q
            else:
                perm = rng.permutation(n)
                lmk[b, h, perm[:60]] = q
                lmk[b, h, perm[60:90]] = synth.round_to_dtype_np(0.8 * q, cfg.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("kind", ["all_equal", "top_heavy", "boundary"])
def test_decode_tied_scores(lib, kind, dtype):
    """Ties at the k-th score go to the smaller chunk index: the selection equals the oracle's
    exactly (no tolerance band: tied scores are bit-identical on both sides)."""
    cfg = synth.DecodeConfig(f"ties_{kind}_{dtype}", 2, 2, 64000, 128, 64, 64, dtype, 32, 512,
                             kv_len=(64000, 40001))
    print(f"[case] decode {cfg}", flush=True)
    inp = synth.make_decode_inputs_np(cfg)
    _tied_landmarks(inp, cfg, kind)
    o, idx, w = _run(_to_dev(inp, cfg.dtype), cfg)
    _torch().cuda.synchronize()
    pairs = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    res = O.decode(inp, cfg.chunk, cfg.topk, cfg.dtype, pairs=pairs)
    got = idx.cpu().numpy()
    for p in pairs:
        np.testing.assert_array_equal(got[p], res[p]["idx"], err_msg=str(p))
        if kind == "all_equal":
            np.testing.assert_array_equal(got[p], np.arange(cfg.topk), err_msg=str(p))
    _compare(inp, cfg, o, idx, w, pairs)


def test_decode_tied_scores_whole_pair(lib):
    """All landmarks of every (sequence, head) equal, 516 chunks, 256 pairs: the whole-pair
    attention path runs the selection itself, here over more tied candidates than one wave
    ranks.  The selection is the first k chunks with equal weights 1/k."""
    torch = _torch()
    cfg = synth.DecodeConfig("ties_whole_pair", 2, 128, 33000, 64, 64, 64, "bf16", 16, 256,
                             kv_len=(33000, 32000))
    print(f"[case] decode {cfg}", flush=True)
    inp = synth.make_decode_inputs_np(cfg)
    _tied_landmarks(inp, cfg, "all_equal")
    o, idx, w = _run(_to_dev(inp, cfg.dtype), cfg)
    torch.cuda.synchronize()
    got, gw = idx.cpu().numpy(), w.cpu().numpy()
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            np.testing.assert_array_equal(got[b, h], np.arange(cfg.topk), err_msg=str((b, h)))
            np.testing.assert_allclose(gw[b, h], 1.0 / cfg.topk, rtol=1e-6, err_msg=str((b, h)))
    _compare(inp, cfg, o, idx, w, [(0, 0), (1, 77), (1, 127)])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_long_cache_dense_scores(lib, dtype):
    """Caches of more than 8192 chunks: dense landmark scores and the radix selection."""
    cfg = synth.DecodeConfig(f"long_cache_{dtype}", 1, 2, 600000, 64, 64, 64, dtype, 8, 128,
                             kv_len=(599937,), needles=4)
    print(f"[case] decode {cfg}", flush=True)
    inp = synth.make_decode_inputs_np(cfg)
    o, idx, w = _run(_to_dev(inp, cfg.dtype), cfg)
    _torch().cuda.synchronize()
    pairs = [(0, h) for h in range(cfg.heads)]
    _compare(inp, cfg, o, idx, w, pairs)
    got = idx.cpu().numpy()
    for b, h in pairs:
        assert set(inp["needle_ids"][b, h]) <= set(got[b, h]), (b, h)
