"""The chunk-major attention mode (attn_mode = 1) through the C ABI: against the CPU oracle, against
the union-walk mode on the same selection, and run to run."""
import numpy as np
import pytest

from chunk_wise_sparse_amd import hils, synth
from parity import sample_rows
from test_gpu_prefill import SMALL, _compare, _run, _to_dev, _torch

pytestmark = pytest.mark.gpu

CM = hils.ATTN_CHUNK_MAJOR
SMALL_BF16 = [c for c in SMALL if c.dtype == "bf16"]


@pytest.mark.parametrize("cfg", SMALL_BF16, ids=lambda c: c.name)
def test_chunk_major_all_rows(lib, cfg):
    print(f"[case] chunk-major all rows {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    o, idx, w = _run(lib, _to_dev(inp, cfg.dtype), cfg, attn_mode=CM)
    _torch().cuda.synchronize()
    rows = [(b, h, i) for b in range(cfg.batch) for h in range(cfg.heads) for i in range(cfg.seq_len)]
    _compare(inp, cfg, o, idx, w, rows)


def test_chunk_major_long_lists(lib):
    """256 chunks, k = 32, i.i.d. queries: early chunks are chosen by thousands of rows (many
    128-row work items per chunk), late ones by few (ragged last items)."""
    cfg = synth.PrefillConfig("bf16_16k_k32_cm", 1, 2, 16384, 128, 64, 32, "bf16", 32, 512)
    print(f"[case] {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    o, idx, w = _run(lib, _to_dev(inp, cfg.dtype), cfg, attn_mode=CM)
    rows = sample_rows(1, 2, cfg.seq_len, 160, seed=21)
    rows = sorted(set(rows) | {(0, h, i) for h in range(2) for i in range(0, 128, 3)})
    _compare(inp, cfg, o, idx, w, rows)


def test_chunk_major_pair_batches(lib):
    """B = 2, H = 16 at 16K tokens and d = 128: the (batch, head) pairs run in three batches of
    eleven, eleven and ten (each kernel takes one batch per launch).  The same selection and every
    row within the bf16 tolerance of the union walk; sampled rows of the last pair against the
    oracle."""
    torch = _torch()
    cfg = synth.PrefillConfig("bf16_pairs_cm", 2, 16, 16384, 128, 64, 16, "bf16", 16, 256)
    print(f"[case] {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    dev = _to_dev(inp, cfg.dtype)
    o_u, idx_u, w_u = _run(lib, dev, cfg)
    o_c, idx_c, w_c = _run(lib, dev, cfg, attn_mode=CM)
    torch.cuda.synchronize()
    assert torch.equal(idx_u, idx_c) and torch.equal(w_u, w_c)
    diff = (o_u.float() - o_c.float()).abs()
    print(f"[parity] pair batches chunk-major vs union: max {diff.max().item():.3g} "
          f"mean {diff.mean().item():.3g}", flush=True)
    assert diff.max().item() <= 2e-2 and diff.mean().item() <= 1e-3
    rows = [(1, 15, i) for i in sorted({r[2] for r in sample_rows(1, 1, cfg.seq_len, 40, seed=31)})]
    _compare(inp, cfg, o_c, idx_c, w_c, rows)


def test_chunk_major_deterministic(lib):
    cfg = SMALL_BF16[0]
    dev = _to_dev(synth.make_prefill_inputs_np(cfg), cfg.dtype)
    a = _run(lib, dev, cfg, attn_mode=CM)
    b = _run(lib, dev, cfg, attn_mode=CM)
    torch = _torch()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["prefill_128k", "prefill_512k_iid"])
def test_chunk_major_matches_union_full_size(lib, name):
    """Full-size workloads: the same selection (bitwise), and outputs of the two modes within the
    bf16 tolerance on every row; rows of one head against the oracle."""
    torch = _torch()
    cfg = synth.CONFIGS[name]
    print(f"[case] full size {cfg}", flush=True)
    dev = synth.make_prefill_inputs_torch(cfg, "cuda")
    o_u, idx_u, w_u = _run(lib, dev, cfg)
    o_c, idx_c, w_c = _run(lib, dev, cfg, attn_mode=CM)
    torch.cuda.synchronize()
    assert torch.equal(idx_u, idx_c) and torch.equal(w_u, w_c)
    diff = (o_u.float() - o_c.float()).abs()
    print(f"[parity] {name} chunk-major vs union: max {diff.max().item():.3g} mean {diff.mean().item():.3g}",
          flush=True)
    assert diff.max().item() <= 2e-2 and diff.mean().item() <= 1e-3
    del diff, o_u, idx_u, w_u
    heads = [cfg.heads - 1]
    d = cfg.head_dim
    rows = sample_rows(1, 1, cfg.seq_len, 12, seed=23)
    sub = {key: dev[key][:, heads].float().cpu().numpy() for key in ("q", "k", "v", "lmk")}
    pos = sorted({r[2] for r in rows})
    h_sub = np.zeros((1, cfg.seq_len, cfg.hidden), dtype=np.float32)
    h_sub[:, pos] = dev["h"][:, pos].float().cpu().numpy()
    sub["h"] = h_sub
    sub["w_down"] = dev["w_down"].float().cpu().numpy()
    sub["w_up"] = np.concatenate([dev["w_up"][hh * d:(hh + 1) * d].float().cpu().numpy() for hh in heads])
    sub_cfg = synth.PrefillConfig(cfg.name, 1, 1, cfg.seq_len, d, cfg.chunk, cfg.topk, cfg.dtype,
                                  cfg.qcal_rank, cfg.hidden)
    _compare(sub, sub_cfg, o_c[:, heads], idx_c[:, heads], w_c[:, heads], rows)


EDGE = [
    synth.PrefillConfig("cm_one_chunk", 1, 2, 64, 128, 64, 4, "bf16", 0, 0),
    synth.PrefillConfig("cm_three_chunks_k1", 2, 1, 192, 64, 64, 1, "bf16", 8, 128),
    synth.PrefillConfig("cm_five_chunks_k64", 1, 3, 320, 128, 64, 64, "bf16", 4, 128),
]


@pytest.mark.parametrize("cfg", EDGE, ids=lambda c: c.name)
def test_chunk_major_edge_sizes(lib, cfg):
    """One chunk (a single list), a length that is not a multiple of 128 rows with k = 1, and k
    larger than the number of chunks (padded selections: fewer valid slots than k)."""
    print(f"[case] chunk-major {cfg}", flush=True)
    inp = synth.make_prefill_inputs_np(cfg)
    o, idx, w = _run(lib, _to_dev(inp, cfg.dtype), cfg, attn_mode=CM)
    _torch().cuda.synchronize()
    rows = [(b, h, i) for b in range(cfg.batch) for h in range(cfg.heads) for i in range(cfg.seq_len)]
    _compare(inp, cfg, o, idx, w, rows)


@pytest.mark.parametrize("q_mode,expect", [("iid", CM), ("walk", hils.ATTN_UNION)])
def test_auto_mode_choice(lib, q_mode, expect):
    """attn_mode = AUTO measures the selection's overlap: i.i.d. queries over 256 chunks with
    k = 4 (about 55 k distinct chunks per 128-row group) take the chunk-major mode, random-walk
    queries (about 2 k) the union walk.  The two modes round differently, so the output
    identifies the mode taken."""
    torch = _torch()
    cfg = synth.PrefillConfig(f"auto_{q_mode}", 1, 4, 16384, 128, 64, 4 if q_mode == "iid" else 16, "bf16",
                              16, 256, q_mode=q_mode, h_mode=q_mode)
    print(f"[case] {cfg}", flush=True)
    dev = synth.make_prefill_inputs_torch(cfg, "cuda")
    o_a, idx_a, _ = _run(lib, dev, cfg, attn_mode=hils.ATTN_AUTO)
    o_e, idx_e, _ = _run(lib, dev, cfg, attn_mode=expect)
    o_o, _, _ = _run(lib, dev, cfg, attn_mode=CM if expect == hils.ATTN_UNION else hils.ATTN_UNION)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_e)
    assert torch.equal(o_a, o_e)
    assert not torch.equal(o_a, o_o)


@pytest.mark.parametrize("mode", [CM, hils.ATTN_AUTO])
def test_chunk_major_selection_in_workspace(lib, mode):
    """Without selection outputs, idx / w live in the workspace beside the mode's own lists and
    partials: the output must equal the run that returns the selection."""
    cfg = synth.PrefillConfig("bf16_8k_k8_ws", 1, 2, 8192, 128, 64, 8, "bf16", 16, 256)
    dev = _to_dev(synth.make_prefill_inputs_np(cfg), cfg.dtype)
    o1, _, _ = _run(lib, dev, cfg, attn_mode=mode)
    o2 = hils.prefill(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["h"], dev["w_down"], dev["w_up"],
                      topk=cfg.topk, attn_mode=mode)
    assert _torch().equal(o1, o2)
