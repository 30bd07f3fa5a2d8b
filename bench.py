"""Benchmark of the HiLS forward pass on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  prefill of the 7B-shape 128K workload (B=1, H=32, L=131072, d=128, C=64, k=32, Q-Cal r=32,
  D=4096, bf16, random-walk queries and hidden states), then
  one decode step of the 7B-shape 512K workload (8 sequences x 1 token, H=32, d=128, cache 524288,
  C=64, k=64, r=32, 4 needles per (sequence, head)).
Inputs are resident in HBM before timing starts.  `value` is the prefill's algorithmic TFLOP/s
(the work the method must do, not the work the kernels execute); decode figures sit in "decode".

Printed: one JSON line (rank 0).  python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import dataclasses
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HiLS prefill TFLOP/s + decode µs/token & HBM GB/s at 128K–512K, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def prefill_work(cfg):
    """Algorithmic FLOP per stage: Q-Cal code, selection (scores + Q-Cal offset), attention."""
    B, H, L, d, C, k, r, D = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.chunk, cfg.topk, \
        cfg.qcal_rank, cfg.hidden
    N = L // C
    scoring = B * H * 2 * d * C * N * (N + 1) // 2
    pairs = B * H * C * sum(min(k, c + 1) for c in range(N))
    attention = 4 * C * d * pairs
    qcal_code = 2 * B * L * r * D
    qcal_up = 2 * B * L * r * H * d
    return dict(qcal_code=qcal_code, select=scoring + qcal_up, attention=attention,
                total=scoring + attention + qcal_code + qcal_up,
                qcal_code_bytes=B * L * D * 2 + r * D * 2 + B * L * r * 4)


def decode_bytes(cfg):
    """Algorithmic HBM bytes of one decode step (selection outputs not requested)."""
    B, H, d, C, k, r, D = cfg.batch, cfg.heads, cfg.head_dim, cfg.chunk, cfg.topk, cfg.qcal_rank, cfg.hidden
    e = 2
    total = 0
    for b in range(B):
        kv = cfg.kv_len[b]
        n = -(-kv // C)
        total += H * n * d * e                       # landmarks
        total += H * min(k, n) * 2 * C * d * e       # selected chunks' keys and values (full chunks)
    total += 2 * B * H * d * e + B * D * e + r * (D + H * d) * e
    return total


def source_digest(files):
    """sha256 over the given library sources (relative to the package's csrc/), in order."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "chunk_wise_sparse_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


# The dominant kernel's code: a change to any of these files makes stored counters stale.
KERNEL_SOURCES = {"attention": ["attention.hip", "hils_device.h", "hils_launch.h"],
                  "select": ["select_fast.hip", "select.hip", "hils_device.h", "hils_launch.h"],
                  "qcal_code": ["qcal.hip", "hils_device.h", "hils_launch.h"]}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_prefill_128k.txt")


def stored_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when the
    summary is missing or was taken from different kernel sources.  The file holds key = value
    lines; FETCH_SIZE / WRITE_SIZE are KiB per dispatch, scaled by the copy-kernel factors."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
    if kv.get(f"{kernel}.source_digest") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    try:
        fetch = float(kv[f"{kernel}.FETCH_SIZE_KiB"]) * 1024 * float(kv["copy.fetch_factor"])
        write = float(kv[f"{kernel}.WRITE_SIZE_KiB"]) * 1024 * float(kv["copy.write_factor"])
    except (KeyError, ValueError):
        return None
    return fetch + write


def calib_copy(nbytes=1 << 30, reps=3):
    """Plain device-to-device copies of a known size, for counter calibration under rocprofv3."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": nbytes, "reps": reps}), flush=True)


def union_stats(P, cfg, dev):
    """Chunk-union statistics of one prefill's selection (idx written): mean fraction of a row's
    chunks also chosen by the previous row, distinct chunks per 16-row wave block and per
    128-row workgroup, and the attention FLOP the kernel executes (a wave computes every chunk
    any of its 16 rows selected, for all 16 rows)."""
    import torch
    from chunk_wise_sparse_amd import hils
    _, idx, _ = hils.prefill(P["q"], P["k"], P["v"], P["lmk"], P["h"], P["w_down"], P["w_up"],
                             topk=cfg.topk, return_selection=True)
    torch.cuda.synchronize()
    B, H, L, k = idx.shape
    overlap, u16, u128 = 0.0, 0.0, 0.0
    for b in range(B):
        for h in range(H):
            x = idx[b, h].long()
            a, pr = x[1:], x[:-1]
            inter = ((a.unsqueeze(-1) == pr.unsqueeze(-2)) & (a.unsqueeze(-1) >= 0)).any(-1).sum(-1).float()
            overlap += (inter / (a >= 0).sum(-1).float()).mean().item()
            for m, acc in ((16, "u16"), (128, "u128")):
                s, _ = torch.sort(x.reshape(L // m, m * k), dim=-1)
                distinct = ((s[:, 1:] != s[:, :-1]) & (s[:, 1:] >= 0)).sum(-1) + (s[:, 0] >= 0).long()
                if acc == "u16":
                    u16 += distinct.float().sum().item()
                else:
                    u128 += distinct.float().sum().item()
    n_bh = B * H
    del idx
    executed = u16 * 16 * 4 * cfg.chunk * cfg.head_dim      # FLOP: chunk-steps x rows x 4 C d
    return dict(adjacent_overlap=overlap / n_bh,
                union_per_16_rows=u16 / n_bh / (L // 16), union_per_128_rows=u128 / n_bh / (L // 128),
                executed_attention_flop=executed)


def _oracle_rows_worker(args):
    """Pool worker (spawned, imports NumPy and the oracle only): prefill rows, timed."""
    from oracle import hils_oracle as O
    inp, rows, chunk, topk, dtype = args
    t0 = time.perf_counter()
    O.prefill_rows(inp, rows, chunk, topk, dtype)
    return time.perf_counter() - t0


def _oracle_decode_worker(args):
    from oracle import hils_oracle as O
    inp, chunk, topk, dtype = args
    t0 = time.perf_counter()
    O.decode(inp, chunk, topk, dtype)
    return time.perf_counter() - t0


def _pool(n):
    import concurrent.futures
    import multiprocessing as mp
    return concurrent.futures.ProcessPoolExecutor(n, mp_context=mp.get_context("spawn"))


def oracle_workers():
    return max(1, min(16, os.cpu_count() or 1))


class _Rows:
    """Hidden states of a few token positions, indexable like h[b, i] (the oracle reads no others)."""

    def __init__(self, rows):
        self.rows = rows

    def __getitem__(self, key):
        return self.rows[key]


def _head_inputs(dev, cfg, h, rows):
    """Host copy of one head of a device prefill workload (the oracle's input for head slot 0),
    with the hidden states of `rows` only."""
    import numpy as np
    inp = {key: dev[key][:, h:h + 1].float().cpu().numpy() for key in ("q", "k", "v", "lmk")}
    if cfg.qcal_rank:
        sel = sorted(set(rows))
        hv = dev["h"][0, sel].float().cpu().numpy()
        inp["h"] = _Rows({(0, i): hv[n] for n, i in enumerate(sel)})
        inp["w_down"] = dev["w_down"].float().cpu().numpy()
        d = cfg.head_dim
        inp["w_up"] = np.zeros((cfg.heads * d, cfg.qcal_rank), np.float32)
        inp["w_up"][:d] = dev["w_up"][h * d:(h + 1) * d].float().cpu().numpy()   # head slot 0 = head h
    return inp


def _prefill_row_flops(cfg, i):
    c = i // cfg.chunk
    d = cfg.head_dim
    return 2 * d * (c + 1) + 4 * cfg.chunk * d * min(cfg.topk, c + 1) + 2 * cfg.qcal_rank * (cfg.hidden + d)


def oracle_prefill_rate(dev, cfg, rows_per_head, heads, seed=11):
    """The oracle on rows_per_head uniform random rows of each of `heads`, one head per worker
    process: returns (TFLOP/s of algorithmic work summed over the workers, rows, worker seconds,
    workers).  The rate is the work over each worker's own compute time (input shipping excluded),
    added over the workers that ran at once."""
    import numpy as np
    rng = np.random.default_rng(seed)
    jobs, flops = [], []
    for h in heads:
        rows = sorted(int(x) for x in rng.integers(0, cfg.seq_len, size=rows_per_head))
        jobs.append((_head_inputs(dev, cfg, h, rows), [(0, 0, i) for i in rows], cfg.chunk, cfg.topk, cfg.dtype))
        flops.append(sum(_prefill_row_flops(cfg, i) for i in rows))
    nw = min(oracle_workers(), len(jobs))
    with _pool(nw) as pool:
        secs = list(pool.map(_oracle_rows_worker, jobs))
    rate = sum(f / t for f, t in zip(flops, secs)) / len(jobs) * nw / 1e12
    return rate, rows_per_head * len(heads), sum(secs), nw


def cpu_baseline(dev, cfg):
    """The oracle, as it stands, on sampled rows of the 128K workload (4 heads x 256 random rows),
    in a pool of worker processes on the host's cores; a rate, so no extrapolation is needed."""
    heads = tuple(range(0, cfg.heads, max(1, cfg.heads // oracle_workers())))[:oracle_workers()]
    rate, rows, secs, nw = oracle_prefill_rate(dev, cfg, 64, heads=heads)
    return dict(value=rate, unit="TFLOP/s", cores=nw, kind="oracle",
                sample=f"{rows} uniform random query rows of prefill_128k ({len(heads)} heads x 64 rows), one head "
                       f"per worker process on {nw} host cores ({secs:.1f} s of worker compute); the algorithmic "
                       "TFLOP/s of those rows, per worker, summed over the workers")


def cpu_baseline_detail(P32, D512, dcfg):
    """The oracle on the other workloads: the tiny fp32 case in full, the 32K prefill and the 512K
    decode step sampled (labelled, extrapolated to the whole workload by its work)."""
    import numpy as np
    from chunk_wise_sparse_amd import synth
    nw = oracle_workers()
    out = {}
    # tiny fp32, every row (host inputs, as the tests use them)
    tcfg = synth.CONFIGS["tiny_fp32"]
    inp = synth.make_prefill_inputs_np(tcfg)
    rows = [(0, h, i) for h in range(tcfg.heads) for i in range(tcfg.seq_len)]
    jobs = [(inp, rows[w::nw], tcfg.chunk, tcfg.topk, tcfg.dtype) for w in range(nw)]
    t0 = time.perf_counter()
    with _pool(nw) as pool:
        list(pool.map(_oracle_rows_worker, jobs))
    out["tiny_fp32"] = dict(seconds=time.perf_counter() - t0, rows=len(rows), cores=nw, kind="oracle",
                            sample="full workload")
    # 32K prefill: 512 random rows of each of 4 heads
    scfg = synth.CONFIGS["prefill_32k"]
    rate, nrows, secs, nws = oracle_prefill_rate(P32, scfg, 256, heads=tuple(range(scfg.heads)))
    work = prefill_work(scfg)["total"]
    out["prefill_32k"] = dict(tflops=rate, seconds_extrapolated=work / (rate * 1e12), cores=nws, kind="oracle",
                              sample=f"{nrows} random rows (256 of each of the 16 heads, {secs:.1f} s of worker "
                                     "compute); the full workload's time is extrapolated by algorithmic work")
    # 512K decode: 8 of the 256 (sequence, head) pairs, one per sequence
    if D512 is not None:
        B, H, Lm, d = D512["k_cache"].shape
        pairs = [(b, (7 * b + 3) % H) for b in range(B)]
        jobs = []
        for (b, h) in pairs:
            sub = dict(q=D512["q"][b:b + 1, h:h + 1].float().cpu().numpy(),
                       k_cache=D512["k_cache"][b:b + 1, h:h + 1].float().cpu().numpy(),
                       v_cache=D512["v_cache"][b:b + 1, h:h + 1].float().cpu().numpy(),
                       lmk=D512["lmk"][b:b + 1, h:h + 1].float().cpu().numpy(),
                       kv_len=np.asarray([dcfg.kv_len[b]], np.int32), h=D512["h"][b:b + 1].float().cpu().numpy(),
                       w_down=D512["w_down"].float().cpu().numpy(),
                       w_up=D512["w_up"][h * d:(h + 1) * d].float().cpu().numpy())
            jobs.append((sub, dcfg.chunk, dcfg.topk, dcfg.dtype))
        t0 = time.perf_counter()
        with _pool(min(nw, len(jobs))) as pool:
            per = list(pool.map(_oracle_decode_worker, jobs))
        wall = time.perf_counter() - t0
        cpu_s = sum(per)
        out["decode_512k"] = dict(us_per_step_extrapolated=cpu_s / len(pairs) * B * H / min(nw, len(jobs)) * 1e6,
                                  cores=min(nw, len(jobs)), kind="oracle",
                                  sample=f"{len(pairs)} of {B * H} (sequence, head) pairs ({wall:.1f} s wall, "
                                         f"{cpu_s:.1f} s of worker time); one step's time extrapolated as all "
                                         "pairs spread over the workers")
    return out


def time_prefill(P, cfg, reps, **kw):
    """Mean stage times (Q-Cal code, selection, attention) of `reps` prefills, ms."""
    import torch
    from chunk_wise_sparse_amd import hils
    ev = [hils.StageEvents(4) for _ in range(reps)]
    for e in ev:
        hils.prefill(P["q"], P["k"], P["v"], P["lmk"], P.get("h"), P.get("w_down"), P.get("w_up"), topk=cfg.topk,
                     events=e, **kw)
    torch.cuda.synchronize()
    return [sum(e.elapsed_ms(s, s + 1) for e in ev) / reps for s in range(3)]


def event_ms(fn, reps):
    """Mean ms of fn() over reps calls, timed with events on the current stream."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def stage_dict(cfg, st):
    w = prefill_work(cfg)
    ms = sum(st)
    return dict(prefill_ms=ms, qcal_code_ms=st[0], select_ms=st[1], attention_ms=st[2],
                tflops=w["total"] / (ms * 1e-3) / 1e12,
                select_frac=w["select"] / (st[1] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                attention_frac=w["attention"] / (st[2] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS)


def bench_512k(dev):
    """512K-token prefill (k = 64): random-walk queries (union walk) and i.i.d. queries (chunk-major
    and automatic modes; the union walk on them does near-dense work).  Both regimes share k, v,
    landmarks and the Q-Cal weights.  Returns the results and the walk inputs."""
    import torch
    from chunk_wise_sparse_amd import hils, synth
    cfg = synth.CONFIGS["prefill_512k_walk"]
    print("[bench] generating prefill_512k (walk)", file=sys.stderr, flush=True)
    P = synth.make_prefill_inputs_torch(cfg, dev)
    ws = torch.empty(9 << 30, dtype=torch.uint8, device=dev)
    time_prefill(P, cfg, 1, workspace=ws)
    res = dict(walk=stage_dict(cfg, time_prefill(P, cfg, 2, workspace=ws)))
    icfg = synth.CONFIGS["prefill_512k_iid"]
    gq = torch.Generator(device=dev).manual_seed(synth.subseed(icfg.seed, "q"))
    gh = torch.Generator(device=dev).manual_seed(synth.subseed(icfg.seed, "h"))
    Pi = dict(P, q=torch.randn(P["q"].shape, generator=gq, device=dev).to(P["q"].dtype),
              h=torch.randn(P["h"].shape, generator=gh, device=dev).to(P["h"].dtype))
    print("[bench] prefill_512k i.i.d.: chunk-major and automatic modes", file=sys.stderr, flush=True)
    time_prefill(Pi, icfg, 1, workspace=ws, attn_mode=hils.ATTN_CHUNK_MAJOR)
    res["iid_chunk_major"] = stage_dict(icfg, time_prefill(Pi, icfg, 2, workspace=ws, attn_mode=hils.ATTN_CHUNK_MAJOR))
    res["iid_auto"] = stage_dict(icfg, time_prefill(Pi, icfg, 1, workspace=ws, attn_mode=hils.ATTN_AUTO))
    res["walk_auto"] = stage_dict(cfg, time_prefill(P, cfg, 1, workspace=ws, attn_mode=hils.ATTN_AUTO))
    del Pi, ws
    torch.cuda.empty_cache()
    return res, P


def length_sweep_from(P512, lengths=(32768, 65536, 131072, 262144, 524288)):
    """HiLS prefill (k = 32, the 128K workload's shape) and this library's dense causal attention
    on the first L tokens of the 512K random-walk workload, L = 32K..512K."""
    import torch
    from chunk_wise_sparse_amd import hils, synth
    base = synth.CONFIGS["prefill_128k"]
    ws = torch.empty(3 << 30, dtype=torch.uint8, device=P512["q"].device)
    out = []
    for L in lengths:
        cfg = dataclasses.replace(base, name=f"prefill_{L // 1024}k_k32", seq_len=L)
        P = dict(q=P512["q"][:, :, :L].contiguous(), k=P512["k"][:, :, :L].contiguous(),
                 v=P512["v"][:, :, :L].contiguous(), lmk=P512["lmk"][:, :, :L // 64].contiguous(),
                 h=P512["h"][:, :L].contiguous(), w_down=P512["w_down"], w_up=P512["w_up"])
        time_prefill(P, cfg, 1, workspace=ws)
        st = time_prefill(P, cfg, 2, workspace=ws)
        ms = sum(st)
        o = torch.empty_like(P["q"])
        hils.dense_prefill(P["q"], P["k"], P["v"], out=o)
        dense_ms = event_ms(lambda: hils.dense_prefill(P["q"], P["k"], P["v"], out=o), 1 if L >= 262144 else 2)
        dense_flop = 4 * base.heads * base.head_dim * L * (L + 1) / 2
        out.append(dict(seq_len=L, prefill_ms=ms, qcal_code_ms=st[0], select_ms=st[1], attention_ms=st[2],
                        tflops=prefill_work(cfg)["total"] / (ms * 1e-3) / 1e12, dense_causal_ms=dense_ms,
                        dense_tflops=dense_flop / (dense_ms * 1e-3) / 1e12, dense_over_hils=dense_ms / ms))
        print(f"[bench] sweep {L}: hils {ms:.2f} ms, dense {dense_ms:.1f} ms", file=sys.stderr, flush=True)
        del P, o
        torch.cuda.empty_cache()
    return out


def prefill_chunk_sizes(scfg, dev):
    """The 32K prefill workload at chunk sizes 32 and 128 (MFMA selection, chunk-major MFMA
    attention): stage times of three calls after one untimed call."""
    from chunk_wise_sparse_amd import synth
    out = {}
    for C in (32, 128):
        ccfg = dataclasses.replace(scfg, chunk=C, name=f"prefill_32k_chunk{C}")
        PC = synth.make_prefill_inputs_torch(ccfg, dev)
        time_prefill(PC, ccfg, 1, chunk=C)
        st = time_prefill(PC, ccfg, 3, chunk=C)
        out[f"prefill_32k_chunk{C}"] = dict(
            prefill_ms=sum(st), qcal_code_ms=st[0], select_ms=st[1], attention_ms=st[2],
            tflops=prefill_work(ccfg)["total"] / (sum(st) * 1e-3) / 1e12)
        del PC
    return out


def chunk_sizes_only():
    """bench.py --chunk-sizes: the chunk-size extras alone, one JSON line."""
    import torch
    from chunk_wise_sparse_amd import hils, synth
    hils.load()
    dev = torch.device("cuda:0")
    res = prefill_chunk_sizes(synth.CONFIGS["prefill_32k"], dev)
    dcfg = synth.CONFIGS["decode_512k"]
    D = synth.make_decode_inputs_torch(dcfg, dev)
    res["decode_chunk_sizes"] = bench_decode_chunk_sizes(D, dcfg, dev)
    print(json.dumps(res), flush=True)


def bench_decode_chunk_sizes(D, dcfg, dev):
    """The 512K decode step at chunk 128 and its first 256K tokens at chunk 32 (the generic
    selection's limit is 8192 chunks): the same q, caches and Q-Cal inputs, landmarks made for the
    chunk size by the workload's recipe (chunk means plus noise, no needles)."""
    import torch
    from chunk_wise_sparse_amd import hils, synth
    out = {}
    for C, L in ((128, dcfg.max_kv_len), (32, dcfg.max_kv_len // 2)):
        kc = D["k_cache"] if L == dcfg.max_kv_len else D["k_cache"][:, :, :L].contiguous()
        vc = D["v_cache"] if L == dcfg.max_kv_len else D["v_cache"][:, :, :L].contiguous()
        lmk = synth.chunk_landmarks_dev(kc, C, dcfg.seed)
        kvl = torch.full_like(D["kv_len"], L)
        run = lambda: hils.decode(D["q"], kc, vc, lmk, kvl, D["h"], D["w_down"], D["w_up"], topk=dcfg.topk,
                                  chunk=C)
        run()
        ms = event_ms(run, 5)
        nb = dcfg.batch * dcfg.heads * ((L // C) * dcfg.head_dim * 2 + 2 * dcfg.topk * C * dcfg.head_dim * 2)
        out[f"chunk{C}"] = dict(kv_len=L, us_per_step=ms * 1e3, GBps=nb / (ms * 1e-3) / 1e9,
                                frac_hbm=nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                note="landmarks + selected keys/values read once per step")
        del kc, vc, lmk
    torch.cuda.empty_cache()
    return out


def bench_backward(P, cfg, o, dev):
    """Backward pass of the 128K prefill for a random dout: ms and algorithmic TFLOP/s.  Work per
    selected (row, chunk): S, dP, dq, dk and dv products, 10 C d FLOP; Q-Cal: four rank-r products."""
    import torch
    from chunk_wise_sparse_amd import hils
    _, idx, w = hils.prefill(P["q"], P["k"], P["v"], P["lmk"], P["h"], P["w_down"], P["w_up"], topk=cfg.topk,
                             return_selection=True)
    g = torch.Generator(device=dev).manual_seed(77)
    dout = torch.randn(P["q"].shape, generator=g, device=dev).to(P["q"].dtype)
    ws = torch.empty(8 << 30, dtype=torch.uint8, device=dev)
    run = lambda: hils.prefill_bwd(P["q"], P["k"], P["v"], P["lmk"], P["h"], P["w_down"], P["w_up"], idx, w, dout,
                                   topk=cfg.topk, workspace=ws)
    run()
    ms = event_ms(run, 2)
    B, H, L, d, C, k, r, D = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.chunk, cfg.topk, cfg.qcal_rank, \
        cfg.hidden
    pairs = B * H * C * sum(min(k, c + 1) for c in range(L // C))
    flop = 10 * C * d * pairs + 4 * B * L * r * H * d + 4 * B * L * r * D
    del idx, w, dout, ws
    torch.cuda.empty_cache()
    return dict(ms=ms, algorithmic_flop=flop, tflops=flop / (ms * 1e-3) / 1e12,
                frac=flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                note="one backward pass (all gradients, Q-Cal included) of prefill_128k for a random dout, "
                     "the forward's selection given; two timed calls")


def length_sweep():
    """The --sweep mode: length_sweep_from on the 512K random-walk workload's inputs, one JSON line
    per length (HiLS prefill stages and this library's dense causal prefill of the same q, k, v)."""
    import torch
    from chunk_wise_sparse_amd import hils, synth
    hils.load()
    dev = torch.device("cuda:0")
    P512 = synth.make_prefill_inputs_torch(synth.CONFIGS["prefill_512k_walk"], dev)
    for row in length_sweep_from(P512):
        print(json.dumps(row), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-union-stats", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the 32K/512K workloads, the length sweep, q_tile 64, the backward pass and "
                         "the dense comparators")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run plain 1 GiB device copies (counter calibration) and exit")
    ap.add_argument("--chunk-sizes", action="store_true",
                    help="only time the 32K prefill workload at chunk sizes 32 and 128 and the 512K decode step "
                         "at chunk 128 (256K at chunk 32), one JSON line, and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="only time the prefill of the 128K workload's shape at 32K..512K tokens "
                         "(one JSON line per length, beside this library's dense causal prefill of "
                         "the same q, k, v) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.calib_copy:
        calib_copy()
        return
    if args.sweep:
        length_sweep()
        return
    if args.chunk_sizes:
        chunk_sizes_only()
        return

    import torch
    from chunk_wise_sparse_amd import hils, synth

    hils.load()
    dev = torch.device("cuda:0")
    pcfg = synth.CONFIGS["prefill_128k"]
    dcfg = synth.CONFIGS["decode_512k"]
    print(f"[bench] generating {pcfg.name}", file=sys.stderr, flush=True)
    P = synth.make_prefill_inputs_torch(pcfg, dev)
    D = None
    if not args.no_decode:
        print(f"[bench] generating {dcfg.name}", file=sys.stderr, flush=True)
        D = synth.make_decode_inputs_torch(dcfg, dev)
    o = torch.empty_like(P["q"])
    pev = [hils.StageEvents(4) for _ in range(args.steps)]       # one set per timed step, read after
    # The decode step is timed by two events around it (events recorded between its kernels
    # would add their own gaps); its stage breakdown comes from separate steps with stage events.
    dec_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    dev_ev = [hils.StageEvents(5) for _ in range(args.steps)]
    od = torch.empty_like(D["q"]) if D is not None else None
    pws = torch.empty(1 << 31, dtype=torch.uint8, device=dev)     # >= the prefill workspace
    dws = torch.empty(1 << 26, dtype=torch.uint8, device=dev)

    def run_decode(events=None):
        hils.decode(D["q"], D["k_cache"], D["v_cache"], D["lmk"], D["kv_len"], D["h"], D["w_down"],
                    D["w_up"], topk=dcfg.topk, out=od, workspace=dws, events=events)

    def step(i):
        hils.prefill(P["q"], P["k"], P["v"], P["lmk"], P["h"], P["w_down"], P["w_up"], topk=pcfg.topk,
                     out=o, workspace=pws, events=pev[i] if i >= 0 else None)
        if D is not None:
            if i >= 0:
                dec_ev[i][0].record()
            run_decode()
            if i >= 0:
                dec_ev[i][1].record()

    for _ in range(args.warmup):
        step(-1)
    torch.cuda.synchronize()
    print(f"[bench] warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)
    stage_p = [0.0, 0.0, 0.0]
    stage_d = [0.0, 0.0, 0.0, 0.0]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    dec_ms = 0.0
    for i in range(args.steps):
        for s in range(3):
            stage_p[s] += pev[i].elapsed_ms(s, s + 1)
        if D is not None:
            dec_ms += dec_ev[i][0].elapsed_time(dec_ev[i][1])
    cold_ms = 0.0
    if D is not None:                          # stage breakdown (informational)
        for i in range(args.steps):
            run_decode(dev_ev[i])
        torch.cuda.synchronize()
        for i in range(args.steps):
            for s in range(4):
                stage_d[s] += dev_ev[i].elapsed_ms(s, s + 1)
        # Cold caches: a read sweep over 1 GiB evicts L2 and the 256 MB MALL before each step
        # (a read leaves no dirty lines behind to be written back during the step).
        sweep = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.empty(1, dtype=torch.float32, device=dev)
        for i in range(args.steps):
            torch.sum(sweep, dim=0, keepdim=True, out=sink)
            dec_ev[i][0].record()
            run_decode()
            dec_ev[i][1].record()
        torch.cuda.synchronize()
        cold_ms = sum(dec_ev[i][0].elapsed_time(dec_ev[i][1]) for i in range(args.steps)) / args.steps
        del sweep
    K = args.steps
    stage_p = [x / K for x in stage_p]
    stage_d = [x / K for x in stage_d]
    work = prefill_work(pcfg)
    prefill_ms = sum(stage_p)
    value = work["total"] / (prefill_ms * 1e-3) / 1e12

    stages = {
        "qcal_code": dict(ms=stage_p[0], bound="hbm", achieved=work["qcal_code_bytes"] / stage_p[0] / 1e6,
                          unit="GB/s", peak=PEAK_HBM_GBS),
        "select": dict(ms=stage_p[1], bound="mfma", achieved=work["select"] / stage_p[1] / 1e9,
                       unit="TFLOP/s", peak=PEAK_BF16_TFLOPS),
        "attention": dict(ms=stage_p[2], bound="mfma", achieved=work["attention"] / stage_p[2] / 1e9,
                          unit="TFLOP/s", peak=PEAK_BF16_TFLOPS),
    }
    for s in stages.values():
        s["frac"] = s["achieved"] / s["peak"]
    dom_name = max(stages, key=lambda n: stages[n]["ms"])
    dom = stages[dom_name]
    per_launch = {"qcal_code": work["qcal_code_bytes"], "select": work["select"],
                  "attention": work["attention"]}[dom_name]
    roofline = dict(kernel=dom_name, bound=dom["bound"], achieved=dom["achieved"], peak=dom["peak"],
                    unit=dom["unit"], frac=dom["frac"], traffic=stored_traffic(dom_name),
                    work_per_launch=per_launch, avg_launch_ms=dom["ms"])

    decode = None
    if D is not None:
        dms = dec_ms / K
        dbytes = decode_bytes(dcfg)
        decode = dict(workload=dcfg.name, us_per_step=dms * 1e3, us_per_token=dms * 1e3 / dcfg.batch,
                      algorithmic_bytes=dbytes, GBps=dbytes / (dms * 1e-3) / 1e9,
                      frac_hbm=dbytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      cold_cache=dict(us_per_step=cold_ms * 1e3, GBps=dbytes / (cold_ms * 1e-3) / 1e9,
                                      frac_hbm=dbytes / (cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                      note="after a read sweep of 1 GiB before each step"),
                      stages_us=dict(qcal=stage_d[0] * 1e3, scores=stage_d[1] * 1e3, select=stage_d[2] * 1e3,
                                     attend=stage_d[3] * 1e3,
                                     note="separate steps with an event between stages (the events "
                                          "add gaps of their own); select is empty when the attention "
                                          "kernel selects"))

    ustats = None
    if not args.no_union_stats:
        print("[bench] union statistics of one selection", file=sys.stderr, flush=True)
        ustats = union_stats(P, pcfg, dev)
        ustats["executed_over_algorithmic"] = ustats["executed_attention_flop"] / work["attention"]
        # The same workload with i.i.d. N(0, 1) queries: adjacent rows share few chunks, so the
        # union of a query group (and the attention kernel's executed work) grows towards k per
        # row.  Informational: two timed prefills and the same union statistics.
        print("[bench] i.i.d. queries: union statistics and two timed prefills", file=sys.stderr, flush=True)
        gq = torch.Generator(device=dev).manual_seed(2024)
        Pi = dict(P, q=torch.randn(P["q"].shape, generator=gq, device=dev).to(P["q"].dtype))
        istats = union_stats(Pi, pcfg, dev)
        istats["executed_over_algorithmic"] = istats["executed_attention_flop"] / work["attention"]
        iev = [hils.StageEvents(4) for _ in range(2)]
        for e in iev:
            hils.prefill(Pi["q"], Pi["k"], Pi["v"], Pi["lmk"], Pi["h"], Pi["w_down"], Pi["w_up"],
                         topk=pcfg.topk, out=o, workspace=pws, events=e)
        torch.cuda.synchronize()
        ist = [sum(e.elapsed_ms(s, s + 1) for e in iev) / len(iev) for s in range(3)]
        istats.update(prefill_ms=sum(ist), qcal_code_ms=ist[0], select_ms=ist[1], attention_ms=ist[2])
        # The same i.i.d. workload with the chunk-major attention mode (two timed prefills).
        cev = [hils.StageEvents(4) for _ in range(2)]
        for e in cev:
            hils.prefill(Pi["q"], Pi["k"], Pi["v"], Pi["lmk"], Pi["h"], Pi["w_down"], Pi["w_up"],
                         topk=pcfg.topk, out=o, events=e, attn_mode=hils.ATTN_CHUNK_MAJOR)
        torch.cuda.synchronize()
        cst = [sum(e.elapsed_ms(s, s + 1) for e in cev) / len(cev) for s in range(3)]
        istats["chunk_major"] = dict(prefill_ms=sum(cst), select_ms=cst[1], attention_ms=cst[2])
        ustats["iid_queries"] = istats
        del Pi

    extras = {}
    if not args.no_extras:
        # idx/w written to caller buffers (the headline keeps them in the workspace)
        print("[bench] extras: selection outputs, q_tile 64, backward", file=sys.stderr, flush=True)
        sel_run = lambda: hils.prefill(P["q"], P["k"], P["v"], P["lmk"], P["h"], P["w_down"], P["w_up"],
                                       topk=pcfg.topk, out=o, return_selection=True)
        sel_run()
        sel_ms = event_ms(sel_run, 3)
        nosel_ms = event_ms(lambda: hils.prefill(P["q"], P["k"], P["v"], P["lmk"], P["h"], P["w_down"], P["w_up"],
                                                 topk=pcfg.topk, out=o, workspace=pws), 3)
        extras["prefill_128k_selection_written"] = dict(
            ms=sel_ms, ms_without=nosel_ms,
            note="whole prefill calls (events around the call): idx/w returned in caller buffers, and kept in "
                 "the workspace")
        st64 = time_prefill(P, pcfg, 3, out=o, workspace=pws, q_tile=64)
        extras["prefill_128k_q_tile_64"] = stage_dict(pcfg, st64)
        if D is not None:
            dsel_ms = event_ms(lambda: hils.decode(D["q"], D["k_cache"], D["v_cache"], D["lmk"], D["kv_len"], D["h"],
                                                   D["w_down"], D["w_up"], topk=dcfg.topk, out=od,
                                                   return_selection=True), 5)
            extras["decode_512k_selection_written"] = dict(us_per_step=dsel_ms * 1e3)
            dd_ms = event_ms(lambda: hils.dense_decode(D["q"], D["k_cache"], D["v_cache"], D["kv_len"], out=od), 3)
            kvb = 2 * dcfg.batch * dcfg.heads * dcfg.max_kv_len * dcfg.head_dim * 2
            extras["dense_decode_512k"] = dict(
                us_per_step=dd_ms * 1e3, GBps=kvb / (dd_ms * 1e-3) / 1e9, frac_hbm=kvb / (dd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                dense_over_hils=dd_ms / (dec_ms / K),
                note="this library's dense attention of the same 8 x 32 queries over the whole 512K caches")
            extras["decode_chunk_sizes"] = bench_decode_chunk_sizes(D, dcfg, dev)
        extras["backward_128k"] = bench_backward(P, pcfg, o, dev)
        # HoPE rotation of the 128K workload's q and k (a copy, rotated in place): bytes read and
        # written once each.
        qk = torch.cat([P["q"], P["k"]], dim=1).contiguous()
        hope = lambda: hils.hope_rotate(qk, rope_base=10000.0, train_len=4096)
        hope()
        hope_ms = event_ms(hope, 5)
        hb = 2 * qk.numel() * qk.element_size()
        extras["hope_128k"] = dict(ms=hope_ms, GBps=hb / (hope_ms * 1e-3) / 1e9,
                                   frac_hbm=hb / (hope_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                   note="HoPE (base 10000, 4096-token window) on q and k of prefill_128k, "
                                        "rotated in place: 2 x 2 GiB moved")
        del qk
        print("[bench] extras: prefill_32k", file=sys.stderr, flush=True)
        scfg = synth.CONFIGS["prefill_32k"]
        P32 = synth.make_prefill_inputs_torch(scfg, dev)
        # i.i.d. queries (the workload's recipe): the automatic mode, which picks chunk-major on
        # them, and the union walk for comparison
        time_prefill(P32, scfg, 1, attn_mode=hils.ATTN_AUTO)
        extras["prefill_32k"] = dict(stage_dict(scfg, time_prefill(P32, scfg, 5, attn_mode=hils.ATTN_AUTO)),
                                     attn_mode="auto")
        time_prefill(P32, scfg, 1)
        extras["prefill_32k"]["union_walk"] = stage_dict(scfg, time_prefill(P32, scfg, 5))
        extras.update(prefill_chunk_sizes(scfg, dev))
        extras["prefill_512k"], P512 = bench_512k(dev)
        print("[bench] extras: length sweep 32K..512K", file=sys.stderr, flush=True)
        extras["length_sweep"] = length_sweep_from(P512)
        del P512
        torch.cuda.empty_cache()
    else:
        P32 = None

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on samples", file=sys.stderr, flush=True)
        cpu = cpu_baseline(P, pcfg)
        if P32 is None:
            P32 = synth.make_prefill_inputs_torch(synth.CONFIGS["prefill_32k"], dev)
        extras["cpu_baseline_detail"] = cpu_baseline_detail(P32, D, dcfg)

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": wall_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill_128k + decode_512k",
                   "prefill": dict(batch=pcfg.batch, heads=pcfg.heads, seq_len=pcfg.seq_len,
                                   head_dim=pcfg.head_dim, chunk=pcfg.chunk, topk=pcfg.topk,
                                   q_tile=128, qcal_rank=pcfg.qcal_rank, hidden=pcfg.hidden,
                                   queries="random walk", hidden_states="random walk"),
                   "decode": dict(batch=dcfg.batch, heads=dcfg.heads, kv_len=dcfg.max_kv_len,
                                  head_dim=dcfg.head_dim, chunk=dcfg.chunk, topk=dcfg.topk,
                                  qcal_rank=dcfg.qcal_rank, hidden=dcfg.hidden, needles=dcfg.needles),
                   "parallelism": "single GPU"},
        "prefill_ms": prefill_ms, "prefill_algorithmic_flop": work["total"],
        "stages": stages, "roofline": roofline, "decode": decode, "union": ustats, "cpu_baseline": cpu,
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
