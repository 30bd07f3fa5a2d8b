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


def cpu_baseline(dev, cfg, budget_s=12.0):
    """The oracle, as it stands, on rows of one head of the same workload, for about budget_s."""
    import numpy as np
    from oracle import hils_oracle as O
    h = 5
    inp = {key: dev[key][:, h:h + 1].float().cpu().numpy() for key in ("q", "k", "v", "lmk")}
    rng = np.random.default_rng(11)
    rows = [int(x) for x in rng.integers(0, cfg.seq_len, size=4096)]
    inp["h"] = np.zeros((1, cfg.seq_len, cfg.hidden), np.float32)
    sel = sorted(set(rows))
    inp["h"][:, sel] = dev["h"][:, sel].float().cpu().numpy()
    inp["w_down"] = dev["w_down"].float().cpu().numpy()
    inp["w_up"] = np.zeros((cfg.heads * cfg.head_dim, cfg.qcal_rank), np.float32)
    d = cfg.head_dim
    inp["w_up"][:d] = dev["w_up"][h * d:(h + 1) * d].float().cpu().numpy()   # head slot 0 = head h
    flops, done = 0, 0
    t0 = time.perf_counter()
    for i in rows:
        O.prefill_rows(inp, [(0, 0, i)], cfg.chunk, cfg.topk, cfg.dtype)
        c = i // cfg.chunk
        flops += 2 * d * (c + 1) + 4 * cfg.chunk * d * min(cfg.topk, c + 1) + 2 * cfg.qcal_rank * (cfg.hidden + d)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=1, kind="oracle",
                sample=f"{done} random query rows of head {h} of prefill_128k, timed end to end "
                       f"({dt:.1f} s, single-threaded NumPy oracle)")


def length_sweep(lengths=(32768, 65536, 131072, 262144, 524288), reps=3):
    """Prefill time against sequence length on the 128K workload's shape (H = 32, d = 128, k = 32,
    Q-Cal r = 32, random-walk queries): stage times and algorithmic TFLOP/s per length.  The
    scoring work grows as L^2 / C and the attention work as L * k * C."""
    import dataclasses
    import torch
    from chunk_wise_sparse_amd import hils, synth
    hils.load()
    dev = torch.device("cuda:0")
    base = synth.CONFIGS["prefill_128k"]
    for L in lengths:
        cfg = dataclasses.replace(base, name=f"prefill_{L // 1024}k_k32", seq_len=L)
        P = synth.make_prefill_inputs_torch(cfg, dev)
        o = torch.empty_like(P["q"])
        ws = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
        run = lambda e=None: hils.prefill(P["q"], P["k"], P["v"], P["lmk"], P["h"], P["w_down"], P["w_up"],
                                          topk=cfg.topk, out=o, workspace=ws, events=e)
        run()
        ev = [hils.StageEvents(4) for _ in range(reps)]
        for e in ev:
            run(e)
        torch.cuda.synchronize()
        st = [sum(e.elapsed_ms(s, s + 1) for e in ev) / reps for s in range(3)]
        w = prefill_work(cfg)
        ms = sum(st)
        # Context only: dense causal attention of the same shape through PyTorch's own
        # scaled_dot_product_attention (not this library), timed with events on its stream.
        dense_ms = None
        try:
            f = torch.nn.functional.scaled_dot_product_attention
            f(P["q"], P["k"], P["v"], is_causal=True)
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            for _ in range(reps):
                f(P["q"], P["k"], P["v"], is_causal=True)
            a1.record()
            torch.cuda.synchronize()
            dense_ms = a0.elapsed_time(a1) / reps
        except RuntimeError as ex:
            print(f"[bench] dense attention at {L}: {ex}", file=sys.stderr, flush=True)
        print(json.dumps(dict(seq_len=L, prefill_ms=ms, qcal_code_ms=st[0], select_ms=st[1], attention_ms=st[2],
                              tflops=w["total"] / (ms * 1e-3) / 1e12,
                              select_tflops=w["select"] / (st[1] * 1e-3) / 1e12,
                              attention_tflops=w["attention"] / (st[2] * 1e-3) / 1e12,
                              dense_causal_sdpa_ms=dense_ms)), flush=True)
        del P, o, ws
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-union-stats", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run plain 1 GiB device copies (counter calibration) and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="only time the prefill of the 128K workload's shape at 32K..512K tokens "
                         "(one JSON line per length, with PyTorch's dense causal attention of the "
                         "same shape for context) and exit")
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

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(P, pcfg)

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": wall_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill_128k + decode_512k",
                   "prefill": dict(batch=pcfg.batch, heads=pcfg.heads, seq_len=pcfg.seq_len,
                                   head_dim=pcfg.head_dim, chunk=pcfg.chunk, topk=pcfg.topk,
                                   q_tile=pcfg.q_tile, qcal_rank=pcfg.qcal_rank, hidden=pcfg.hidden,
                                   queries="random walk", hidden_states="random walk"),
                   "decode": dict(batch=dcfg.batch, heads=dcfg.heads, kv_len=dcfg.max_kv_len,
                                  head_dim=dcfg.head_dim, chunk=dcfg.chunk, topk=dcfg.topk,
                                  qcal_rank=dcfg.qcal_rank, hidden=dcfg.hidden, needles=dcfg.needles),
                   "parallelism": "single GPU"},
        "prefill_ms": prefill_ms, "prefill_algorithmic_flop": work["total"],
        "stages": stages, "roofline": roofline, "decode": decode, "union": ustats, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
