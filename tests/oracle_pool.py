"""The CPU oracle over many rows in a pool of worker processes (test infrastructure).

Workers are started with the "spawn" method and import only NumPy and the oracle: they never
touch the GPU, whatever the parent process has initialised.  Rows are split into contiguous
slices; the result is the same dict the oracle returns for all rows at once.
"""
from __future__ import annotations

import concurrent.futures
import multiprocessing as mp
import os
from typing import Dict, Iterable, Optional

_INP = None


def _init(inp):
    global _INP
    _INP = inp


def _prefill_slice(args):
    from oracle import hils_oracle as O
    rows, chunk, topk, dtype, scale, force_local = args
    return O.prefill_rows(_INP, rows, chunk, topk, dtype, scale=scale, force_local=force_local)


def workers() -> int:
    """At most 16 workers (the CPU share of one GPU), at most the host's cores."""
    return max(1, min(16, os.cpu_count() or 1))


def prefill_rows(inp: Dict, rows: Iterable[tuple], chunk: int, topk: int, dtype: str,
                 scale: Optional[float] = None, min_rows_per_worker: int = 64,
                 force_local: bool = False) -> Dict[tuple, dict]:
    rows = list(rows)
    n = min(workers(), max(1, len(rows) // min_rows_per_worker))
    if n <= 1:
        from oracle import hils_oracle as O
        return O.prefill_rows(inp, rows, chunk, topk, dtype, scale=scale, force_local=force_local)
    # interleave rows so that every slice holds early (cheap) and late (costly) rows
    slices = [rows[i::n] for i in range(n)]
    # A worker that fails to start breaks the pool (BrokenProcessPool) instead of being respawned.
    with concurrent.futures.ProcessPoolExecutor(n, mp_context=mp.get_context("spawn"), initializer=_init,
                                                initargs=(inp,)) as pool:
        parts = list(pool.map(_prefill_slice, [(s, chunk, topk, dtype, scale, force_local) for s in slices]))
    out = {}
    for p in parts:
        out.update(p)
    return out
