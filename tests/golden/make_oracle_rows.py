"""Write tests/golden/tiny_fp32_rows.json: oracle outputs for a few rows of the tiny fp32 workload.

A drift guard for the oracle itself: the values are produced by this script from oracle/ and the
seeded generators only (python tests/golden/make_oracle_rows.py)."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from chunk_wise_sparse_amd import synth  # noqa: E402
from oracle import hils_oracle as O  # noqa: E402

ROWS = [(0, 0, 0), (0, 0, 63), (0, 0, 64), (0, 1, 255), (0, 1, 1000), (0, 0, 2047)]


def compute():
    cfg = synth.CONFIGS["tiny_fp32"]
    inp = synth.make_prefill_inputs_np(cfg)
    res = O.prefill_rows(inp, ROWS, cfg.chunk, cfg.topk, cfg.dtype)
    return {f"{b},{h},{i}": dict(idx=[int(x) for x in r["idx"]], w=[float(x) for x in r["w"]],
                                 o=[float(x) for x in r["o"]]) for (b, h, i), r in res.items()}


if __name__ == "__main__":
    out = dict(config="tiny_fp32", source="oracle/hils_oracle.py via tests/golden/make_oracle_rows.py",
               rows=compute())
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_rows.json"), "w") as f:
        json.dump(out, f, indent=1)
