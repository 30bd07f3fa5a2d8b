"""Oracle drift guard: rows of the tiny fp32 workload against values stored by make_oracle_rows.py."""
import json
import os

import numpy as np

from golden.make_oracle_rows import compute


def test_oracle_rows_unchanged():
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_fp32_rows.json")) as f:
        stored = json.load(f)["rows"]
    now = compute()
    assert stored.keys() == now.keys()
    for key in stored:
        assert stored[key]["idx"] == now[key]["idx"]
        assert np.allclose(stored[key]["w"], now[key]["w"], rtol=0, atol=1e-12)
        assert np.allclose(stored[key]["o"], now[key]["o"], rtol=0, atol=1e-12)
