"""The seeded generators: reproducible, and drawing what their recipe says."""
import math

import numpy as np

from chunk_wise_sparse_amd import synth


def test_prefill_generator_reproducible_and_landmark_recipe():
    cfg = synth.PrefillConfig("t", 1, 2, 512, 32, 64, 4, "bf16", 4, 48)
    a = synth.make_prefill_inputs_np(cfg)
    b = synth.make_prefill_inputs_np(cfg)
    for key in a:
        assert np.array_equal(a[key], b[key])
    # landmark = chunk mean of the keys + 0.1 N(0,1): the residual has std ~0.1
    mean = a["k"].reshape(1, 2, 8, 64, 32).astype(np.float64).mean(axis=3)
    resid = a["lmk"] - mean
    assert 0.08 < resid.std() < 0.12
    # bf16 runs hold bf16-exact values
    for key in ("q", "k", "v", "lmk", "h", "w_down", "w_up"):
        u = a[key].view(np.uint32)
        assert np.all((u & 0xFFFF) == 0), key
    assert 0.015 < a["w_down"].std() < 0.025


def test_random_walk_norm_and_step():
    rng = np.random.default_rng(0)
    w = synth.random_walk(rng, 3, 2000, 128, math.sqrt(128))
    assert np.allclose(np.linalg.norm(w, axis=-1), math.sqrt(128), rtol=1e-5)
    cos = np.sum(w[:, 1:] * w[:, :-1], axis=-1) / 128.0
    # one step of N(0, 0.05^2) per coordinate on a radius-sqrt(d) sphere: cos ~ 1 - 0.05^2/2
    assert abs(cos.mean() - (1 - 0.05 ** 2 / 2)) < 5e-4


def test_decode_needles_have_cosine_09():
    cfg = synth.DecodeConfig("t", 2, 3, 1000, 64, 64, 4, "fp32", 0, 0, kv_len=(1000, 300), needles=4)
    a = synth.make_decode_inputs_np(cfg)
    ids = a["needle_ids"]
    for b in range(2):
        nb = -(-cfg.kv_len[b] // 64)
        for h in range(3):
            assert len(set(ids[b, h])) == 4 and ids[b, h].max() < nb
            q = a["q"][b, h].astype(np.float64)
            for j in ids[b, h]:
                l = a["lmk"][b, h, j].astype(np.float64)
                assert abs(q.dot(l) / np.linalg.norm(q) / np.linalg.norm(l) - 0.9) < 1e-5
