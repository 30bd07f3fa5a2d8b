"""The C ABI without a GPU: the library loads, exports what include/hils.h declares, and rejects
bad arguments before launching anything (only invalid calls are made here)."""
import ctypes
import os
import re

import pytest

from chunk_wise_sparse_amd import hils

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 40   # 256-byte aligned, never dereferenced: every call below fails validation first


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "hils.h")).read()
    return sorted(set(re.findall(r"\b(hils_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = hils.load()
    declared = _declared_functions()
    assert set(declared) == set(hils.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.hils_abi_version() == 5


def _pp(**kw):
    base = dict(batch=1, heads=2, seq_len=2048, head_dim=64, chunk=64, topk=4, q_tile=64, hidden=128,
                qcal_rank=8, scale=0.0, dtype=hils.DTYPE_FP32, stage_events=None, n_stage_events=0,
                attn_mode=0, kv_heads=0)
    base.update(kw)
    return hils.PrefillParams(**base)


def _dp(**kw):
    base = dict(batch=2, heads=2, max_kv_len=1000, head_dim=64, chunk=64, topk=4, hidden=128,
                qcal_rank=8, scale=0.0, dtype=hils.DTYPE_FP32, stage_events=None, n_stage_events=0,
                kv_heads=0, block_table=None, block_table_stride=0, num_pages=0)
    base.update(kw)
    return hils.DecodeParams(**base)


def _prefill(lib, p, ptrs=None, ws=FAKE, wsb=1 << 40, **over):
    t = dict(q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32), lmk=FAKE + (3 << 32), h=FAKE + (4 << 32),
             w_down=FAKE + (5 << 32), w_up=FAKE + (6 << 32), o=FAKE + (7 << 32), idx=None, w=None)
    t.update(over)
    return lib.hils_prefill_fwd(ctypes.byref(p) if p is not None else None, t["q"], t["k"], t["v"], t["lmk"],
                                t["h"], t["w_down"], t["w_up"], t["o"], t["idx"], t["w"],
                                FAKE + (9 << 32) if ws == FAKE else ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), -2), (dict(chunk=32), -2), (dict(topk=0), -2), (dict(topk=65), -2),
    (dict(seq_len=2000), -2), (dict(q_tile=32), -2), (dict(qcal_rank=65), -2), (dict(hidden=100), -2),
    (dict(dtype=7), -2), (dict(batch=0), -1), (dict(heads=-1), -1), (dict(scale=float("nan")), -1),
    (dict(seq_len=64 * 65536), -2), (dict(n_stage_events=3), -1), (dict(attn_mode=3), -2),
    (dict(attn_mode=2), -2),                                   # auto is bf16 only
    (dict(kv_heads=3), -1), (dict(kv_heads=-1), -1), (dict(kv_heads=4), -1),   # must divide heads = 2
    (dict(attn_mode=1), -2),                                   # chunk-major is bf16 only
])
def test_prefill_rejects_bad_params(kw, status):
    lib = hils.load()
    assert _prefill(lib, _pp(**kw)) == status
    assert lib.hils_last_error().decode() != ""
    assert lib.hils_prefill_workspace_size(ctypes.byref(_pp(**kw)), 0) == 0


def test_prefill_rejects_bad_pointers():
    lib = hils.load()
    p = _pp()
    assert _prefill(lib, None) == -1
    assert _prefill(lib, p, q=None) == -1
    assert _prefill(lib, p, h=None) == -1                      # Q-Cal needs h, w_down, w_up
    assert _prefill(lib, _pp(qcal_rank=0)) == -1               # ... and forbids them without Q-Cal
    assert _prefill(lib, p, idx=FAKE + (10 << 32)) == -1       # idx without w
    assert _prefill(lib, p, q=FAKE + 8) == -3                  # misaligned
    assert _prefill(lib, p, ws=None) == -4                     # workspace missing
    assert _prefill(lib, p, wsb=16) == -4                      # workspace too small
    assert _prefill(lib, p, ws=FAKE + (9 << 32) + 16) == -3    # workspace misaligned
    assert _prefill(lib, p, o=FAKE + (1 << 32) + 4096) == -1   # output overlaps k
    assert _prefill(lib, p, idx=FAKE + (10 << 32), w=FAKE + (10 << 32) + 256) == -1   # idx overlaps w


def test_prefill_workspace_size():
    lib = hils.load()
    p = _pp()
    a256 = lambda x: (x + 255) // 256 * 256
    t = a256(1 * 2048 * 8 * 4)
    sel = a256(1 * 2 * 2048 * 4 * 4)
    assert lib.hils_prefill_workspace_size(ctypes.byref(p), 0) == t + 2 * sel
    assert lib.hils_prefill_workspace_size(ctypes.byref(p), 1) == t
    # chunk-major: per-chunk counters and offsets, the list and the bf16 partials of one pair
    pc = _pp(dtype=hils.DTYPE_BF16, attn_mode=1)
    N = 2048 // 64
    cm = 256 + 2 * a256(N * 4) + 2 * a256((N + 1) * 4) + a256(2048 * 4 * 4) + a256(2048 * 4 * 64 * 2)
    assert lib.hils_prefill_workspace_size(ctypes.byref(pc), 1) == t + cm


def test_decode_rejects_bad_arguments():
    lib = hils.load()

    def call(p, **over):
        t = dict(q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32), lmk=FAKE + (3 << 32), kv=FAKE + (4 << 32),
                 h=FAKE + (5 << 32), wd=FAKE + (6 << 32), wu=FAKE + (7 << 32), o=FAKE + (8 << 32),
                 idx=None, w=None, ws=FAKE + (9 << 32), wsb=1 << 40)
        t.update(over)
        return lib.hils_decode_fwd(ctypes.byref(p) if p is not None else None, t["q"], t["k"], t["v"], t["lmk"],
                                   t["kv"], t["h"], t["wd"], t["wu"], t["o"], t["idx"], t["w"], t["ws"],
                                   t["wsb"], None)

    assert call(None) == -1
    assert call(_dp(head_dim=80)) == -2
    assert call(_dp(topk=100)) == -2
    assert call(_dp(max_kv_len=64 * 65536)) == -2
    assert call(_dp(kv_heads=3)) == -1                          # must divide heads = 2
    assert lib.hils_decode_workspace_size(ctypes.byref(_dp(kv_heads=1)), 0) > 0   # divides: accepted
    assert lib.hils_decode_workspace_size(ctypes.byref(_dp(kv_heads=3)), 0) == 0
    # paged caches: a short block table row or an empty pool is rejected
    assert call(_dp(block_table=FAKE + (11 << 32), block_table_stride=15, num_pages=100)) == -1
    assert call(_dp(block_table=FAKE + (11 << 32), block_table_stride=16, num_pages=0)) == -1
    assert call(_dp(block_table=FAKE + (11 << 32) + 2, block_table_stride=16, num_pages=100)) == -3
    assert call(_dp(), kv=None) == -1
    assert call(_dp(), kv=FAKE + (4 << 32) + 2) == -3
    assert call(_dp(), ws=None) == -4
    assert call(_dp(), wsb=100) == -4
    assert call(_dp(), o=FAKE + (1 << 32) + 64) == -1
    need = lib.hils_decode_workspace_size(ctypes.byref(_dp()), 0)
    a256 = lambda x: (x + 255) // 256 * 256
    # selection candidates: one scan workgroup per (sequence, head), 64 entries of 8 bytes
    assert need == a256(2 * 64 * 4) + a256(2 * 2 * 64 * 8) + 2 * a256(2 * 2 * 4 * 4) + a256(2 * 2 * 4 * 64 * 4)


def test_status_strings():
    lib = hils.load()
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.hils_status_string(code).decode()
