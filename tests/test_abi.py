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
    assert lib.hils_abi_version() == 10


def _pp(**kw):
    base = dict(batch=1, heads=2, seq_len=2048, head_dim=64, chunk=64, topk=4, q_tile=64, hidden=128,
                qcal_rank=8, scale=0.0, dtype=hils.DTYPE_FP32, stage_events=None, n_stage_events=0,
                attn_mode=0, kv_heads=0, block_table=None, block_table_stride=0, num_pages=0,
                force_local=0)
    base.update(kw)
    return hils.PrefillParams(**base)


def _dp(**kw):
    base = dict(batch=2, heads=2, max_kv_len=1000, head_dim=64, chunk=64, topk=4, hidden=128,
                qcal_rank=8, scale=0.0, dtype=hils.DTYPE_FP32, stage_events=None, n_stage_events=0,
                kv_heads=0, block_table=None, block_table_stride=0, num_pages=0, force_local=0)
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
    (dict(head_dim=96), -2), (dict(chunk=48), -2), (dict(chunk=256), -2), (dict(topk=0), -2), (dict(topk=65), -2),
    (dict(chunk=32, seq_len=32 * 8192 + 1), -2),              # other chunk sizes: at most 8192 chunks
    (dict(seq_len=64 * 65535 + 1), -2), (dict(q_tile=48), -2), (dict(q_tile=256), -2), (dict(qcal_rank=65), -2), (dict(hidden=100), -2),
    (dict(dtype=7), -2), (dict(batch=0), -1), (dict(heads=-1), -1), (dict(scale=float("nan")), -1),
    (dict(seq_len=64 * 65536), -2), (dict(n_stage_events=3), -1), (dict(attn_mode=3), -2),
    (dict(attn_mode=2), -2),                                   # auto is bf16 only
    (dict(kv_heads=3), -1), (dict(kv_heads=-1), -1), (dict(kv_heads=4), -1),   # must divide heads = 2
    (dict(attn_mode=1), -2),                                   # chunk-major is bf16 only
    (dict(force_local=2), -1),
])
def test_prefill_rejects_bad_params(kw, status):
    lib = hils.load()
    assert _prefill(lib, _pp(**kw)) == status
    assert lib.hils_last_hip_error().decode() != ""
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
    # chunk-major: per-chunk counters and offsets, the list (entry and weight), the work items
    # (at most L k / 128 + N of them) and the bf16 partials of every pair of a batch: both pairs
    # here (they fit in 8 GiB)
    pc = _pp(dtype=hils.DTYPE_BF16, attn_mode=1)
    N, P = 2048 // 64, 2
    items = 2048 * 4 // 128 + N + 1
    cm = (256 + 2 * a256(P * N * 4) + 2 * a256(P * (N + 1) * 4) + a256(P * 2048 * 4 * 8)
          + a256(P * items * 8) + a256(P * 2048 * 4 * 64 * 2))
    assert lib.hils_prefill_workspace_size(ctypes.byref(pc), 1) == t + cm
    # a pair's partials alone above 8 GiB: one pair per batch
    L, k, d = 64 * 16384, 64, 128
    pb = _pp(dtype=hils.DTYPE_BF16, attn_mode=1, seq_len=L, topk=k, head_dim=d, qcal_rank=0, hidden=0)
    N = L // 64
    cm1 = (256 + 2 * a256(N * 4) + 2 * a256((N + 1) * 4) + a256(L * k * 8) + a256((L * k // 128 + N + 1) * 8)
           + a256(L * k * d * 2))
    assert lib.hils_prefill_workspace_size(ctypes.byref(pb), 1) == cm1


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


def test_decode_noalloc_rejects_oversized():
    """The no-allocation decode entry checks its scratch need against the static buffer before
    touching the device (fake pointers: the call must fail first)."""
    lib = hils.load()
    p = _dp(batch=256, heads=64, max_kv_len=64 * 8192, head_dim=128, topk=64, qcal_rank=0, hidden=0,
            dtype=hils.DTYPE_BF16)
    need = lib.hils_decode_workspace_size(ctypes.byref(p), 0)
    assert need > hils.STATIC_SCRATCH_BYTES
    st = lib.hils_decode_fwd_noalloc(ctypes.byref(p), FAKE, FAKE + (1 << 32), FAKE + (2 << 32), FAKE + (3 << 32),
                                     FAKE + (4 << 32), None, None, None, FAKE + (8 << 32), None, None, None)
    assert st == -4, st
    assert "static scratch" in lib.hils_last_hip_error().decode()
    assert lib.hils_decode_fwd_noalloc(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None, None,
                                       None) == -1


def test_prefill_partial_chunk_workspace():
    """A sequence that is not a multiple of the chunk is accepted; it is staged padded to whole
    chunks in the workspace (q, k, v, h and o copies, the selection kept in the workspace)."""
    lib = hils.load()
    a256 = lambda x: (x + 255) // 256 * 256
    p = _pp(seq_len=2000)
    Lp = 2048
    inner = a256(1 * Lp * 8 * 4) + 2 * a256(1 * 2 * Lp * 4 * 4)
    pads = 4 * a256(1 * 2 * Lp * 64 * 4) + a256(1 * Lp * 128 * 4)
    assert lib.hils_prefill_workspace_size(ctypes.byref(p), 0) == inner + pads
    assert lib.hils_prefill_workspace_size(ctypes.byref(p), 1) == inner + pads
    assert lib.hils_prefill_bwd_workspace_size(ctypes.byref(p)) == 0      # the backward needs whole chunks


def test_prefill_paged_rejects_bad_tables():
    lib = hils.load()
    bt = FAKE + (11 << 32)
    assert _prefill(lib, _pp(block_table=bt, block_table_stride=31, num_pages=100)) == -1   # 32 chunks
    assert _prefill(lib, _pp(block_table=bt, block_table_stride=32, num_pages=0)) == -1
    assert _prefill(lib, _pp(block_table=bt + 2, block_table_stride=32, num_pages=100)) == -3
    assert _prefill(lib, _pp(seq_len=2000, block_table=bt, block_table_stride=32, num_pages=100)) == -2
    assert lib.hils_prefill_bwd_workspace_size(ctypes.byref(_pp(block_table=bt, block_table_stride=32,
                                                                 num_pages=100))) == 0


def test_hope_rejects_bad_arguments():
    lib = hils.load()

    def call(p, x=FAKE):
        return lib.hils_hope_rotate(ctypes.byref(p) if p is not None else None, x, None, None)

    good = dict(batch=1, heads=2, seq_len=64, head_dim=128, rope_base=10000.0, train_len=4096, pos0=0,
                dtype=hils.DTYPE_BF16)
    mk = lambda **o: hils.HopeParams(**dict(good, **o))
    assert call(None) == -1
    assert call(mk(), x=None) == -1
    assert call(mk(batch=0)) == -1
    assert call(mk(head_dim=96)) == -2
    assert call(mk(dtype=7)) == -2
    assert call(mk(rope_base=1.0)) == -1
    assert call(mk(train_len=0)) == -1
    assert call(mk(), x=FAKE + 4) == -3


def test_other_chunk_sizes_accepted():
    """Chunk sizes 32 and 128 (any sequence length, up to 8192 chunks): the fp32 prefill workspace
    holds the Q-Cal code and, when not returned, the selection; no paged prefill and no backward;
    paged decode caches of C-row pages, with a block table of at least ceil(max_kv_len / C)
    entries per sequence."""
    lib = hils.load()
    a256 = lambda x: (x + 255) // 256 * 256
    for C in (32, 128):
        p = _pp(chunk=C, seq_len=1000)
        t = a256(1 * 1000 * 8 * 4)
        sel = a256(1 * 2 * 1000 * 4 * 4)
        assert lib.hils_prefill_workspace_size(ctypes.byref(p), 0) == t + 2 * sel
        assert lib.hils_prefill_workspace_size(ctypes.byref(p), 1) == t
        assert lib.hils_prefill_bwd_workspace_size(ctypes.byref(p)) == 0       # the backward needs chunk 64
        assert lib.hils_decode_workspace_size(ctypes.byref(_dp(chunk=C)), 1) > 0
        pb = _pp(chunk=C, block_table=FAKE, block_table_stride=64, num_pages=64)
        assert lib.hils_prefill_workspace_size(ctypes.byref(pb), 1) == 0       # paged needs chunk 64
        n = -(-1000 // C)
        assert lib.hils_decode_workspace_size(ctypes.byref(_dp(chunk=C, block_table=FAKE, block_table_stride=n,
                                                               num_pages=64)), 1) > 0
        assert lib.hils_decode_workspace_size(ctypes.byref(_dp(chunk=C, block_table=FAKE, block_table_stride=n - 1,
                                                               num_pages=64)), 1) == 0



def test_partial_landmark_rejects_bad_arguments():
    lib = hils.load()

    def call(p, k=FAKE, lm=FAKE + (1 << 30), kv=FAKE + (2 << 30)):
        return lib.hils_partial_landmark(ctypes.byref(p) if p is not None else None, k, lm, kv, None)

    good = dict(batch=2, kv_heads=4, max_kv_len=1000, head_dim=128, chunk=64, dtype=hils.DTYPE_BF16)
    mk = lambda **o: hils.LandmarkParams(**dict(good, **o))
    assert call(None) == -1
    assert call(mk(), k=None) == -1
    assert call(mk(), kv=None) == -1
    assert call(mk(batch=0)) == -1
    assert call(mk(max_kv_len=0)) == -1
    assert call(mk(head_dim=96)) == -2
    assert call(mk(chunk=16)) == -2
    assert call(mk(dtype=7)) == -2
    assert call(mk(), lm=FAKE + 8) == -3
    assert call(mk(), kv=FAKE + (2 << 30) + 2) == -3
    assert call(mk(), lm=FAKE + 4096) == -1           # lmk inside k_cache


def test_header_compiles_as_c_and_cpp(tmp_path):
    """include/hils.h is a plain C header: it compiles alone as C99 (pedantic) and as C++17."""
    import shutil
    import subprocess
    src = tmp_path / "use.c"
    src.write_text('#include "hils.h"\n'
                   'int main(void) { hils_landmark_params p = {1, 1, 64, 64, 64, 0}; (void)p;\n'
                   '  return hils_abi_version() == HILS_ABI_VERSION ? 0 : 1; }\n')
    inc = os.path.join(ROOT, "include")
    for cc, flags in (("gcc", ["-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror"]),
                      ("g++", ["-std=c++17", "-Wall", "-Werror", "-x", "c++"])):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not available")
        r = subprocess.run([cc, *flags, "-I", inc, "-c", str(src), "-o", str(tmp_path / "use.o")],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
