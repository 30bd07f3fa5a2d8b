"""Thin Python binding of libhils.so (the HiLS C ABI, include/hils.h).

Argument marshalling only: tensors are checked for device, dtype and contiguity, outputs and the
workspace are allocated with torch on the tensors' device, and the call is enqueued on torch's
current stream.  Every step of the computation runs in the library's HIP kernels; if the library
is missing, load() raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhils.so")

HILS_OK = 0
DTYPE_BF16 = 0
DTYPE_FP32 = 1
ATTN_UNION = 0
ATTN_CHUNK_MAJOR = 1
ATTN_AUTO = 2
STATUS = {0: "HILS_OK", -1: "HILS_ERR_INVALID_ARG", -2: "HILS_ERR_UNSUPPORTED", -3: "HILS_ERR_ALIGNMENT",
          -4: "HILS_ERR_WORKSPACE", -5: "HILS_ERR_HIP"}
EXPORTED = ["hils_abi_version", "hils_prefill_workspace_size", "hils_decode_workspace_size",
            "hils_prefill_fwd", "hils_decode_fwd", "hils_decode_fwd_noalloc", "hils_status_string",
            "hils_last_hip_error", "hils_dense_prefill_fwd", "hils_dense_decode_workspace_size",
            "hils_dense_decode_fwd", "hils_prefill_bwd_workspace_size", "hils_prefill_bwd",
            "hils_hope_rotate", "hils_partial_landmark"]
STATIC_SCRATCH_BYTES = 64 << 20   # HILS_STATIC_SCRATCH_BYTES


class PrefillParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("chunk", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("q_tile", ctypes.c_int32), ("hidden", ctypes.c_int32), ("qcal_rank", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("stage_events", ctypes.POINTER(ctypes.c_void_p)), ("n_stage_events", ctypes.c_int32),
                ("attn_mode", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("force_local", ctypes.c_int32)]


class DecodeParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("max_kv_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("chunk", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("qcal_rank", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("stage_events", ctypes.POINTER(ctypes.c_void_p)), ("n_stage_events", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("block_table_stride", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("force_local", ctypes.c_int32)]


class DenseParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


class HopeParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rope_base", ctypes.c_float), ("train_len", ctypes.c_int32),
                ("pos0", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class LandmarkParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("max_kv_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH):
    """Open libhils.so and declare its signatures.  Raises RuntimeError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m chunk_wise_sparse_amd.csrc.build` (there is no fallback)")
    # One HIP runtime per process: torch ships its own libamdhip64, and the library must bind to
    # that same runtime (it resolves libamdhip64.so.7 by soname to the copy already loaded).
    # Opening the library first would load a second runtime that then finds no free device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.hils_abi_version.restype = i32
    lib.hils_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillParams), i32]
    lib.hils_prefill_workspace_size.restype = sz
    lib.hils_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeParams), i32]
    lib.hils_decode_workspace_size.restype = sz
    lib.hils_prefill_fwd.argtypes = [ctypes.POINTER(PrefillParams)] + [vp] * 10 + [vp, sz, vp]
    lib.hils_prefill_fwd.restype = i32
    lib.hils_decode_fwd.argtypes = [ctypes.POINTER(DecodeParams)] + [vp] * 11 + [vp, sz, vp]
    lib.hils_decode_fwd.restype = i32
    lib.hils_decode_fwd_noalloc.argtypes = [ctypes.POINTER(DecodeParams)] + [vp] * 11 + [vp]
    lib.hils_decode_fwd_noalloc.restype = i32
    lib.hils_dense_prefill_fwd.argtypes = [ctypes.POINTER(DenseParams)] + [vp] * 5
    lib.hils_dense_prefill_fwd.restype = i32
    lib.hils_dense_decode_workspace_size.argtypes = [ctypes.POINTER(DenseParams)]
    lib.hils_dense_decode_workspace_size.restype = sz
    lib.hils_dense_decode_fwd.argtypes = [ctypes.POINTER(DenseParams)] + [vp] * 6 + [sz, vp]
    lib.hils_dense_decode_fwd.restype = i32
    lib.hils_hope_rotate.argtypes = [ctypes.POINTER(HopeParams), vp, vp, vp]
    lib.hils_hope_rotate.restype = i32
    lib.hils_partial_landmark.argtypes = [ctypes.POINTER(LandmarkParams), vp, vp, vp, vp]
    lib.hils_partial_landmark.restype = i32
    lib.hils_prefill_bwd_workspace_size.argtypes = [ctypes.POINTER(PrefillParams)]
    lib.hils_prefill_bwd_workspace_size.restype = sz
    lib.hils_prefill_bwd.argtypes = [ctypes.POINTER(PrefillParams)] + [vp] * 17 + [vp, sz, vp]
    lib.hils_prefill_bwd.restype = i32
    lib.hils_status_string.argtypes = [i32]
    lib.hils_status_string.restype = ctypes.c_char_p
    lib.hils_last_hip_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(status: int, what: str):
    if status != HILS_OK:
        lib = load()
        msg = lib.hils_status_string(status).decode()
        detail = lib.hils_last_hip_error().decode()
        raise RuntimeError(f"{what} failed: {STATUS.get(status, status)} ({msg}): {detail}")


# ----------------------------------------------------------------------------------------------
# HIP events for per-stage timing (the library records them on the launch stream)
# ----------------------------------------------------------------------------------------------
class StageEvents:
    """n hipEvent_t handles created through libamdhip64; elapsed_ms(i, j) after a sync."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.n = n
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.arr[i] = ev
        self.ptr = ctypes.cast(self.arr, ctypes.POINTER(ctypes.c_void_p))

    def synchronize(self):
        rc = self.hip.hipEventSynchronize(ctypes.c_void_p(self.arr[self.n - 1]))
        if rc != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({rc})")

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.arr[i]),
                                          ctypes.c_void_p(self.arr[j]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        try:
            for i in range(self.n):
                self.hip.hipEventDestroy(ctypes.c_void_p(self.arr[i]))
        except Exception:
            pass


# ----------------------------------------------------------------------------------------------
# Calls
# ----------------------------------------------------------------------------------------------
def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require(tensors: Sequence, device, dtype):
    for name, t in tensors:
        if t is None:
            continue
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if t.dtype != dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _stream_handle(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def prefill(q, k, v, lmk, h=None, w_down=None, w_up=None, *, topk: int, chunk: int = 64,
            q_tile: int = 0, scale: Optional[float] = None, return_selection: bool = False,
            out=None, workspace=None, events: Optional[StageEvents] = None, attn_mode: int = 0,
            block_table=None, force_local: bool = False):
    """HiLS prefill.  q [B,H,L,d]; k, v [B,Hkv,L,d]; lmk [B,Hkv,ceil(L/C),d]; h [B,L,D];
    w_down [r,D]; w_up [H*d,r].  Hkv divides H (grouped-query attention when Hkv < H).
    chunk: 32, 64 or 128 keys per chunk.
    attn_mode: ATTN_UNION (0), ATTN_CHUNK_MAJOR (1, bf16; for selections with little overlap
    between neighbouring rows) or ATTN_AUTO (2, bf16; measures the overlap and picks one; waits
    on the stream once).  Chunks of 32 and 128 keys always attend chunk-major (bf16) and ignore
    attn_mode and q_tile.

    Paged keys/values: block_table [B, S] int32 (device) and k, v pools [pages, Hkv, C, d]; chunk j
    of sequence b is page block_table[b, j].

    Returns o [B,H,L,d], or (o, idx [B,H,L,k] int32, w [B,H,L,k] float32)."""
    import torch
    lib = load()
    B, H, L, d = q.shape
    paged = block_table is not None
    if paged and (block_table.dtype != torch.int32 or block_table.device != q.device
                  or not block_table.is_contiguous() or block_table.dim() != 2 or block_table.shape[0] != B):
        raise ValueError("block_table must be a contiguous [B, S] int32 tensor on the query's device")
    _require([("q", q), ("k", k), ("v", v), ("lmk", lmk), ("h", h), ("w_down", w_down), ("w_up", w_up)],
             q.device, q.dtype)
    r = 0 if w_down is None else w_down.shape[0]
    D = 0 if h is None else h.shape[-1]
    p = PrefillParams(B, H, L, d, chunk, topk, q_tile, D, r, 0.0 if scale is None else float(scale),
                      _dtype_code(q), events.ptr if events else None, events.n if events else 0,
                      int(attn_mode), int(k.shape[1]), block_table.data_ptr() if paged else None,
                      int(block_table.shape[1]) if paged else 0, int(k.shape[0]) if paged else 0,
                      int(bool(force_local)))
    o = out if out is not None else torch.empty_like(q)
    idx = w = None
    if return_selection:
        idx = torch.empty((B, H, L, topk), dtype=torch.int32, device=q.device)
        w = torch.empty((B, H, L, topk), dtype=torch.float32, device=q.device)
    need = lib.hils_prefill_workspace_size(ctypes.byref(p), 1 if return_selection else 0)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib.hils_prefill_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(lmk), _ptr(h), _ptr(w_down),
                              _ptr(w_up), _ptr(o), _ptr(idx), _ptr(w), workspace.data_ptr(), need,
                              _stream_handle(q.device))
    check(st, "hils_prefill_fwd")
    return (o, idx, w) if return_selection else o


def decode(q, k_cache, v_cache, lmk, kv_len, h=None, w_down=None, w_up=None, *, topk: int,
           chunk: int = 64, scale: Optional[float] = None, return_selection: bool = False,
           out=None, workspace=None, events: Optional[StageEvents] = None, block_table=None,
           max_kv_len: Optional[int] = None, no_alloc: bool = False, force_local: bool = False):
    """HiLS decode step.  q [B,H,d]; caches [B,Hkv,Lmax,d]; lmk [B,Hkv,ceil(Lmax/C),d] (Hkv divides
    H); kv_len [B] int32 (device); h [B,D].  Returns o [B,H,d], or (o, idx [B,H,k], w [B,H,k]).
    Paged caches: block_table [B, S] int32 (device) and caches [pages, Hkv, C, d]; chunk j of
    sequence b is page block_table[b, j]; max_kv_len (<= S * C) is then required.
    no_alloc: call hils_decode_fwd_noalloc (the library's static scratch; no workspace)."""
    import torch
    lib = load()
    B, H, d = q.shape
    paged = block_table is not None
    if paged:
        if (max_kv_len is None or block_table.dtype != torch.int32 or block_table.device != q.device
                or not block_table.is_contiguous() or block_table.dim() != 2 or block_table.shape[0] != B):
            raise ValueError("block_table must be a contiguous [B, S] int32 tensor on the query's device, "
                             "with max_kv_len given")
    Lmax = int(max_kv_len) if paged else k_cache.shape[2]
    _require([("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("lmk", lmk), ("h", h),
              ("w_down", w_down), ("w_up", w_up)], q.device, q.dtype)
    if kv_len.dtype != torch.int32 or kv_len.device != q.device or not kv_len.is_contiguous():
        raise ValueError("kv_len must be a contiguous int32 tensor on the query's device")
    r = 0 if w_down is None else w_down.shape[0]
    D = 0 if h is None else h.shape[-1]
    p = DecodeParams(B, H, Lmax, d, chunk, topk, D, r, 0.0 if scale is None else float(scale),
                     _dtype_code(q), events.ptr if events else None, events.n if events else 0,
                     int(k_cache.shape[1]), block_table.data_ptr() if paged else None,
                     int(block_table.shape[1]) if paged else 0, int(k_cache.shape[0]) if paged else 0,
                     int(bool(force_local)))
    o = out if out is not None else torch.empty_like(q)
    idx = w = None
    if return_selection:
        idx = torch.empty((B, H, topk), dtype=torch.int32, device=q.device)
        w = torch.empty((B, H, topk), dtype=torch.float32, device=q.device)
    if no_alloc:
        st = lib.hils_decode_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lmk),
                                         kv_len.data_ptr(), _ptr(h), _ptr(w_down), _ptr(w_up), _ptr(o), _ptr(idx),
                                         _ptr(w), _stream_handle(q.device))
        check(st, "hils_decode_fwd_noalloc")
        return (o, idx, w) if return_selection else o
    need = lib.hils_decode_workspace_size(ctypes.byref(p), 1 if return_selection else 0)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib.hils_decode_fwd(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lmk),
                             kv_len.data_ptr(), _ptr(h), _ptr(w_down), _ptr(w_up), _ptr(o), _ptr(idx), _ptr(w),
                             workspace.data_ptr(), need, _stream_handle(q.device))
    check(st, "hils_decode_fwd")
    return (o, idx, w) if return_selection else o


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def dense_prefill(q, k, v, *, scale: Optional[float] = None, out=None):
    """Dense causal attention (the full-attention baseline).  q [B,H,L,d]; k, v [B,Hkv,L,d]."""
    import torch
    lib = load()
    B, H, L, d = q.shape
    _require([("q", q), ("k", k), ("v", v)], q.device, q.dtype)
    p = DenseParams(B, H, L, d, int(k.shape[1]), 0.0 if scale is None else float(scale), _dtype_code(q))
    o = out if out is not None else torch.empty_like(q)
    st = lib.hils_dense_prefill_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _stream_handle(q.device))
    check(st, "hils_dense_prefill_fwd")
    return o


def dense_decode(q, k_cache, v_cache, kv_len, *, scale: Optional[float] = None, out=None, workspace=None):
    """Dense attention of one new token per sequence over its cache.  q [B,H,d];
    caches [B,Hkv,Lmax,d]; kv_len [B] int32 (device)."""
    import torch
    lib = load()
    B, H, d = q.shape
    _require([("q", q), ("k_cache", k_cache), ("v_cache", v_cache)], q.device, q.dtype)
    if kv_len.dtype != torch.int32 or kv_len.device != q.device or not kv_len.is_contiguous():
        raise ValueError("kv_len must be a contiguous int32 tensor on the query's device")
    p = DenseParams(B, H, int(k_cache.shape[2]), d, int(k_cache.shape[1]), 0.0 if scale is None else float(scale),
                    _dtype_code(q))
    o = out if out is not None else torch.empty_like(q)
    need = lib.hils_dense_decode_workspace_size(ctypes.byref(p))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib.hils_dense_decode_fwd(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), kv_len.data_ptr(),
                                   _ptr(o), workspace.data_ptr(), need, _stream_handle(q.device))
    check(st, "hils_dense_decode_fwd")
    return o


def prefill_bwd(q, k, v, lmk, h, w_down, w_up, sel_idx, sel_w, dout, *, topk: int, chunk: int = 64,
                scale: Optional[float] = None, workspace=None):
    """Backward pass of the prefill given dout = dL/do and the forward's selection (sel_idx,
    sel_w from prefill(..., return_selection=True)).  Returns a dict of gradients: dq, dk, dv,
    dlmk and, with Q-Cal, dh, dw_down, dw_up (each shaped and typed like its input)."""
    import torch
    lib = load()
    B, H, L, d = q.shape
    _require([("q", q), ("k", k), ("v", v), ("lmk", lmk), ("h", h), ("w_down", w_down), ("w_up", w_up),
              ("dout", dout)], q.device, q.dtype)
    for name, t, dt in (("sel_idx", sel_idx, torch.int32), ("sel_w", sel_w, torch.float32)):
        if t.dtype != dt or t.device != q.device or not t.is_contiguous() or tuple(t.shape) != (B, H, L, topk):
            raise ValueError(f"{name} must be a contiguous [B,H,L,topk] {dt} tensor on the query's device")
    r = 0 if w_down is None else w_down.shape[0]
    D = 0 if h is None else h.shape[-1]
    p = PrefillParams(B, H, L, d, chunk, topk, 0, D, r, 0.0 if scale is None else float(scale),
                      _dtype_code(q), None, 0, 0, int(k.shape[1]), None, 0, 0, 0)
    g = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v), dlmk=torch.empty_like(lmk))
    if r > 0:
        g.update(dh=torch.empty_like(h), dw_down=torch.empty_like(w_down), dw_up=torch.empty_like(w_up))
    need = lib.hils_prefill_bwd_workspace_size(ctypes.byref(p))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib.hils_prefill_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(lmk), _ptr(h), _ptr(w_down),
                              _ptr(w_up), _ptr(sel_idx), _ptr(sel_w), _ptr(dout), _ptr(g["dq"]), _ptr(g["dk"]),
                              _ptr(g["dv"]), _ptr(g["dlmk"]), _ptr(g.get("dh")), _ptr(g.get("dw_down")),
                              _ptr(g.get("dw_up")), workspace.data_ptr(), need, _stream_handle(q.device))
    check(st, "hils_prefill_bwd")
    return g


def hope_rotate(x, *, rope_base: float, train_len: int, pos0: int = 0, positions=None):
    """HoPE in place on x [B, H, L, d] (q, or k with its key/value heads): pair (2i, 2i+1) of row i
    of sequence b turned by (positions[b] or pos0, plus i) * rope_base^(-2i/d) when its wavelength
    fits train_len tokens.  positions: int32 [B] on x's device, or None.  Returns x."""
    import torch
    lib = load()
    if x.dim() == 3:                          # [B, H, d]: one row per (sequence, head)
        x4 = x.unsqueeze(2)
    else:
        x4 = x
    B, H, L, d = x4.shape
    _require([("x", x)], x.device, x.dtype)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous: it is rotated in place")
    if positions is not None and (positions.dtype != torch.int32 or positions.device != x.device
                                  or not positions.is_contiguous() or positions.numel() != B):
        raise ValueError("positions must be a contiguous int32 tensor of batch entries on x's device")
    p = HopeParams(B, H, L, d, float(rope_base), int(train_len), int(pos0), _dtype_code(x))
    st = lib.hils_hope_rotate(ctypes.byref(p), _ptr(x), None if positions is None else positions.data_ptr(),
                              _stream_handle(x.device))
    check(st, "hils_hope_rotate")
    return x


def partial_landmark(k_cache, lmk, kv_len, *, chunk: int = 64):
    """The landmark of the chunk holding each sequence's newest key, in place: lmk[b, g, j] = the
    mean of k_cache[b, g, j*chunk : n] with n = kv_len[b] and j = (n - 1) // chunk.  k_cache
    [B, Hkv, Lmax, d]; lmk [B, Hkv, ceil(Lmax/chunk), d]; kv_len [B] int32 (device).  Returns lmk."""
    import torch
    lib = load()
    B, Hk, Lmax, d = k_cache.shape
    _require([("k_cache", k_cache), ("lmk", lmk)], k_cache.device, k_cache.dtype)
    if not lmk.is_contiguous():
        raise ValueError("lmk must be contiguous: it is updated in place")
    if tuple(lmk.shape) != (B, Hk, -(-Lmax // chunk), d):
        raise ValueError(f"lmk must be [{B}, {Hk}, {-(-Lmax // chunk)}, {d}]")
    if (kv_len.dtype != torch.int32 or kv_len.device != k_cache.device or kv_len.numel() != B
            or not kv_len.is_contiguous()):
        raise ValueError("kv_len must be a contiguous int32 tensor of batch entries on the cache's device")
    p = LandmarkParams(B, Hk, Lmax, d, int(chunk), _dtype_code(k_cache))
    st = lib.hils_partial_landmark(ctypes.byref(p), _ptr(k_cache), _ptr(lmk), _ptr(kv_len),
                                   _stream_handle(k_cache.device))
    check(st, "hils_partial_landmark")
    return lmk
