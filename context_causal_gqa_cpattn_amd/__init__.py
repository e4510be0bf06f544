"""Python binding of the cpattn C-ABI (libcpattn.so, gfx950).

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind include/cpattn.h.  PyTorch provides device memory and the current
stream.  There is no fallback: if the library or a GPU is missing, calls raise.

Names follow the C entry points: fwd, bwd, bwd_prepass, bwd_dkdv, bwd_dq,
bwd_dbias, bwd_dkdv_ds, bwd_dq_ds, bwd_dbias_ds, fwd_window, merge, bwd_window, validate, pack,
unpack.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcpattn.so")

OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3
OP_FWD, OP_BWD, OP_BWD_DS = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 64 << 20  # CPATTN_NOALLOC_SCRATCH_BYTES
DEV_ERR_BITS = {
    0x01: "ESEQ_LEN", 0x02: "ESEQ_RANGE", 0x04: "ECHUNK_SEQ", 0x08: "ECHUNK_ROWS",
    0x10: "ECHUNK_POS", 0x20: "EBIAS", 0x40: "ELAYOUT",
}
EXPORTS = [
    "cpattn_status_str", "cpattn_last_error", "cpattn_version", "cpattn_workspace_size",
    "cpattn_validate", "cpattn_fwd", "cpattn_bwd", "cpattn_bwd_prepass", "cpattn_bwd_dkdv",
    "cpattn_bwd_dq", "cpattn_bwd_dbias", "cpattn_bwd_dkdv_ds", "cpattn_bwd_dq_ds",
    "cpattn_bwd_dbias_ds", "cpattn_pack",
    "cpattn_unpack", "cpattn_fwd_window", "cpattn_merge", "cpattn_bwd_window",
    "cpattn_a2a_split_heads", "cpattn_a2a_merge_heads", "cpattn_a2a_scatter_rows",
    "cpattn_a2a_gather_rows", "cpattn_bwd_noalloc",
]


class CpattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class DeviceError(RuntimeError):
    def __init__(self, bits: int):
        names = [n for b, n in DEV_ERR_BITS.items() if bits & b]
        super().__init__(f"device promise check failed: 0x{bits:x} {names}")
        self.bits = bits


class Problem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("q_rows", ctypes.c_int64), ("kv_rows", ctypes.c_int64),
        ("num_chunks", ctypes.c_int32), ("max_chunk_len", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32), ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
        ("bias_len", ctypes.c_int32), ("q_head_pitch", ctypes.c_int32),
        ("kv_head_pitch", ctypes.c_int32), ("ds_blocks", ctypes.c_int64),
    ]


class A2aRows(ctypes.Structure):
    """Sizes of an A2A row copy (cpattn_a2a_rows)."""
    _fields_ = [
        ("cp", ctypes.c_int32), ("chunks_per_rank", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
        ("max_chunk_len", ctypes.c_int32), ("rows_per_rank", ctypes.c_int64), ("full_rows", ctypes.c_int64),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
    ]


_lib = None
_vp = ctypes.c_void_p


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libcpattn.so (built in-tree by build.py).  Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} not found: build it with `python -m context_causal_gqa_cpattn_amd.build`")
    lib = ctypes.CDLL(p)
    lib.cpattn_status_str.restype = ctypes.c_char_p
    lib.cpattn_status_str.argtypes = [ctypes.c_int]
    lib.cpattn_last_error.restype = ctypes.c_char_p
    lib.cpattn_last_error.argtypes = []
    lib.cpattn_version.restype = ctypes.c_int
    lib.cpattn_workspace_size.restype = ctypes.c_size_t
    lib.cpattn_workspace_size.argtypes = [ctypes.POINTER(Problem), ctypes.c_int]
    P = ctypes.POINTER(Problem)
    i64, i32, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sigs = {
        "cpattn_validate": [P, _vp, _vp, _vp, _vp, _vp],
        "cpattn_fwd": [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, sz, _vp, _vp],
        "cpattn_bwd": [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                       ctypes.c_int, _vp, sz, _vp, _vp],
        "cpattn_bwd_noalloc": [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               ctypes.c_int, _vp, _vp],
        "cpattn_bwd_prepass": [P, _vp, _vp, _vp, _vp, _vp, _vp, sz, _vp, _vp],
        "cpattn_bwd_dkdv": [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, sz, _vp, _vp,
                            ctypes.c_int, _vp, _vp],
        "cpattn_bwd_dq": [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, sz, _vp, _vp, _vp],
        "cpattn_bwd_dbias": [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, sz, _vp, _vp, _vp],
        "cpattn_bwd_dkdv_ds": [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, sz, _vp, _vp,
                               ctypes.c_int, _vp, _vp],
        "cpattn_bwd_dq_ds": [P, _vp, _vp, _vp, _vp, _vp, sz, _vp, _vp, _vp],
        "cpattn_bwd_dbias_ds": [P, _vp, _vp, _vp, _vp, sz, _vp, _vp, _vp],
        "cpattn_fwd_window": [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, i32, i32, _vp, _vp, _vp, _vp],
        "cpattn_merge": [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
        "cpattn_bwd_window": [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, i32, i32, ctypes.c_int,
                              _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, sz, _vp, _vp],
        "cpattn_pack": [_vp, _vp, i32, i32, i32, i32, i64, _vp, _vp, _vp, _vp],
        "cpattn_unpack": [_vp, _vp, i32, i32, i32, i32, i64, _vp, _vp, _vp, _vp],
        "cpattn_a2a_split_heads": [_vp, _vp, i64, i32, i32, i32, _vp],
        "cpattn_a2a_merge_heads": [_vp, _vp, i64, i32, i32, i32, _vp],
        "cpattn_a2a_scatter_rows": [ctypes.POINTER(A2aRows), _vp, _vp, _vp, _vp, _vp, _vp, _vp],
        "cpattn_a2a_gather_rows": [ctypes.POINTER(A2aRows), _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    }
    for name, args in sigs.items():
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != OK:
        lib = load()
        raise CpattnError(status, f"{lib.cpattn_status_str(status).decode()}: "
                                  f"{lib.cpattn_last_error().decode()}")


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t, name, dtype, shape=None, pitch=None):
    """Device, dtype and shape checks.  With `pitch`, t is [rows, heads, D] and may be a
    head slice of a larger [rows, pitch, D] tensor (row stride pitch*D); else contiguous."""
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if pitch is None:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    elif head_pitch(t, name) != pitch:
        raise ValueError(f"{name} has {head_pitch(t, name)} heads per row in memory, expected {pitch}")


def head_pitch(t, name="tensor") -> int:
    """Heads per row in memory of a [rows, heads, D] tensor or head slice of one."""
    if t.dim() != 3:
        raise ValueError(f"{name} must be [rows, heads, head_dim]")
    rows, heads, D = t.shape
    if t.stride(2) != 1 or (heads > 1 and t.stride(1) != D):
        raise ValueError(f"{name} needs contiguous heads and head dims")
    if rows <= 1:
        return heads
    if t.stride(0) % D or t.stride(0) // D < heads:
        raise ValueError(f"{name} row stride {t.stride(0)} is not a whole number of heads >= {heads}")
    return t.stride(0) // D


def _like(t):
    """A new tensor with t's shape and strides (a head slice's pitch is kept)."""
    return _torch().empty_strided(tuple(t.shape), tuple(t.stride()), dtype=t.dtype, device=t.device)


@dataclasses.dataclass
class Layout:
    """Sequence and chunk descriptors on the device plus their host-side bounds."""
    seq_offsets: object   # int32 [B] on the GPU
    seq_lens: object      # int32 [B]
    chunks: object        # int32 [C, 4]
    num_seqs: int
    num_chunks: int
    max_chunk_len: int
    max_kv_len: int
    host_chunks: Optional[np.ndarray] = None  # int32 [C, 4], the same descriptors on the host
    host_seq_lens: Optional[np.ndarray] = None


def ds_blocks(chunks, seq_lens, causal: bool) -> int:
    """The dS store bound of cpattn_problem.ds_blocks: sum over chunks of ceil(len / 32)
    times the 32-key blocks its last row sees (causal: pos0 + len keys; else L)."""
    ch = np.asarray(chunks, dtype=np.int64).reshape(-1, 4)
    if len(ch) == 0:
        return 0
    sl = np.asarray(seq_lens, dtype=np.int64)
    keys = ch[:, 2] + ch[:, 3] if causal else sl[ch[:, 0]]
    return int((((ch[:, 3] + 31) // 32) * ((keys + 31) // 32)).sum())


def make_layout(seq_offsets: Sequence[int], seq_lens: Sequence[int], chunks, device="cuda",
                max_chunk_len: Optional[int] = None, max_kv_len: Optional[int] = None) -> Layout:
    torch = _torch()
    so = np.ascontiguousarray(seq_offsets, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    ch = np.ascontiguousarray(chunks, dtype=np.int32).reshape(-1, 4)
    mcl = int(ch[:, 3].max()) if len(ch) and max_chunk_len is None else (max_chunk_len or 0)
    mkl = int(sl.max()) if len(sl) and max_kv_len is None else (max_kv_len or 0)
    return Layout(torch.from_numpy(so).to(device), torch.from_numpy(sl).to(device),
                  torch.from_numpy(ch).to(device), len(so), len(ch), max(mcl, 0), max(mkl, 0),
                  ch, sl)


def problem(layout: Layout, q_rows: int, kv_rows: int, hq: int, hkv: int, head_dim: int,
            causal: bool = True, scale: Optional[float] = None, bias_len: int = 0,
            q_head_pitch: int = 0, kv_head_pitch: int = 0) -> Problem:
    dsb = 0
    if layout.host_chunks is not None and layout.host_seq_lens is not None:
        dsb = ds_blocks(layout.host_chunks, layout.host_seq_lens, causal)
    return Problem(layout.num_seqs, hq, hkv, head_dim, q_rows, kv_rows, layout.num_chunks,
                   layout.max_chunk_len, layout.max_kv_len, 1 if causal else 0,
                   (1.0 / math.sqrt(head_dim)) if scale is None else float(scale), bias_len,
                   q_head_pitch, kv_head_pitch, dsb)


def new_dev_err(device="cuda"):
    return _torch().zeros(1, dtype=_torch().int32, device=device)


def check(dev_err) -> None:
    """Synchronize on the error word and raise DeviceError if a promise was broken."""
    bits = int(dev_err.item())
    if bits:
        raise DeviceError(bits)


def workspace_size(prob: Problem, op: int) -> int:
    return int(load().cpattn_workspace_size(ctypes.byref(prob), op))


def _shapes(q, k, v):
    q_rows, hq, D = q.shape
    kv_rows, hkv, D2 = k.shape
    if D2 != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q/k/v head dims or k/v shapes disagree")
    return q_rows, hq, kv_rows, hkv, D


def _prob_for(q, k, v, layout, causal, scale, bias):
    """The problem of q, k, v; each may be a head slice of a larger tensor (head pitch)."""
    torch = _torch()
    q_rows, hq, kv_rows, hkv, D = _shapes(q, k, v)
    qp, kvp = head_pitch(q, "q"), head_pitch(k, "k")
    _need(q, "q", torch.bfloat16, pitch=qp)
    _need(k, "k", torch.bfloat16, pitch=kvp)
    _need(v, "v", torch.bfloat16, pitch=kvp)
    bias_len = 0
    if bias is not None:
        _need(bias, "bias", torch.float32)
        if bias.dim() != 3 or bias.shape[0] != hq or bias.shape[1] != bias.shape[2]:
            raise ValueError("bias must be [hq, bias_len, bias_len]")
        bias_len = int(bias.shape[1])
    return problem(layout, q_rows, kv_rows, hq, hkv, D, causal, scale, bias_len, qp, kvp)


def validate(prob: Problem, layout: Layout, dev_err, stream=None):
    lib = load()
    _check(lib.cpattn_validate(ctypes.byref(prob), _ptr(layout.seq_offsets), _ptr(layout.seq_lens),
                               _ptr(layout.chunks), _ptr(dev_err), _stream(stream)))


def fwd(q, k, v, layout: Layout, causal: bool = True, scale: Optional[float] = None, bias=None,
        o=None, lse=None, dev_err=None, stream=None):
    """O [q_rows, hq, D] bf16 and LSE [hq, q_rows] fp32 (chunk rows written only)."""
    torch = _torch()
    lib = load()
    prob = _prob_for(q, k, v, layout, causal, scale, bias)
    if o is None:
        o = _like(q)
    if lse is None:
        lse = torch.empty((prob.hq, prob.q_rows), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.bfloat16, q.shape, prob.q_head_pitch)
    _need(lse, "lse", torch.float32, (prob.hq, prob.q_rows))
    if dev_err is None:
        dev_err = new_dev_err(q.device)
    _check(lib.cpattn_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(layout.seq_offsets),
                          _ptr(layout.seq_lens), _ptr(layout.chunks), _ptr(bias), _ptr(o), _ptr(lse),
                          None, 0, _ptr(dev_err), _stream(stream)))
    return o, lse, dev_err


def bwd(q, k, v, layout: Layout, o, lse, do, causal: bool = True, scale: Optional[float] = None,
        bias=None, dq=None, dk=None, dv=None, dkv_accumulate: bool = False, want_dbias: bool = True,
        dbias=None, ws=None, dev_err=None, stream=None, store_ds: Optional[bool] = None):
    """dQ, dK, dV (bf16) and dBias (fp32, when a bias is given).

    store_ds: size the workspace for the stored-dS backward (dK/dV stores dS, dQ
    multiplies it); None = whenever the head dim allows it.  A given `ws` decides
    by its size, as in the C entry point."""
    torch = _torch()
    lib = load()
    prob = _prob_for(q, k, v, layout, causal, scale, bias)
    _need(o, "o", torch.bfloat16, q.shape, prob.q_head_pitch)
    _need(do, "do", torch.bfloat16, q.shape, prob.q_head_pitch)
    _need(lse, "lse", torch.float32, (prob.hq, prob.q_rows))
    if dq is None:
        dq = _like(q)
    if dk is None:
        if dkv_accumulate:
            raise ValueError("dkv_accumulate needs existing dk/dv")
        dk = _like(k)
    if dv is None:
        dv = _like(v)
    for n, t, ref, pt in (("dq", dq, q, prob.q_head_pitch), ("dk", dk, k, prob.kv_head_pitch),
                          ("dv", dv, v, prob.kv_head_pitch)):
        _need(t, n, torch.bfloat16, ref.shape, pt)
    if bias is not None and want_dbias and dbias is None:
        dbias = torch.empty_like(bias)
    need = workspace_size(prob, OP_BWD)
    if store_ds is not False and ws is None:
        need = max(need, workspace_size(prob, OP_BWD_DS))
        if store_ds and need == workspace_size(prob, OP_BWD):
            raise ValueError("the stored-dS backward needs head_dim >= 32")
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if dev_err is None:
        dev_err = new_dev_err(q.device)
    _check(lib.cpattn_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(layout.seq_offsets),
                          _ptr(layout.seq_lens), _ptr(layout.chunks), _ptr(bias), _ptr(o), _ptr(lse),
                          _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias),
                          1 if dkv_accumulate else 0, _ptr(ws), ws.numel(), _ptr(dev_err),
                          _stream(stream)))
    return dq, dk, dv, dbias, dev_err


def bwd_noalloc(q, k, v, layout: Layout, o, lse, do, dq, dk, dv, causal: bool = True,
                scale: Optional[float] = None, bias=None, dbias=None, dkv_accumulate: bool = False,
                dev_err=None, stream=None):
    """cpattn_bwd_noalloc: the backward with the library's static scratch as workspace.
    The caller passes every output (nothing is allocated here either)."""
    torch = _torch()
    lib = load()
    prob = _prob_for(q, k, v, layout, causal, scale, bias)
    _need(o, "o", torch.bfloat16, q.shape, prob.q_head_pitch)
    _need(do, "do", torch.bfloat16, q.shape, prob.q_head_pitch)
    _need(lse, "lse", torch.float32, (prob.hq, prob.q_rows))
    for n, t, ref, pt in (("dq", dq, q, prob.q_head_pitch), ("dk", dk, k, prob.kv_head_pitch),
                          ("dv", dv, v, prob.kv_head_pitch)):
        _need(t, n, torch.bfloat16, ref.shape, pt)
    if dev_err is None:
        raise ValueError("bwd_noalloc needs a caller-provided dev_err")
    _check(lib.cpattn_bwd_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(layout.seq_offsets),
                                  _ptr(layout.seq_lens), _ptr(layout.chunks), _ptr(bias), _ptr(o), _ptr(lse),
                                  _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias),
                                  1 if dkv_accumulate else 0, _ptr(dev_err), _stream(stream)))
    return dq, dk, dv, dbias, dev_err


def fwd_window(q, k, v, layout: Layout, kv_lo: int, kv_hi: int, causal: bool = True,
               scale: Optional[float] = None, bias=None, o=None, lse=None, dev_err=None, stream=None):
    """Partial O (bf16) and LSE (fp32) over the keys at positions [kv_lo, kv_hi)."""
    torch = _torch()
    lib = load()
    prob = _prob_for(q, k, v, layout, causal, scale, bias)
    if o is None:
        o = _like(q)
    if lse is None:
        lse = torch.empty((prob.hq, prob.q_rows), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.bfloat16, q.shape, prob.q_head_pitch)
    _need(lse, "lse", torch.float32, (prob.hq, prob.q_rows))
    if dev_err is None:
        dev_err = new_dev_err(q.device)
    _check(lib.cpattn_fwd_window(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(layout.seq_offsets),
                                 _ptr(layout.seq_lens), _ptr(layout.chunks), _ptr(bias), int(kv_lo), int(kv_hi),
                                 _ptr(o), _ptr(lse), _ptr(dev_err), _stream(stream)))
    return o, lse, dev_err


def merge(prob: Problem, layout: Layout, o_a, lse_a, o_b, lse_b, o=None, lse=None, dev_err=None,
          stream=None):
    """Merge two partial results over disjoint key sets; o/lse default to o_a/lse_a (in place)."""
    lib = load()
    if o is None:
        o = o_a
    if lse is None:
        lse = lse_a
    if dev_err is None:
        dev_err = new_dev_err(o_a.device)
    _check(lib.cpattn_merge(ctypes.byref(prob), _ptr(layout.chunks), _ptr(o_a), _ptr(lse_a), _ptr(o_b),
                            _ptr(lse_b), _ptr(o), _ptr(lse), _ptr(dev_err), _stream(stream)))
    return o, lse


def bwd_window(q, k, v, layout: Layout, o, lse, do, kv_lo: int, kv_hi: int, causal: bool = True,
               scale: Optional[float] = None, bias=None, prepass: bool = True, dq=None,
               dq_accumulate: bool = False, dk=None, dv=None, dkv_accumulate: bool = False, ws=None,
               dev_err=None, stream=None, store_ds: Optional[bool] = None):
    """The key window [kv_lo, kv_hi)'s dQ share (store or add) and its keys' dK/dV.

    store_ds: size a new workspace for the stored-dS path (dK/dV store the window's dS,
    the dQ share multiplies it); None = whenever the head dim allows it.  A given `ws`
    decides by its size."""
    torch = _torch()
    lib = load()
    prob = _prob_for(q, k, v, layout, causal, scale, bias)
    if dq is None:
        if dq_accumulate:
            raise ValueError("dq_accumulate needs an existing dq")
        dq = _like(q)
    if dk is None:
        if dkv_accumulate:
            raise ValueError("dkv_accumulate needs existing dk/dv")
        dk = _like(k)
    if dv is None:
        dv = _like(v)
    need = workspace_size(prob, OP_BWD)
    if store_ds is not False:
        need = max(need, workspace_size(prob, OP_BWD_DS))
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if dev_err is None:
        dev_err = new_dev_err(q.device)
    _check(lib.cpattn_bwd_window(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(layout.seq_offsets),
                                 _ptr(layout.seq_lens), _ptr(layout.chunks), _ptr(bias), _ptr(o), _ptr(lse),
                                 _ptr(do), int(kv_lo), int(kv_hi), 1 if prepass else 0, _ptr(dq),
                                 1 if dq_accumulate else 0, _ptr(dk), _ptr(dv), 1 if dkv_accumulate else 0,
                                 _ptr(ws), ws.numel(), _ptr(dev_err), _stream(stream)))
    return dq, dk, dv, ws, dev_err


def bwd_prepass(prob: Problem, layout: Layout, q, o, do, lse, ws, dev_err, stream=None):
    """Delta, the transposed Q/dO tiles and their row statistics into the backward
    workspace `ws` (uint8)."""
    lib = load()
    _check(lib.cpattn_bwd_prepass(ctypes.byref(prob), _ptr(q), _ptr(layout.chunks), _ptr(o), _ptr(do),
                                  _ptr(lse), _ptr(ws), ws.numel(), _ptr(dev_err), _stream(stream)))


def bwd_dkdv(prob: Problem, layout: Layout, q, k, v, bias, lse, do, ws, dk, dv,
             dkv_accumulate: bool, dev_err, stream=None):
    lib = load()
    _check(lib.cpattn_bwd_dkdv(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(layout.seq_offsets),
                               _ptr(layout.seq_lens), _ptr(layout.chunks), _ptr(bias), _ptr(lse),
                               _ptr(do), _ptr(ws), ws.numel(), _ptr(dk), _ptr(dv),
                               1 if dkv_accumulate else 0, _ptr(dev_err), _stream(stream)))


def bwd_dq(prob: Problem, layout: Layout, q, k, v, bias, lse, do, ws, dq, dev_err, stream=None):
    lib = load()
    _check(lib.cpattn_bwd_dq(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(layout.seq_offsets),
                             _ptr(layout.seq_lens), _ptr(layout.chunks), _ptr(bias), _ptr(lse),
                             _ptr(do), _ptr(ws), ws.numel(), _ptr(dq), _ptr(dev_err), _stream(stream)))


def bwd_dkdv_ds(prob: Problem, layout: Layout, q, k, v, bias, lse, do, ws, dk, dv,
                dkv_accumulate: bool, dev_err, stream=None):
    """bwd_dkdv that also stores dS in the workspace (OP_BWD_DS bytes)."""
    lib = load()
    _check(lib.cpattn_bwd_dkdv_ds(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(layout.seq_offsets),
                                  _ptr(layout.seq_lens), _ptr(layout.chunks), _ptr(bias), _ptr(lse),
                                  _ptr(do), _ptr(ws), ws.numel(), _ptr(dk), _ptr(dv),
                                  1 if dkv_accumulate else 0, _ptr(dev_err), _stream(stream)))


def bwd_dq_ds(prob: Problem, layout: Layout, k, ws, dq, dev_err, stream=None):
    """dQ from the dS that bwd_dkdv_ds stored in `ws`."""
    lib = load()
    _check(lib.cpattn_bwd_dq_ds(ctypes.byref(prob), _ptr(k), _ptr(layout.seq_offsets), _ptr(layout.seq_lens),
                                _ptr(layout.chunks), _ptr(ws), ws.numel(), _ptr(dq), _ptr(dev_err),
                                _stream(stream)))


def bwd_dbias_ds(prob: Problem, layout: Layout, ws, dbias, dev_err, stream=None):
    """dBias summed from the dS that bwd_dkdv_ds stored in `ws`."""
    lib = load()
    _check(lib.cpattn_bwd_dbias_ds(ctypes.byref(prob), _ptr(layout.seq_offsets), _ptr(layout.seq_lens),
                                   _ptr(layout.chunks), _ptr(ws), ws.numel(), _ptr(dbias), _ptr(dev_err),
                                   _stream(stream)))


def bwd_dbias(prob: Problem, layout: Layout, q, k, v, bias, lse, do, ws, dbias, dev_err, stream=None):
    lib = load()
    _check(lib.cpattn_bwd_dbias(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(layout.seq_offsets),
                                _ptr(layout.seq_lens), _ptr(layout.chunks), _ptr(bias), _ptr(lse),
                                _ptr(do), _ptr(ws), ws.numel(), _ptr(dbias), _ptr(dev_err),
                                _stream(stream)))


def pack(bhsd, seq_offsets, seq_lens, thd_rows: int, thd=None, dev_err=None, stream=None):
    """THD [thd_rows, H, D] from BHSD [B, H, S_pitch, D]; only valid rows are written."""
    torch = _torch()
    lib = load()
    _need(bhsd, "bhsd", torch.bfloat16)
    B, H, S, D = bhsd.shape
    if thd is None:
        thd = torch.empty((thd_rows, H, D), dtype=torch.bfloat16, device=bhsd.device)
    _need(thd, "thd", torch.bfloat16, (thd_rows, H, D))
    if dev_err is None:
        dev_err = new_dev_err(bhsd.device)
    _check(lib.cpattn_pack(_ptr(bhsd), _ptr(thd), B, H, S, D, thd_rows, _ptr(seq_offsets),
                           _ptr(seq_lens), _ptr(dev_err), _stream(stream)))
    return thd, dev_err


def unpack(thd, seq_offsets, seq_lens, B: int, S_pitch: int, bhsd=None, dev_err=None, stream=None):
    """BHSD [B, H, S_pitch, D] from THD [thd_rows, H, D]; only valid rows are written."""
    torch = _torch()
    lib = load()
    _need(thd, "thd", torch.bfloat16)
    thd_rows, H, D = thd.shape
    if bhsd is None:
        bhsd = torch.empty((B, H, S_pitch, D), dtype=torch.bfloat16, device=thd.device)
    _need(bhsd, "bhsd", torch.bfloat16, (B, H, S_pitch, D))
    if dev_err is None:
        dev_err = new_dev_err(thd.device)
    _check(lib.cpattn_unpack(_ptr(thd), _ptr(bhsd), B, H, S_pitch, D, thd_rows, _ptr(seq_offsets),
                             _ptr(seq_lens), _ptr(dev_err), _stream(stream)))
    return bhsd, dev_err


# ---------------------------------------------------------------- A2A swap copies

def a2a_split_heads(src, cp: int, dst=None, stream=None):
    """[rows, H, D] -> [cp, rows, H / cp, D]: block j holds heads [j H/cp, (j+1) H/cp)."""
    torch = _torch()
    _need(src, "src", torch.bfloat16)
    rows, H, D = src.shape
    if H % cp:
        raise ValueError(f"H ({H}) is not a multiple of cp ({cp})")
    if dst is None:
        dst = torch.empty((cp, rows, H // cp, D), dtype=torch.bfloat16, device=src.device)
    _need(dst, "dst", torch.bfloat16, (cp, rows, H // cp, D))
    _check(load().cpattn_a2a_split_heads(_ptr(src), _ptr(dst), rows, H, D, cp, _stream(stream)))
    return dst


def a2a_merge_heads(src, dst=None, stream=None):
    """[cp, rows, Hc, D] -> [rows, cp Hc, D]: the inverse of a2a_split_heads."""
    torch = _torch()
    _need(src, "src", torch.bfloat16)
    cp, rows, Hc, D = src.shape
    if dst is None:
        dst = torch.empty((rows, cp * Hc, D), dtype=torch.bfloat16, device=src.device)
    _need(dst, "dst", torch.bfloat16, (rows, cp * Hc, D))
    _check(load().cpattn_a2a_merge_heads(_ptr(src), _ptr(dst), rows, cp * Hc, D, cp, _stream(stream)))
    return dst


@dataclasses.dataclass
class A2aLayout:
    """Rank maps and sequence descriptors of an A2A swap on the device, with host bounds."""
    rank_maps: object     # int32 [cp, chunks_per_rank, 4] {seq, q_row, pos0, len}
    seq_offsets: object   # int32 [B]: row of position 0 in the sequence-ordered tensor
    seq_lens: object      # int32 [B]
    cp: int
    chunks_per_rank: int
    num_seqs: int
    max_chunk_len: int


def make_a2a_layout(rank_maps, seq_offsets, seq_lens, device="cuda") -> A2aLayout:
    """rank_maps: one [C_r, 4] array per rank; shorter maps are padded with len = 0."""
    torch = _torch()
    maps = [np.asarray(m, np.int32).reshape(-1, 4) for m in rank_maps]
    C = max((len(m) for m in maps), default=0)
    arr = np.zeros((len(maps), C, 4), np.int32)
    for r, m in enumerate(maps):
        arr[r, :len(m)] = m
    mcl = int(arr[..., 3].max()) if arr.size else 0
    so = np.ascontiguousarray(seq_offsets, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    return A2aLayout(torch.from_numpy(arr).to(device), torch.from_numpy(so).to(device),
                     torch.from_numpy(sl).to(device), len(maps), C, len(so), max(mcl, 0))


def _a2a_rows(lay: A2aLayout, rows_per_rank: int, full_rows: int, heads: int, D: int) -> A2aRows:
    return A2aRows(lay.cp, lay.chunks_per_rank, lay.num_seqs, lay.max_chunk_len, rows_per_rank,
                   full_rows, heads, D)


def a2a_scatter_rows(blocks, lay: A2aLayout, full_rows: int, full=None, dev_err=None, stream=None):
    """Blocks [cp, rows_per_rank, Hc, D] received from every rank -> the sequence-ordered
    [full_rows, Hc, D] tensor; rows no chunk names keep their contents."""
    torch = _torch()
    _need(blocks, "blocks", torch.bfloat16)
    cp, rpr, Hc, D = blocks.shape
    if cp != lay.cp:
        raise ValueError(f"blocks hold {cp} ranks, the layout {lay.cp}")
    if full is None:
        full = torch.empty((full_rows, Hc, D), dtype=torch.bfloat16, device=blocks.device)
    _need(full, "full", torch.bfloat16, (full_rows, Hc, D))
    if dev_err is None:
        dev_err = new_dev_err(blocks.device)
    p = _a2a_rows(lay, rpr, full_rows, Hc, D)
    _check(load().cpattn_a2a_scatter_rows(ctypes.byref(p), _ptr(blocks), _ptr(full), _ptr(lay.rank_maps),
                                          _ptr(lay.seq_offsets), _ptr(lay.seq_lens), _ptr(dev_err),
                                          _stream(stream)))
    return full, dev_err


def a2a_gather_rows(full, lay: A2aLayout, rows_per_rank: int, blocks=None, dev_err=None, stream=None):
    """The sequence-ordered [full_rows, Hc, D] tensor -> blocks [cp, rows_per_rank, Hc, D],
    block s holding rank s's rows; rows no chunk names keep their contents."""
    torch = _torch()
    _need(full, "full", torch.bfloat16)
    full_rows, Hc, D = full.shape
    if blocks is None:
        blocks = torch.empty((lay.cp, rows_per_rank, Hc, D), dtype=torch.bfloat16, device=full.device)
    _need(blocks, "blocks", torch.bfloat16, (lay.cp, rows_per_rank, Hc, D))
    if dev_err is None:
        dev_err = new_dev_err(full.device)
    p = _a2a_rows(lay, rows_per_rank, full_rows, Hc, D)
    _check(load().cpattn_a2a_gather_rows(ctypes.byref(p), _ptr(full), _ptr(blocks), _ptr(lay.rank_maps),
                                         _ptr(lay.seq_offsets), _ptr(lay.seq_lens), _ptr(dev_err),
                                         _stream(stream)))
    return blocks, dev_err


# ---------------------------------------------------------------- host <-> device helpers

def to_device_bf16(bits: np.ndarray, device="cuda"):
    """BF16 bit patterns (uint16 numpy) -> torch.bfloat16 device tensor, bit-exact."""
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_host_bits(t) -> np.ndarray:
    """torch.bfloat16 tensor -> uint16 numpy bit patterns."""
    torch = _torch()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
