"""ctypes binding of libattn.so (C ABI declared in include/attn.h).

Argument marshalling only: every step of the computation runs in the HIP kernels of the library.
torch supplies device memory (outputs, workspace) and the current stream. There is no CPU
fallback: if the library is missing this module raises when it is first used.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_LIB_PATH = os.environ.get("ATTN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

# status codes (attn_status)
ATTN_OK = 0
ATTN_ERR_NULL = 1
ATTN_ERR_SHAPE = 2
ATTN_ERR_ALIGN = 3
ATTN_ERR_DTYPE = 4
ATTN_ERR_MASK = 5
ATTN_ERR_WORKSPACE = 6
ATTN_ERR_ALIAS = 7
ATTN_ERR_UNSUPPORTED = 8
ATTN_ERR_HIP = 9

ATTN_F32 = 0
ATTN_BF16 = 1
ATTN_FP8_E4M3 = 2  # forward inputs only; O is bf16

ATTN_BWD_ATOMIC_DQ = 1  # attn_bwd_ex flag: single-pass backward with atomic fp32 dQ accumulation

MASK_KINDS = {"none": 0, "causal": 1, "padding": 2, "block": 3, "dense": 4}

EXPORTED = ("attn_fwd", "attn_bwd", "attn_fwd_workspace_bytes", "attn_bwd_workspace_bytes",
            "attn_status_string", "attn_version")


class AttnProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("seq_q", ctypes.c_int32), ("seq_k", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class AttnMask(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("lengths", ctypes.c_void_p), ("block_layout", ctypes.c_void_p),
                ("layout_stride_b", ctypes.c_int64), ("layout_stride_h", ctypes.c_int64),
                ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32), ("dense", ctypes.c_void_p),
                ("dense_stride_b", ctypes.c_int64), ("dense_stride_h", ctypes.c_int64)]


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libattn status {status}: {message}")
        self.status = status


_lib = None


def load_library(path: str = _LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so once and declare the C signatures. Raises if the library is missing.

    The default is the in-tree build next to this file; the ATTN_LIBRARY environment variable
    names another build of the same library (used to compare kernel variants)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libattn.so not found at {path}; build it with "
                           "`python -m attention_attn_fwd_09_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pp, pm = ctypes.POINTER(AttnProblem), ctypes.POINTER(AttnMask)
    lib.attn_fwd_workspace_bytes.argtypes = [pp, pm]
    lib.attn_fwd_workspace_bytes.restype = sz
    lib.attn_bwd_workspace_bytes.argtypes = [pp, pm]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_fwd.argtypes = [pp, vp, vp, vp, pm, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_ex.argtypes = [pp, vp, vp, vp, pm, ctypes.c_float, vp, vp, vp, sz, ctypes.c_int32, vp]
    lib.attn_fwd_ex.restype = ctypes.c_int
    lib.attn_fwd_ex_workspace_bytes.argtypes = [pp, pm, ctypes.c_int32]
    lib.attn_fwd_ex_workspace_bytes.restype = sz
    lib.attn_fwd_kv_splits.argtypes = [pp, pm, ctypes.c_int32]
    lib.attn_fwd_kv_splits.restype = ctypes.c_int32
    lib.attn_bwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, pm, ctypes.c_float, vp, vp, vp, vp, sz, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_ex.argtypes = [pp, vp, vp, vp, vp, vp, vp, pm, ctypes.c_float, vp, vp, vp, vp, sz, ctypes.c_int32,
                                vp]
    lib.attn_bwd_ex.restype = ctypes.c_int
    lib.attn_bwd_ex_workspace_bytes.argtypes = [pp, pm, ctypes.c_int32]
    lib.attn_bwd_ex_workspace_bytes.restype = sz
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(status).decode()


@dataclass
class Mask:
    """Mask descriptor: kind in {"none", "causal", "padding", "block", "dense"}.

    lengths: int32 device tensor [batch] (padding). layout: uint8 device tensor, [nb_q, nb_k]
    shared by all (b, h), or [batch, heads_q, nb_q, nb_k] (block, 64x64 tiles). dense: uint8 (or
    bool) device tensor [seq_q, seq_k] shared by all (b, h), or [batch, heads_q, seq_q, seq_k];
    non-zero keeps the pair (dense).
    """

    kind: str = "none"
    lengths: Optional[torch.Tensor] = None
    layout: Optional[torch.Tensor] = None
    block: int = 64
    dense: Optional[torch.Tensor] = None

    def to_c(self) -> AttnMask:
        m = AttnMask()
        m.kind = MASK_KINDS[self.kind]
        m.block_q = m.block_k = self.block
        if self.lengths is not None:
            m.lengths = self.lengths.data_ptr()
        if self.layout is not None:
            m.block_layout = self.layout.data_ptr()
            if self.layout.dim() == 4:
                m.layout_stride_b = self.layout.stride(0)
                m.layout_stride_h = self.layout.stride(1)
        if self.dense is not None:
            if self.dense.element_size() != 1 or not self.dense.is_contiguous():
                raise ValueError("dense mask must be a contiguous uint8 or bool tensor")
            m.dense = self.dense.data_ptr()
            if self.dense.dim() == 4:
                m.dense_stride_b = self.dense.stride(0)
                m.dense_stride_h = self.dense.stride(1)
        return m


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float8_e4m3fn:
        return ATTN_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _problem(q: torch.Tensor, k: torch.Tensor) -> AttnProblem:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [batch, heads, seq, head_dim]")
    p = AttnProblem()
    p.batch, p.heads_q, p.seq_q, p.head_dim = q.shape
    p.heads_kv, p.seq_k = k.shape[1], k.shape[2]
    p.dtype = _dtype_code(q)
    return p


def _check_tensors(*ts: torch.Tensor):
    dev = ts[0].device
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("libattn needs contiguous tensors")
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")


def _stream_ptr(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _raise(status: int):
    if status != ATTN_OK:
        raise AttnError(status, attn_status_string(status))


def attn_fwd_workspace_bytes(q: torch.Tensor, k: torch.Tensor, mask: Optional[Mask] = None,
                             kv_splits: int = 0) -> int:
    lib = load_library()
    m = (mask or Mask()).to_c()
    return int(lib.attn_fwd_ex_workspace_bytes(ctypes.byref(_problem(q, k)), ctypes.byref(m), int(kv_splits)))


def attn_fwd_kv_splits(q: torch.Tensor, k: torch.Tensor, mask: Optional[Mask] = None, kv_splits: int = 0) -> int:
    """Number of key-range splits attn_fwd would use (0 for an invalid problem)."""
    lib = load_library()
    m = (mask or Mask()).to_c()
    return int(lib.attn_fwd_kv_splits(ctypes.byref(_problem(q, k)), ctypes.byref(m), int(kv_splits)))


def attn_bwd_workspace_bytes(q: torch.Tensor, k: torch.Tensor, mask: Optional[Mask] = None, flags: int = 0) -> int:
    lib = load_library()
    m = (mask or Mask()).to_c()
    return int(lib.attn_bwd_ex_workspace_bytes(ctypes.byref(_problem(q, k)), ctypes.byref(m), int(flags)))


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: Optional[Mask] = None,
             scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None,
             kv_splits: int = 0):
    """Forward: returns (O, LSE). O has q's dtype; LSE is float32 [batch, heads_q, seq_q].

    kv_splits: 0 lets the library choose a split of each item's key range, 1 never splits,
    n > 1 forces n splits (attn_fwd_ex)."""
    lib = load_library()
    _check_tensors(q, k, v)
    mask = mask or Mask()
    prob = _problem(q, k)
    cm = mask.to_c()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype,
                          device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    need = int(lib.attn_fwd_ex_workspace_bytes(ctypes.byref(prob), ctypes.byref(cm), int(kv_splits)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.attn_fwd_ex(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(cm),
                         float(scale), out.data_ptr(), lse.data_ptr(), ws_ptr, ws_bytes, int(kv_splits),
                         _stream_ptr(stream))
    _raise(st)
    return out, lse


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, do: torch.Tensor,
             lse: torch.Tensor, mask: Optional[Mask] = None, scale: Optional[float] = None,
             dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None,
             flags: int = 0):
    """Backward: returns (dQ, dK, dV) in q's dtype.

    flags: 0 (two passes, deterministic) or ATTN_BWD_ATOMIC_DQ (single pass, dQ accumulated with
    fp32 atomics; attn_bwd_ex)."""
    lib = load_library()
    _check_tensors(q, k, v, o, do, lse)
    mask = mask or Mask()
    prob = _problem(q, k)
    cm = mask.to_c()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = int(lib.attn_bwd_ex_workspace_bytes(ctypes.byref(prob), ctypes.byref(cm), int(flags)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.attn_bwd_ex(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                         do.data_ptr(), lse.data_ptr(), ctypes.byref(cm), float(scale), dq.data_ptr(), dk.data_ptr(),
                         dv.data_ptr(), ws_ptr, ws_bytes, int(flags), _stream_ptr(stream))
    _raise(st)
    return dq, dk, dv
