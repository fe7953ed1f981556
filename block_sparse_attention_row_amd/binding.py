"""ctypes binding of libsparse_attn.so (argument marshalling only).

Every computation runs in the HIP kernels behind the C-ABI declared in
``include/sparse_attn.h``; this module only turns torch tensors into
pointers, sizes and the caller's stream.  There is no fallback: if the
library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_attn.so")

SPARSE_ATTN_F32 = 0
SPARSE_ATTN_BF16 = 1

SPARSE_ATTN_OK = 0
SPARSE_ATTN_INVALID_ARGUMENT = -1
SPARSE_ATTN_UNSUPPORTED = -2
SPARSE_ATTN_CAPACITY = -3
SPARSE_ATTN_WORKSPACE = -4
SPARSE_ATTN_HIP_ERROR = -5

EXPORTED = (
    "sparse_attn_version",
    "sparse_attn_status_string",
    "sparse_attn_csr_capacity",
    "sparse_attn_workspace_size",
    "sparse_attn_select",
    "sparse_attn_select_sip",
    "sparse_attn_select_ibcs",
    "sparse_attn_forward",
    "sparse_attn_forward_biased",
    "sparse_attn_mask_to_csr",
    "sparse_attn_radial_csr",
    "sparse_attn_backward",
    "sparse_attn_full_csr",
    "sparse_attn_to_tiles",
    "sparse_attn_from_tiles",
    "sparse_attn_select_raster",
)


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("grid_t", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
        ("tile_t", ctypes.c_int32), ("tile_h", ctypes.c_int32), ("tile_w", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
    ]


class SelectParams(ctypes.Structure):
    _fields_ = [
        ("threshold", ctypes.c_float),
        ("head_thresholds", ctypes.POINTER(ctypes.c_float)),
        ("win_t", ctypes.c_int32), ("win_h", ctypes.c_int32), ("win_w", ctypes.c_int32),
    ]


class RadialParams(ctypes.Structure):
    _fields_ = [("r0", ctypes.c_float), ("gamma", ctypes.c_float), ("lambda_", ctypes.c_int32)]


class SipParams(ctypes.Structure):
    _fields_ = [("budget", ctypes.c_float), ("seed", ctypes.c_uint64)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_row_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        SP = ctypes.POINTER(Shape)
        L.sparse_attn_version.argtypes = []
        L.sparse_attn_version.restype = ctypes.c_int32
        L.sparse_attn_status_string.argtypes = [ctypes.c_int32]
        L.sparse_attn_status_string.restype = ctypes.c_char_p
        L.sparse_attn_csr_capacity.argtypes = [SP]
        L.sparse_attn_csr_capacity.restype = I64
        L.sparse_attn_workspace_size.argtypes = [SP]
        L.sparse_attn_workspace_size.restype = I64
        L.sparse_attn_select.argtypes = [SP, ctypes.POINTER(SelectParams), P, P, P, P, I64, P, I64, P]
        L.sparse_attn_select.restype = ctypes.c_int32
        L.sparse_attn_select_sip.argtypes = [SP, ctypes.POINTER(SipParams), P, P, P, P, P, I64, P, I64, P]
        L.sparse_attn_select_sip.restype = ctypes.c_int32
        L.sparse_attn_select_ibcs.argtypes = [SP, ctypes.POINTER(SelectParams), P, P, P, P, I64, P, I64, P]
        L.sparse_attn_select_ibcs.restype = ctypes.c_int32
        L.sparse_attn_forward.argtypes = [SP, P, P, P, P, P, I64, P, P, P, I64, P]
        L.sparse_attn_forward.restype = ctypes.c_int32
        L.sparse_attn_forward_biased.argtypes = [SP, P, P, P, P, P, P, I64, P, P, P, I64, P]
        L.sparse_attn_forward_biased.restype = ctypes.c_int32
        L.sparse_attn_mask_to_csr.argtypes = [SP, P, P, P, I64, P, I64, P]
        L.sparse_attn_mask_to_csr.restype = ctypes.c_int32
        L.sparse_attn_radial_csr.argtypes = [SP, ctypes.POINTER(RadialParams), P, P, I64, P, I64, P]
        L.sparse_attn_radial_csr.restype = ctypes.c_int32
        L.sparse_attn_backward.argtypes = [SP, P, P, P, P, P, P, P, P, I64, P, P, P, P, P, I64, P]
        L.sparse_attn_backward.restype = ctypes.c_int32
        L.sparse_attn_full_csr.argtypes = [SP, P, P, I64, P]
        L.sparse_attn_full_csr.restype = ctypes.c_int32
        L.sparse_attn_select_raster.argtypes = [SP, ctypes.POINTER(SelectParams), P, P, P, P, P, P, I64, P, I64, P]
        L.sparse_attn_select_raster.restype = ctypes.c_int32
        for name in ("sparse_attn_to_tiles", "sparse_attn_from_tiles"):
            getattr(L, name).argtypes = [SP, P, P, P]
            getattr(L, name).restype = ctypes.c_int32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sparse_attn_status_string(int(status)).decode()


def sparse_attn_version() -> int:
    return int(lib().sparse_attn_version())


def make_shape(batch, heads, head_dim, grid, dtype, scale=0.0, tile=(1, 8, 8)) -> Shape:
    code = {"f32": SPARSE_ATTN_F32, "bf16": SPARSE_ATTN_BF16}.get(dtype, dtype)
    return Shape(int(batch), int(heads), int(head_dim), *(int(g) for g in grid), *(int(t) for t in tile),
                 int(code), float(scale))


def shape_of(q, grid, scale=0.0, tile=(1, 8, 8)) -> Shape:
    import torch
    B, H, N, d = q.shape
    dt = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(q.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return make_shape(B, H, d, grid, dt, scale, tile)


def sparse_attn_csr_capacity(shape: Shape) -> int:
    return int(lib().sparse_attn_csr_capacity(ctypes.byref(shape)))


def sparse_attn_workspace_size(shape: Shape) -> int:
    return int(lib().sparse_attn_workspace_size(ctypes.byref(shape)))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    return int(getattr(stream, "cuda_stream", stream))


def _check(status: int, where: str):
    if status != SPARSE_ATTN_OK:
        raise SparseAttnError(status, where)


@dataclass
class Buffers:
    """Caller-owned device buffers for one shape (the library allocates nothing)."""
    workspace: "object"
    row_ptr: "object"
    col_idx: "object"


def alloc_buffers(shape: Shape, device="cuda") -> Buffers:
    import torch
    ws = sparse_attn_workspace_size(shape)
    cap = sparse_attn_csr_capacity(shape)
    if ws < 0 or cap < 0:
        raise SparseAttnError(min(ws, cap), "shape")
    nb = shape.grid_t * shape.grid_h * shape.grid_w // 64
    rows = shape.batch * shape.heads * nb
    return Buffers(torch.empty(ws, dtype=torch.uint8, device=device),
                   torch.empty(rows + 1, dtype=torch.int32, device=device),
                   torch.empty(cap, dtype=torch.int32, device=device))


def sparse_attn_select(shape: Shape, q, k, threshold: float = 0.9,
                       head_thresholds: Optional[Sequence[float]] = None, window=(-1, -1, -1),
                       buffers: Optional[Buffers] = None, stream=None) -> Tuple[object, object]:
    """Run the selection; returns (row_ptr, col_idx) views of the caller-owned buffers."""
    bufs = buffers or alloc_buffers(shape, q.device)
    ht = None
    if head_thresholds is not None:
        arr = (ctypes.c_float * shape.heads)(*[float(x) for x in head_thresholds])
        ht = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    params = SelectParams(float(threshold), ht, *(int(w) for w in window))
    st = lib().sparse_attn_select(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k),
                                  _ptr(bufs.row_ptr), _ptr(bufs.col_idx), bufs.col_idx.numel(),
                                  _ptr(bufs.workspace), bufs.workspace.numel(), _stream(stream))
    _check(st, "sparse_attn_select")
    return bufs.row_ptr, bufs.col_idx


def sparse_attn_select_raster(shape: Shape, q, k, q_tiles=None, k_tiles=None, threshold: float = 0.9,
                              head_thresholds: Optional[Sequence[float]] = None, window=(-1, -1, -1),
                              buffers: Optional[Buffers] = None, stream=None):
    """The selection on raster-ordered q, k, with the tile-major copies written on the way;
    returns (row_ptr, col_idx, q_tiles, k_tiles)."""
    import torch
    bufs = buffers or alloc_buffers(shape, q.device)
    q_tiles = torch.empty_like(q) if q_tiles is None else q_tiles
    k_tiles = torch.empty_like(k) if k_tiles is None else k_tiles
    ht = None
    if head_thresholds is not None:
        arr = (ctypes.c_float * shape.heads)(*[float(x) for x in head_thresholds])
        ht = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    params = SelectParams(float(threshold), ht, *(int(w) for w in window))
    st = lib().sparse_attn_select_raster(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(q_tiles),
                                         _ptr(k_tiles), _ptr(bufs.row_ptr), _ptr(bufs.col_idx),
                                         bufs.col_idx.numel(), _ptr(bufs.workspace), bufs.workspace.numel(),
                                         _stream(stream))
    _check(st, "sparse_attn_select_raster")
    return bufs.row_ptr, bufs.col_idx, q_tiles, k_tiles


def sparse_attn_select_ibcs(shape: Shape, q, k, threshold: float = 0.9,
                            head_thresholds: Optional[Sequence[float]] = None, window=(-1, -1, -1),
                            buffers: Optional[Buffers] = None, stream=None) -> Tuple[object, object]:
    """The clustering selector with NABLA's CDF cut; returns (row_ptr, col_idx)."""
    bufs = buffers or alloc_buffers(shape, q.device)
    ht = None
    if head_thresholds is not None:
        arr = (ctypes.c_float * shape.heads)(*[float(x) for x in head_thresholds])
        ht = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    params = SelectParams(float(threshold), ht, *(int(w) for w in window))
    st = lib().sparse_attn_select_ibcs(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k),
                                       _ptr(bufs.row_ptr), _ptr(bufs.col_idx), bufs.col_idx.numel(),
                                       _ptr(bufs.workspace), bufs.workspace.numel(), _stream(stream))
    _check(st, "sparse_attn_select_ibcs")
    return bufs.row_ptr, bufs.col_idx


def sparse_attn_select_sip(shape: Shape, q, k, budget: float, seed: int = 0, buffers: Optional[Buffers] = None,
                           col_bias=None, stream=None):
    """Sampling with inclusion probabilities; returns (row_ptr, col_idx, col_bias), the
    first two views of the caller-owned buffers, col_bias fp32 of their capacity."""
    import torch
    bufs = buffers or alloc_buffers(shape, q.device)
    if col_bias is None:
        col_bias = torch.empty(bufs.col_idx.numel(), dtype=torch.float32, device=q.device)
    if col_bias.numel() < bufs.col_idx.numel() or col_bias.dtype != torch.float32:
        raise ValueError("col_bias must be float32 with the capacity of col_idx")
    params = SipParams(float(budget), int(seed) & 0xFFFFFFFFFFFFFFFF)
    st = lib().sparse_attn_select_sip(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k),
                                      _ptr(bufs.row_ptr), _ptr(bufs.col_idx), _ptr(col_bias), bufs.col_idx.numel(),
                                      _ptr(bufs.workspace), bufs.workspace.numel(), _stream(stream))
    _check(st, "sparse_attn_select_sip")
    return bufs.row_ptr, bufs.col_idx, col_bias


def sparse_attn_forward(shape: Shape, q, k, v, row_ptr, col_idx, out=None, lse=None, want_lse: bool = False,
                        workspace=None, stream=None):
    """Block-sparse attention; returns out (and lse when requested)."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        B, H, N, _ = q.shape
        lse = torch.empty(B, H, N, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(sparse_attn_workspace_size(shape), dtype=torch.uint8, device=q.device)
    st = lib().sparse_attn_forward(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr), _ptr(col_idx),
                                   col_idx.numel(), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                   _stream(stream))
    _check(st, "sparse_attn_forward")
    return (out, lse) if (want_lse or lse is not None) else out


def sparse_attn_forward_biased(shape: Shape, q, k, v, row_ptr, col_idx, col_bias, out=None, lse=None,
                               want_lse: bool = False, workspace=None, stream=None):
    """Block-sparse attention with a logit offset per col_idx entry (fp32 col_bias)."""
    import torch
    if col_bias.numel() < col_idx.numel() or col_bias.dtype != torch.float32:
        raise ValueError("col_bias must be float32 with one value per col_idx entry")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        B, H, N, _ = q.shape
        lse = torch.empty(B, H, N, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(sparse_attn_workspace_size(shape), dtype=torch.uint8, device=q.device)
    st = lib().sparse_attn_forward_biased(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr),
                                          _ptr(col_idx), _ptr(col_bias), col_idx.numel(), _ptr(out), _ptr(lse),
                                          _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "sparse_attn_forward_biased")
    return (out, lse) if (want_lse or lse is not None) else out


def sparse_attn_radial_csr(shape: Shape, r0: float, gamma: float, lam: int = 0, buffers: Optional[Buffers] = None,
                           device=None, stream=None):
    """DynamicRad's radial window as a block list -> (row_ptr, col_idx)."""
    bufs = buffers or alloc_buffers(shape, device or "cuda")
    params = RadialParams(float(r0), float(gamma), int(lam))
    st = lib().sparse_attn_radial_csr(ctypes.byref(shape), ctypes.byref(params), _ptr(bufs.row_ptr),
                                      _ptr(bufs.col_idx), bufs.col_idx.numel(), _ptr(bufs.workspace),
                                      bufs.workspace.numel(), _stream(stream))
    _check(st, "sparse_attn_radial_csr")
    return bufs.row_ptr, bufs.col_idx


def sparse_attn_mask_to_csr(shape: Shape, block_mask, buffers: Optional[Buffers] = None, stream=None):
    """Dense uint8 block mask [B, H, nB, nB] -> (row_ptr, col_idx)."""
    bufs = buffers or alloc_buffers(shape, block_mask.device)
    st = lib().sparse_attn_mask_to_csr(ctypes.byref(shape), _ptr(block_mask), _ptr(bufs.row_ptr),
                                       _ptr(bufs.col_idx), bufs.col_idx.numel(), _ptr(bufs.workspace),
                                       bufs.workspace.numel(), _stream(stream))
    _check(st, "sparse_attn_mask_to_csr")
    return bufs.row_ptr, bufs.col_idx


def sparse_attn_backward(shape: Shape, q, k, v, out, lse, dout, row_ptr, col_idx, workspace=None, t_idx=None,
                         stream=None, grads=None):
    """Gradients (dq, dk, dv) of sparse_attn_forward for the upstream gradient dout
    (written into `grads` = (dq, dk, dv) when given)."""
    import torch
    ws = workspace if workspace is not None else torch.empty(sparse_attn_workspace_size(shape), dtype=torch.uint8,
                                                              device=q.device)
    cc = col_idx.numel()
    t_idx = t_idx if t_idx is not None else torch.empty(max(cc, 1), dtype=torch.int32, device=q.device)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    for g in (dq, dk, dv):
        if g.shape != q.shape or g.dtype != q.dtype or g.device != q.device or not g.is_contiguous():
            raise ValueError("gradient outputs must be contiguous tensors like q")
    st = lib().sparse_attn_backward(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                                    _ptr(row_ptr), _ptr(col_idx), cc, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(t_idx),
                                    _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "sparse_attn_backward")
    return dq, dk, dv


def sparse_attn_full_csr(shape: Shape, buffers: Optional[Buffers] = None, device=None, stream=None):
    """The dense block list (every query block keeps every key block) -> (row_ptr, col_idx)."""
    bufs = buffers or alloc_buffers(shape, device or "cuda")
    st = lib().sparse_attn_full_csr(ctypes.byref(shape), _ptr(bufs.row_ptr), _ptr(bufs.col_idx), bufs.col_idx.numel(),
                                    _stream(stream))
    _check(st, "sparse_attn_full_csr")
    return bufs.row_ptr, bufs.col_idx


def sparse_attn_to_tiles(shape: Shape, src, dst=None, stream=None):
    """Raster-ordered [B, H, N, d] -> tile-major (a new tensor unless dst is given)."""
    import torch
    dst = torch.empty_like(src) if dst is None else dst
    _check(lib().sparse_attn_to_tiles(ctypes.byref(shape), _ptr(src), _ptr(dst), _stream(stream)),
           "sparse_attn_to_tiles")
    return dst


def sparse_attn_from_tiles(shape: Shape, src, dst=None, stream=None):
    """Tile-major [B, H, N, d] -> raster order (a new tensor unless dst is given)."""
    import torch
    dst = torch.empty_like(src) if dst is None else dst
    _check(lib().sparse_attn_from_tiles(ctypes.byref(shape), _ptr(src), _ptr(dst), _stream(stream)),
           "sparse_attn_from_tiles")
    return dst
