"""Python binding of libnvfp4.so (NVFP4 quantize / RHT-quantize / dequantize / GEMM on MI355X).

Argument marshalling only: PyTorch provides device memory and the current HIP stream, every step
of the computation runs in the library's HIP kernels.  The functions carry the C ABI's names
(include/nvfp4.h).  If the shared library has not been built the import of any function raises;
there is no fallback path.

    import torch, nvfp4_bit_block_quantize_amd as nv
    qx = nv.nvfp4_quantize(x)                                   # 1D blocks, nearest-even
    qw = nv.nvfp4_quantize(w, flags=nv.NVFP4_BLOCK2D)           # 16x16 weight tiles
    y  = nv.nvfp4_gemm(qx, qw, out_dtype=torch.bfloat16)        # y = x_hat @ w_hat^T
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

__all__ = [
    "NVFP4_OK", "NVFP4_ERR_NULL", "NVFP4_ERR_SHAPE", "NVFP4_ERR_ALIGN", "NVFP4_ERR_UNSUPPORTED",
    "NVFP4_ERR_HIP", "NVFP4_F32", "NVFP4_BF16", "NVFP4_COLWISE", "NVFP4_BLOCK2D", "NVFP4_SR",
    "NVFP4_FOUR_OVER_SIX", "NVFP4_TS_FOR_FOUR", "NVFP4_SCALE_SEARCH", "NVFP4Error", "NVFP4Tensor", "library_path", "lib",
    "nvfp4_workspace_size", "nvfp4_quantize", "nvfp4_quantize_noalloc", "nvfp4_rht_quantize", "nvfp4_dequantize",
    "nvfp4_gemm", "nvfp4_gemm_nvfp4_out", "nvfp4_scale_from_amax", "nvfp4_gemm_w4a16", "nvfp4_transpose", "nvfp4_status_string", "empty_like_quantized",
]

NVFP4_OK, NVFP4_ERR_NULL, NVFP4_ERR_SHAPE, NVFP4_ERR_ALIGN, NVFP4_ERR_UNSUPPORTED, NVFP4_ERR_HIP = range(6)
NVFP4_F32, NVFP4_BF16 = 0, 1
NVFP4_COLWISE, NVFP4_BLOCK2D, NVFP4_SR, NVFP4_FOUR_OVER_SIX = 1, 2, 4, 8
NVFP4_TS_FOR_FOUR, NVFP4_SCALE_SEARCH = 16, 32

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    return os.path.join(_HERE, "libnvfp4.so")


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("k", ctypes.c_int64), ("flags", ctypes.c_uint32)]


def lib():
    """The loaded libnvfp4.so.  Raises if it has not been built (python -m
    nvfp4_bit_block_quantize_amd.build)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"libnvfp4.so not built at {path}; run python -m nvfp4_bit_block_quantize_amd.build")
        L = ctypes.CDLL(path)
        P, i64, u32, u64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32
        TP = ctypes.POINTER(_Tensor)
        L.nvfp4_workspace_size.argtypes = [i64, i64, u32]
        L.nvfp4_workspace_size.restype = ctypes.c_size_t
        L.nvfp4_quantize.argtypes = [P, ctypes.c_int, i64, i64, i64, u32, u64, u32, TP, P, P]
        L.nvfp4_quantize.restype = ctypes.c_int
        L.nvfp4_quantize_noalloc.argtypes = [P, ctypes.c_int, i64, i64, i64, u32, u64, u32, TP, P]
        L.nvfp4_quantize_noalloc.restype = ctypes.c_int
        L.nvfp4_rht_quantize.argtypes = [P, ctypes.c_int, i64, i64, i64, u32, u64, u32, u64, P, TP, P, P]
        L.nvfp4_rht_quantize.restype = ctypes.c_int
        L.nvfp4_quantize_grouped.argtypes = [P, ctypes.c_int, i64, i64, i64, i64, i64, u32, u64, u32, TP, P, P]
        L.nvfp4_quantize_grouped.restype = ctypes.c_int
        L.nvfp4_dequantize.argtypes = [TP, P, ctypes.c_int, i64, P]
        L.nvfp4_dequantize.restype = ctypes.c_int
        L.nvfp4_gemm.argtypes = [TP, TP, P, ctypes.c_int, i64, i32, ctypes.POINTER(ctypes.c_int64), P]
        L.nvfp4_gemm.restype = ctypes.c_int
        L.nvfp4_gemm_nvfp4_out.argtypes = [TP, TP, TP, P, i32, ctypes.POINTER(ctypes.c_int64), P]
        L.nvfp4_gemm_nvfp4_out.restype = ctypes.c_int
        L.nvfp4_scale_from_amax.argtypes = [P, P, P]
        L.nvfp4_scale_from_amax.restype = ctypes.c_int
        L.nvfp4_gemm_w4a16.argtypes = [P, ctypes.c_int, i64, i64, TP, P, ctypes.c_int, i64, P]
        L.nvfp4_gemm_w4a16.restype = ctypes.c_int
        L.nvfp4_transpose.argtypes = [TP, TP, P]
        L.nvfp4_transpose.restype = ctypes.c_int
        L.nvfp4_status_string.argtypes = [ctypes.c_int]
        L.nvfp4_status_string.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {nvfp4_status_string(status)}")
        self.status = status


def nvfp4_status_string(status: int) -> str:
    return lib().nvfp4_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != NVFP4_OK:
        raise NVFP4Error(status, where)


@dataclass
class NVFP4Tensor:
    """An NVFP4 tensor (logical [rows x k], k contiguous).  For a grouped GEMM weight the three
    buffers hold `groups` consecutive tensors of `rows` rows each."""
    data: torch.Tensor          # uint8 [groups*rows, k/2]
    scales: torch.Tensor        # uint8 [groups*rows, k/16] or [groups*rows/16, k/16]
    tensor_scale: torch.Tensor  # float32 [groups]
    rows: int
    k: int
    flags: int = 0
    groups: int = 1

    def descriptor(self) -> _Tensor:
        return _Tensor(self.data.data_ptr() if self.data.numel() else None,
                       self.scales.data_ptr() if self.scales.numel() else None,
                       self.tensor_scale.data_ptr(), self.rows, self.k, self.flags & NVFP4_BLOCK2D)

    @property
    def block2d(self) -> bool:
        return bool(self.flags & NVFP4_BLOCK2D)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return NVFP4_F32
    if t == torch.bfloat16:
        return NVFP4_BF16
    raise TypeError(f"unsupported dtype {t}; NVFP4 inputs are float32 or bfloat16")


def _stream_handle(device: torch.device):
    if device.type != "cuda":
        return None
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def nvfp4_workspace_size(rows: int, cols: int, flags: int = 0) -> int:
    return int(lib().nvfp4_workspace_size(rows, cols, flags))


def empty_like_quantized(rows: int, k: int, flags: int, device, groups: int = 1) -> NVFP4Tensor:
    """Allocate the output buffers of an NVFP4 tensor of logical shape [rows x k]."""
    data = torch.empty((groups * rows, k // 2), dtype=torch.uint8, device=device)
    if flags & NVFP4_BLOCK2D:
        scales = torch.empty((groups * rows // 16, k // 16), dtype=torch.uint8, device=device)
    else:
        scales = torch.empty((groups * rows, k // 16), dtype=torch.uint8, device=device)
    ts = torch.empty((groups,), dtype=torch.float32, device=device)
    return NVFP4Tensor(data, scales, ts, rows, k, flags & NVFP4_BLOCK2D, groups)


def _logical(x: torch.Tensor, flags: int):
    if x.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    rows, cols = x.shape
    return (cols, rows) if flags & NVFP4_COLWISE else (rows, cols)


def _ld(x: torch.Tensor) -> int:
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("x must be row-major with unit column stride")
    return max(int(x.stride(0)), int(x.shape[1]), 1)


def nvfp4_quantize(x: torch.Tensor, flags: int = 0, seed: int = 0, stream_id: int = 0,
                   out: Optional[NVFP4Tensor] = None, workspace: Optional[torch.Tensor] = None) -> NVFP4Tensor:
    """Quantize x (float32 / bfloat16 [rows x cols]) to NVFP4 (see include/nvfp4.h)."""
    R, K = _logical(x, flags)
    if out is None:
        out = empty_like_quantized(R, K, flags, x.device)
    if workspace is None:
        workspace = torch.empty(nvfp4_workspace_size(*x.shape, flags) // 4, dtype=torch.int32, device=x.device)
    desc = out.descriptor()
    st = lib().nvfp4_quantize(_ptr(x), _dtype_code(x.dtype), x.shape[0], x.shape[1], _ld(x), flags, seed & (2**64 - 1),
                              stream_id, ctypes.byref(desc), _ptr(workspace), _stream_handle(x.device))
    _check(st, "nvfp4_quantize")
    return out


def nvfp4_quantize_noalloc(x: torch.Tensor, out: NVFP4Tensor, flags: int = 0, seed: int = 0,
                           stream_id: int = 0) -> NVFP4Tensor:
    """nvfp4_quantize into caller-allocated `out`, with the amax workspace in the library's own
    device array: the call allocates nothing (see include/nvfp4.h)."""
    desc = out.descriptor()
    st = lib().nvfp4_quantize_noalloc(_ptr(x), _dtype_code(x.dtype), x.shape[0], x.shape[1], _ld(x), flags,
                                      seed & (2**64 - 1), stream_id, ctypes.byref(desc), _stream_handle(x.device))
    _check(st, "nvfp4_quantize_noalloc")
    return out


def nvfp4_quantize_grouped(x: torch.Tensor, flags: int = 0, seed: int = 0, stream_id: int = 0,
                           out: Optional[NVFP4Tensor] = None, workspace: Optional[torch.Tensor] = None) -> NVFP4Tensor:
    """Quantize each x[g] of x (float32 / bfloat16 [groups x rows x cols], each x[g] with unit column
    stride) with its own tensor scale, group g with stream id stream_id + g, into one group-contiguous
    NVFP4 tensor (the grouped GEMM's weight layout; see include/nvfp4.h)."""
    if x.dim() != 3:
        raise ValueError("x must be [groups, rows, cols]")
    G, rows, cols = x.shape
    if G < 1:
        raise ValueError("x needs at least one group")
    R, K = _logical(x[0], flags)
    if out is None:
        out = empty_like_quantized(R, K, flags, x.device, groups=G)
    if workspace is None:
        workspace = torch.empty(G * nvfp4_workspace_size(rows, cols, flags) // 4, dtype=torch.int32, device=x.device)
    desc = out.descriptor()
    ldx = _ld(x[0])
    st = lib().nvfp4_quantize_grouped(_ptr(x), _dtype_code(x.dtype), G, rows, cols, ldx, x.stride(0) if G > 1 else 0,
                                      flags, seed & (2**64 - 1), stream_id, ctypes.byref(desc), _ptr(workspace),
                                      _stream_handle(x.device))
    _check(st, "nvfp4_quantize_grouped")
    return out


def nvfp4_rht_quantize(x: torch.Tensor, sign_seed: int, flags: int = 0, seed: int = 0, stream_id: int = 0,
                       rht_out: Optional[torch.Tensor] = None, out: Optional[NVFP4Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> NVFP4Tensor:
    """16x16 random Hadamard transform along K, then quantize (see include/nvfp4.h).  If rht_out
    (float32 [R x K]) is given, the transformed matrix is written to it as well."""
    R, K = _logical(x, flags)
    if out is None:
        out = empty_like_quantized(R, K, flags, x.device)
    if workspace is None:
        workspace = torch.empty(nvfp4_workspace_size(*x.shape, flags) // 4, dtype=torch.int32, device=x.device)
    desc = out.descriptor()
    st = lib().nvfp4_rht_quantize(_ptr(x), _dtype_code(x.dtype), x.shape[0], x.shape[1], _ld(x), flags,
                                  seed & (2**64 - 1), stream_id, sign_seed & (2**64 - 1), _ptr(rht_out),
                                  ctypes.byref(desc), _ptr(workspace), _stream_handle(x.device))
    _check(st, "nvfp4_rht_quantize")
    return out


def nvfp4_dequantize(t: NVFP4Tensor, dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.empty((t.rows, t.k), dtype=dtype, device=t.data.device)
    desc = t.descriptor()
    st = lib().nvfp4_dequantize(ctypes.byref(desc), _ptr(out), _dtype_code(out.dtype), _ld(out),
                                _stream_handle(out.device))
    _check(st, "nvfp4_dequantize")
    return out


def nvfp4_gemm(a: NVFP4Tensor, b: NVFP4Tensor, out_dtype: torch.dtype = torch.bfloat16,
               group_offsets: Optional[Sequence[int]] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A_hat @ B_hat^T with FP32 accumulation.  Grouped: group_offsets (host ints, G+1) split
    A's rows; b holds G weights of b.rows rows each."""
    M, N = a.rows, b.rows
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.data.device)
    da, db = a.descriptor(), b.descriptor()
    if group_offsets is not None:
        offs = (ctypes.c_int64 * len(group_offsets))(*[int(v) for v in group_offsets])
        G = len(group_offsets) - 1
    else:
        offs, G = None, 1
    st = lib().nvfp4_gemm(ctypes.byref(da), ctypes.byref(db), _ptr(out), _dtype_code(out.dtype), _ld(out), G, offs,
                          _stream_handle(out.device))
    _check(st, "nvfp4_gemm")
    return out


def nvfp4_gemm_nvfp4_out(a: NVFP4Tensor, b: NVFP4Tensor, out: NVFP4Tensor, amax: Optional[torch.Tensor] = None,
                         group_offsets: Optional[Sequence[int]] = None) -> NVFP4Tensor:
    """out = Q(A_hat @ B_hat^T), quantized row-wise (1D, nearest-even) in the GEMM's epilogue with the
    tensor scale already in out.tensor_scale; if amax (float32 [1], device) is given, max |C| is
    folded into it (see include/nvfp4.h)."""
    da, db, dout = a.descriptor(), b.descriptor(), out.descriptor()
    if group_offsets is not None:
        offs = (ctypes.c_int64 * len(group_offsets))(*[int(v) for v in group_offsets])
        G = len(group_offsets) - 1
    else:
        offs, G = None, 1
    st = lib().nvfp4_gemm_nvfp4_out(ctypes.byref(da), ctypes.byref(db), ctypes.byref(dout), _ptr(amax), G, offs,
                                    _stream_handle(out.data.device))
    _check(st, "nvfp4_gemm_nvfp4_out")
    return out


def nvfp4_scale_from_amax(amax: torch.Tensor, ts: torch.Tensor) -> torch.Tensor:
    """ts = amax / 2688 on the device (both float32 [1])."""
    st = lib().nvfp4_scale_from_amax(_ptr(amax), _ptr(ts), _stream_handle(ts.device))
    _check(st, "nvfp4_scale_from_amax")
    return ts


def nvfp4_gemm_w4a16(a: torch.Tensor, b: NVFP4Tensor, out_dtype: torch.dtype = torch.bfloat16,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A @ B_hat^T with A a bf16 [M x K] device matrix (unit stride along K) and B an NVFP4
    weight [N x K]; FP32 accumulation (see include/nvfp4.h)."""
    if a.dim() != 2 or a.stride(1) != 1:
        raise ValueError("nvfp4_gemm_w4a16: A must be 2-D with unit stride along K")
    if a.dtype != torch.bfloat16:
        raise TypeError("nvfp4_gemm_w4a16: A must be bfloat16")
    M, N = a.shape[0], b.rows
    if a.shape[1] != b.k:
        raise ValueError(f"nvfp4_gemm_w4a16: A has K={a.shape[1]}, B has K={b.k}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    db = b.descriptor()
    st = lib().nvfp4_gemm_w4a16(_ptr(a), NVFP4_BF16, M, _ld(a), ctypes.byref(db), _ptr(out),
                                _dtype_code(out.dtype), _ld(out), _stream_handle(out.device))
    _check(st, "nvfp4_gemm_w4a16")
    return out


def nvfp4_transpose(t: NVFP4Tensor, out: Optional[NVFP4Tensor] = None) -> NVFP4Tensor:
    """Transpose of a 16x16-block-scaled NVFP4 tensor (see include/nvfp4.h): codes, scale grid and
    tensor scale of t^T, equal to quantizing the transposed matrix directly."""
    if out is None:
        out = empty_like_quantized(t.k, t.rows, NVFP4_BLOCK2D, t.data.device)
    din, dout = t.descriptor(), out.descriptor()
    st = lib().nvfp4_transpose(ctypes.byref(din), ctypes.byref(dout), _stream_handle(t.data.device))
    _check(st, "nvfp4_transpose")
    return out
