"""ctypes wrapper over the plain CPU oracle (libnvfp4_oracle.so).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  It shares no code with the HIP library: it loads
its own C++ build (``oracle/nvfp4_oracle.cpp``) and never imports ``nvfp4_bit_block_quantize_amd``.

Arrays are numpy.  bf16 inputs are passed as their raw ``uint16`` bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

COLWISE = 1
BLOCK2D = 2
SR = 4
FOUR_OVER_SIX = 8
TS_FOR_FOUR = 16
SCALE_SEARCH = 32

DT_F32 = 0
DT_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib():
    """Load (building first if needed) the oracle shared library."""
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "libnvfp4_oracle.so")
        src = os.path.join(_HERE, "nvfp4_oracle.cpp")
        hdr = os.path.join(_HERE, "nvfp4_oracle.h")
        if (not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src)
                or os.path.getmtime(path) < os.path.getmtime(hdr)):
            _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        u32 = ctypes.c_uint32
        u64 = ctypes.c_uint64
        L.or_e2m1_value.argtypes = [ctypes.c_int]
        L.or_e2m1_value.restype = ctypes.c_float
        L.or_e2m1_rne_index.argtypes = [ctypes.c_float]
        L.or_e2m1_rne_index.restype = ctypes.c_int
        L.or_e4m3_value.argtypes = [ctypes.c_int]
        L.or_e4m3_value.restype = ctypes.c_float
        L.or_e4m3_rne.argtypes = [ctypes.c_float]
        L.or_e4m3_rne.restype = ctypes.c_int
        L.or_philox4x32_10.argtypes = [P, P, P]
        L.or_philox4x32_10.restype = None
        L.or_rht_sign_word.argtypes = [u64]
        L.or_rht_sign_word.restype = u32
        L.or_rht16.argtypes = [P, u32]
        L.or_rht16.restype = None
        L.or_e2m1_rne_array.argtypes = [P, i64, P]
        L.or_e2m1_rne_array.restype = None
        L.or_e4m3_rne_array.argtypes = [P, i64, P]
        L.or_e4m3_rne_array.restype = None
        L.or_philox_array.argtypes = [P, P, i64, P]
        L.or_philox_array.restype = None
        L.or_rht16_array.argtypes = [P, i64, u32]
        L.or_rht16_array.restype = None
        L.or_quantize.argtypes = [P, ctypes.c_int, i64, i64, i64, u32, u64, u32, ctypes.c_int, u64,
                                  P, P, P, P, P, ctypes.c_int]
        L.or_quantize.restype = ctypes.c_int
        L.or_dequantize.argtypes = [P, P, ctypes.c_float, i64, i64, u32, P]
        L.or_quantize_given_ts.argtypes = [P, i64, i64, i64, ctypes.c_float, P, P, ctypes.c_int]
        L.or_quantize_given_ts.restype = ctypes.c_int
        L.or_dequantize.restype = ctypes.c_int
        L.or_gemm_ref.argtypes = [P, P, ctypes.c_float, u32, P, P, ctypes.c_float, u32,
                                  i64, i64, i64, P, i64, P, P, ctypes.c_int]
        L.or_gemm_ref.restype = ctypes.c_int
        L.or_gemm_w4a16_ref.argtypes = [P, i64, P, P, ctypes.c_float, u32, i64, i64, i64, P, i64, P, P, ctypes.c_int]
        L.or_gemm_w4a16_ref.restype = ctypes.c_int
        L.or_tile_sse_2d.argtypes = [P, i64, ctypes.c_float, ctypes.c_float, P]
        L.or_tile_sse_2d.restype = ctypes.c_float
        _LIB = L
    return _LIB


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def default_threads():
    return max(1, min(16, os.cpu_count() or 1))


# ---- format primitives ------------------------------------------------------------------------

def e2m1_value(code):
    return lib().or_e2m1_value(int(code))


def e2m1_rne_index(v):
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32).ravel())
    out = np.empty(v.size, dtype=np.uint8)
    lib().or_e2m1_rne_array(_p(v), v.size, _p(out))
    return out


def e4m3_value(byte):
    return lib().or_e4m3_value(int(byte))


def e4m3_rne(s):
    s = np.ascontiguousarray(np.asarray(s, dtype=np.float32).ravel())
    out = np.empty(s.size, dtype=np.uint8)
    lib().or_e4m3_rne_array(_p(s), s.size, _p(out))
    return out


def philox(ctr, key):
    """ctr: (n,4) uint32, key: (n,2) uint32 -> (n,4) uint32 Philox4x32-10 outputs."""
    ctr = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32).reshape(-1, 4))
    key = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(-1, 2))
    assert ctr.shape[0] == key.shape[0]
    out = np.empty_like(ctr)
    lib().or_philox_array(_p(ctr), _p(key), ctr.shape[0], _p(out))
    return out


def rht_sign_word(sign_seed):
    return int(lib().or_rht_sign_word(int(sign_seed)))


def rht16(u, sign_word):
    """Apply the oracle's 16-point RHT to every contiguous 16-chunk of u (float32); returns a copy."""
    u = np.array(u, dtype=np.float32, copy=True, order="C")
    assert u.size % 16 == 0
    lib().or_rht16_array(_p(u), u.size // 16, int(sign_word))
    return u


# ---- quantize / dequantize / GEMM -------------------------------------------------------------

def logical_shape(rows, cols, flags):
    return (cols, rows) if flags & COLWISE else (rows, cols)


def quantize(x, flags=0, seed=0, stream_id=0, rht=False, sign_seed=0, want_rht_out=False,
             nthreads=None):
    """x: 2-D numpy float32, or uint16 holding bf16 bits.  Returns a dict with
    data [R][K/2] u8, scales u8, ts (np.float32), rht_out (or None), sse (chosen, plain)."""
    if x.dtype == np.uint16:
        dtype = DT_BF16
    elif x.dtype == np.float32:
        dtype = DT_F32
    else:
        raise TypeError("oracle.quantize takes float32 or bf16 bits as uint16")
    assert x.ndim == 2 and x.strides[1] == x.itemsize
    rows, cols = x.shape
    ldx = x.strides[0] // x.itemsize
    R, K = logical_shape(rows, cols, flags)
    if K % 16 or ((flags & BLOCK2D) and R % 16):
        raise ValueError("shape not a multiple of the block size")
    data = np.zeros((R, K // 2), dtype=np.uint8)
    if flags & BLOCK2D:
        scales = np.zeros((R // 16, K // 16), dtype=np.uint8)
    else:
        scales = np.zeros((R, K // 16), dtype=np.uint8)
    ts = np.zeros(1, dtype=np.float32)
    rht_out = np.zeros((R, K), dtype=np.float32) if (rht and want_rht_out) else None
    sse = np.zeros(2, dtype=np.float64)
    rc = lib().or_quantize(_p(x), dtype, rows, cols, ldx, flags, seed, stream_id, int(bool(rht)),
                           sign_seed, _p(data), _p(scales), _p(ts), _p(rht_out), _p(sse),
                           nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle quantize rejected the arguments (code {rc})")
    return {"data": data, "scales": scales, "ts": ts[0], "rht_out": rht_out,
            "sse": (float(sse[0]), float(sse[1])), "flags": flags, "R": R, "K": K}


def quantize_given_ts(y, ts, nthreads=None):
    """Row-wise 1D nearest-even quantization of float32 y [rows x cols] with the given tensor scale.
    Returns (data [rows][cols/2] u8, scales [rows][cols/16] u8)."""
    y = np.asarray(y)
    assert y.dtype == np.float32 and y.ndim == 2 and y.strides[1] == 4
    rows, cols = y.shape
    data = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    rc = lib().or_quantize_given_ts(_p(y), rows, cols, y.strides[0] // 4, float(np.float32(ts)), _p(data), _p(scales),
                                    nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle quantize_given_ts rejected the arguments")
    return data, scales


def tile_sse_2d(tile, ts, T):
    """Four-over-Six error of one 16x16 float32 tile for grid target T under tensor scale ts.
    Returns (sse as np.float32, scale byte)."""
    tile = np.asarray(tile)
    assert tile.dtype == np.float32 and tile.shape == (16, 16) and tile.strides[1] == 4
    sb = np.zeros(1, dtype=np.uint8)
    v = lib().or_tile_sse_2d(_p(tile), tile.strides[0] // 4, float(np.float32(ts)), float(T), _p(sb))
    return np.float32(v), int(sb[0])


def dequantize(data, scales, ts, R, K, flags=0):
    data = np.ascontiguousarray(data, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    y = np.empty((R, K), dtype=np.float32)
    rc = lib().or_dequantize(_p(data), _p(scales), float(ts), R, K, flags, _p(y))
    if rc != 0:
        raise ValueError("oracle dequantize rejected the arguments")
    return y


def gemm_ref(a, b, M, N, K, tiles=None, nthreads=None):
    """a, b: dicts with data/scales/ts/flags (A is M x K, B is N x K).  tiles: list of
    (row0, col0, h, w); None = the full matrix.  Returns (C, bound) as float64 [M x N] arrays
    (NaN outside the requested tiles)."""
    if tiles is None:
        tiles = [(0, 0, M, N)]
    t = np.ascontiguousarray(np.asarray(tiles, dtype=np.int64).reshape(-1, 4))
    c = np.full((M, N), np.nan, dtype=np.float64)
    bnd = np.full((M, N), np.nan, dtype=np.float64)
    ad = np.ascontiguousarray(a["data"], dtype=np.uint8)
    asc = np.ascontiguousarray(a["scales"], dtype=np.uint8)
    bd = np.ascontiguousarray(b["data"], dtype=np.uint8)
    bsc = np.ascontiguousarray(b["scales"], dtype=np.uint8)
    rc = lib().or_gemm_ref(_p(ad), _p(asc), float(a["ts"]), int(a.get("flags", 0)) & BLOCK2D,
                           _p(bd), _p(bsc), float(b["ts"]), int(b.get("flags", 0)) & BLOCK2D,
                           M, N, K, _p(t), t.shape[0], _p(c), _p(bnd), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle gemm rejected the arguments")
    return c, bnd


def gemm_w4a16_ref(a_bf16_bits, b, M, N, K, tiles=None, nthreads=None):
    """A: uint16 bf16 bits [M x lda]; b: dict with data/scales/ts/flags (B is N x K).  Returns
    (C, bound) as float64 [M x N] (NaN outside the requested tiles)."""
    if tiles is None:
        tiles = [(0, 0, M, N)]
    t = np.ascontiguousarray(np.asarray(tiles, dtype=np.int64).reshape(-1, 4))
    a = np.asarray(a_bf16_bits, dtype=np.uint16)
    assert a.ndim == 2 and a.strides[1] == 2
    c = np.full((M, N), np.nan, dtype=np.float64)
    bnd = np.full((M, N), np.nan, dtype=np.float64)
    bd = np.ascontiguousarray(b["data"], dtype=np.uint8)
    bsc = np.ascontiguousarray(b["scales"], dtype=np.uint8)
    rc = lib().or_gemm_w4a16_ref(_p(a), a.strides[0] // 2, _p(bd), _p(bsc), float(b["ts"]),
                                 int(b.get("flags", 0)) & BLOCK2D, M, N, K, _p(t), t.shape[0], _p(c), _p(bnd),
                                 nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle w4a16 gemm rejected the arguments")
    return c, bnd
