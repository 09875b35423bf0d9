"""The C ABI on a machine without a GPU: the library loads, exports every function that
include/nvfp4.h declares, and rejects bad arguments on the host with the documented status codes
before anything is enqueued (fake device addresses are never dereferenced on these paths)."""
import ctypes
import os
import re
import subprocess

import pytest

import nvfp4_bit_block_quantize_amd as nv

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "nvfp4.h")
FAKE = 0x10000  # 16-byte aligned fake device address
MIS = 0x10008   # misaligned


def declared():
    txt = open(HDR).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = declared()
    assert set(names) >= {"nvfp4_quantize", "nvfp4_rht_quantize", "nvfp4_dequantize", "nvfp4_gemm",
                          "nvfp4_workspace_size", "nvfp4_status_string"}
    L = nv.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", nv.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"^[0-9a-f]+ [A-Za-z] (\S+)$", out, flags=re.M))
    # nothing but the declared C ABI is exported (hipcc adds one __hip_cuid_<hash> marker per
    # translation unit)
    extra = {e for e in exported if not e.startswith("__hip_cuid_")}
    assert extra == set(names), (sorted(extra - set(names)), sorted(set(names) - extra))


def _desc(rows, k, flags=0, data=FAKE, scales=FAKE, ts=FAKE):
    return nv._Tensor(data, scales, ts, rows, k, flags)


def _q(x=FAKE, dtype=nv.NVFP4_BF16, rows=32, cols=64, ldx=64, flags=0, out=None, ws=FAKE, rht=False):
    L = nv.lib()
    if out is None:
        R, K = (cols, rows) if flags & nv.NVFP4_COLWISE else (rows, cols)
        out = _desc(R, K, flags)
    ref = ctypes.byref(out) if out is not False else None
    if rht:
        return L.nvfp4_rht_quantize(x, dtype, rows, cols, ldx, flags, 0, 0, 7, None, ref, ws, None)
    return L.nvfp4_quantize(x, dtype, rows, cols, ldx, flags, 0, 0, ref, ws, None)


@pytest.mark.parametrize("rht", [False, True])
def test_quantize_validation(rht):
    assert _q(out=False, rht=rht) == nv.NVFP4_ERR_NULL
    assert _q(x=None, rht=rht) == nv.NVFP4_ERR_NULL
    assert _q(ws=None, rht=rht) == nv.NVFP4_ERR_NULL
    assert _q(dtype=7, rht=rht) == nv.NVFP4_ERR_UNSUPPORTED
    assert _q(cols=40, ldx=40, rht=rht) == nv.NVFP4_ERR_SHAPE            # K % 16
    assert _q(ldx=32, rht=rht) == nv.NVFP4_ERR_SHAPE                     # ldx < cols
    assert _q(rows=-1, rht=rht) == nv.NVFP4_ERR_SHAPE
    assert _q(flags=nv.NVFP4_COLWISE, rows=40, rht=rht) == nv.NVFP4_ERR_SHAPE  # K = rows % 16
    assert _q(flags=nv.NVFP4_COLWISE, rows=32, cols=36, ldx=40, rht=rht) == nv.NVFP4_ERR_SHAPE  # cols % 8
    assert _q(x=MIS, rht=rht) == nv.NVFP4_ERR_ALIGN
    assert _q(ws=MIS, rht=rht) == nv.NVFP4_ERR_ALIGN
    assert _q(ldx=68, rht=rht) == nv.NVFP4_ERR_ALIGN                     # 136 B rows
    assert _q(out=_desc(32, 64, data=MIS), rht=rht) == nv.NVFP4_ERR_ALIGN
    assert _q(out=_desc(31, 64), rht=rht) == nv.NVFP4_ERR_SHAPE          # descriptor mismatch
    assert _q(out=_desc(32, 64, nv.NVFP4_BLOCK2D), rht=rht) == nv.NVFP4_ERR_SHAPE
    assert _q(flags=1 << 7, rht=rht) == nv.NVFP4_ERR_UNSUPPORTED
    assert _q(flags=nv.NVFP4_SR | nv.NVFP4_FOUR_OVER_SIX, rht=rht) == nv.NVFP4_ERR_UNSUPPORTED
    assert _q(flags=nv.NVFP4_SR | nv.NVFP4_BLOCK2D, rht=rht) == nv.NVFP4_ERR_UNSUPPORTED
    assert _q(flags=nv.NVFP4_SCALE_SEARCH | nv.NVFP4_BLOCK2D, rht=rht) == nv.NVFP4_ERR_UNSUPPORTED
    assert _q(flags=nv.NVFP4_SCALE_SEARCH | nv.NVFP4_FOUR_OVER_SIX, rht=rht) == nv.NVFP4_ERR_UNSUPPORTED
    assert _q(flags=nv.NVFP4_SCALE_SEARCH | nv.NVFP4_SR, rht=rht) == nv.NVFP4_ERR_UNSUPPORTED
    assert _q(flags=1 << 6, rht=rht) == nv.NVFP4_ERR_UNSUPPORTED


def test_quantize_grouped_validation():
    L = nv.lib()

    def qg(G=4, stride=32 * 64, flags=0, x=FAKE, dtype=nv.NVFP4_BF16, out=None, ws=FAKE):
        d = out if out is not None else _desc(32, 64, flags)
        return L.nvfp4_quantize_grouped(x, dtype, G, 32, 64, 64, stride, flags, 0, 0, ctypes.byref(d), ws, None)
    assert qg(G=0) == nv.NVFP4_ERR_SHAPE
    assert qg(G=65536) == nv.NVFP4_ERR_SHAPE
    assert qg(stride=-64) == nv.NVFP4_ERR_SHAPE
    assert qg(stride=1 << 40) == nv.NVFP4_ERR_SHAPE              # group offsets beyond the 36-bit range
    assert qg(stride=32 * 64 + 4) == nv.NVFP4_ERR_ALIGN          # 8-byte group step for bf16
    assert qg(x=None) == nv.NVFP4_ERR_NULL
    assert qg(ws=None) == nv.NVFP4_ERR_NULL
    assert qg(x=MIS) == nv.NVFP4_ERR_ALIGN
    assert qg(out=_desc(32, 48)) == nv.NVFP4_ERR_SHAPE            # descriptor is per group: [32 x 64]
    assert qg(flags=nv.NVFP4_SR | nv.NVFP4_FOUR_OVER_SIX) == nv.NVFP4_ERR_UNSUPPORTED
    assert qg(dtype=5) == nv.NVFP4_ERR_UNSUPPORTED


def test_rht_rejects_2d_and_block2d_rows():
    assert _q(flags=nv.NVFP4_BLOCK2D, rht=True) == nv.NVFP4_ERR_UNSUPPORTED
    assert _q(flags=nv.NVFP4_BLOCK2D, rows=40, ldx=64) == nv.NVFP4_ERR_SHAPE  # R % 16 for 2D


def test_dequantize_validation():
    L = nv.lib()
    assert L.nvfp4_dequantize(None, FAKE, 0, 64, None) == nv.NVFP4_ERR_NULL
    d = _desc(32, 64)
    assert L.nvfp4_dequantize(ctypes.byref(d), FAKE, 3, 64, None) == nv.NVFP4_ERR_UNSUPPORTED
    assert L.nvfp4_dequantize(ctypes.byref(d), FAKE, 0, 32, None) == nv.NVFP4_ERR_SHAPE
    assert L.nvfp4_dequantize(ctypes.byref(_desc(32, 40)), FAKE, 0, 64, None) == nv.NVFP4_ERR_SHAPE
    assert L.nvfp4_dequantize(ctypes.byref(_desc(40, 64, nv.NVFP4_BLOCK2D)), FAKE, 0, 64, None) == nv.NVFP4_ERR_SHAPE
    assert L.nvfp4_dequantize(ctypes.byref(d), None, 0, 64, None) == nv.NVFP4_ERR_NULL
    assert L.nvfp4_dequantize(ctypes.byref(d), MIS, 0, 64, None) == nv.NVFP4_ERR_ALIGN
    assert L.nvfp4_dequantize(ctypes.byref(d), FAKE, 1, 68, None) == nv.NVFP4_ERR_ALIGN
    assert L.nvfp4_dequantize(ctypes.byref(_desc(0, 64)), FAKE, 0, 64, None) == nv.NVFP4_OK  # empty: no-op


def test_gemm_validation():
    L = nv.lib()
    a, b = _desc(64, 128), _desc(32, 128)
    g = lambda a_, b_, c=FAKE, dt=1, ldc=32, G=1, offs=None: L.nvfp4_gemm(
        ctypes.byref(a_) if a_ else None, ctypes.byref(b_) if b_ else None, c, dt, ldc, G, offs, None)
    assert g(None, b) == nv.NVFP4_ERR_NULL
    assert g(a, b, dt=5) == nv.NVFP4_ERR_UNSUPPORTED
    assert g(a, _desc(32, 144)) == nv.NVFP4_ERR_SHAPE          # K mismatch
    assert g(_desc(64, 120), _desc(32, 120)) == nv.NVFP4_ERR_SHAPE  # K % 16
    assert g(a, b, ldc=16) == nv.NVFP4_ERR_SHAPE               # ldc < N
    assert g(a, _desc(40, 128, nv.NVFP4_BLOCK2D)) == nv.NVFP4_ERR_SHAPE
    assert g(a, b, c=None) == nv.NVFP4_ERR_NULL
    assert g(_desc(64, 128, data=MIS), b) == nv.NVFP4_ERR_ALIGN
    assert g(a, b, c=FAKE + 1) == nv.NVFP4_ERR_ALIGN
    assert g(a, b, G=2) == nv.NVFP4_ERR_SHAPE                  # groups without offsets
    offs = (ctypes.c_int64 * 3)(0, 70, 64)
    assert g(a, b, G=2, offs=offs) == nv.NVFP4_ERR_SHAPE       # decreasing
    offs = (ctypes.c_int64 * 3)(0, 10, 60)
    assert g(a, b, G=2, offs=offs) == nv.NVFP4_ERR_SHAPE       # does not end at M
    assert g(_desc(0, 128), b) == nv.NVFP4_OK                  # empty: no-op


def test_status_strings_and_workspace():
    for s in range(6):
        assert nv.nvfp4_status_string(s).startswith("NVFP4_")
    assert "unknown" in nv.nvfp4_status_string(99)
    assert nv.nvfp4_workspace_size(8192, 4096, 0) >= 4 * 1024


def test_transpose_validation():
    L = nv.lib()
    t = lambda i, o: L.nvfp4_transpose(ctypes.byref(i) if i else None, ctypes.byref(o) if o else None, None)
    B2 = nv.NVFP4_BLOCK2D
    assert t(None, _desc(64, 32, B2)) == nv.NVFP4_ERR_NULL
    assert t(_desc(32, 64), _desc(64, 32, B2)) == nv.NVFP4_ERR_UNSUPPORTED      # 1D scales do not transpose
    assert t(_desc(32, 64, B2), _desc(64, 32)) == nv.NVFP4_ERR_UNSUPPORTED
    assert t(_desc(32, 64, B2), _desc(32, 64, B2)) == nv.NVFP4_ERR_SHAPE        # out must be [k x rows]
    assert t(_desc(40, 64, B2), _desc(64, 40, B2)) == nv.NVFP4_ERR_SHAPE        # rows % 16
    assert t(_desc(32, 64, B2, data=MIS), _desc(64, 32, B2)) == nv.NVFP4_ERR_ALIGN


def test_gemm_w4a16_validation():
    L = nv.lib()
    b = _desc(32, 128)
    g = lambda a=FAKE, adt=nv.NVFP4_BF16, m=64, lda=128, b_=b, c=FAKE, dt=1, ldc=32: L.nvfp4_gemm_w4a16(
        a, adt, m, lda, ctypes.byref(b_) if b_ else None, c, dt, ldc, None)
    assert g(b_=None) == nv.NVFP4_ERR_NULL
    assert g(adt=nv.NVFP4_F32) == nv.NVFP4_ERR_UNSUPPORTED       # activations are bf16
    assert g(dt=5) == nv.NVFP4_ERR_UNSUPPORTED
    assert g(b_=_desc(32, 96), lda=96) == nv.NVFP4_ERR_SHAPE     # K % 64
    assert g(lda=64) == nv.NVFP4_ERR_SHAPE                       # lda < K
    assert g(ldc=16) == nv.NVFP4_ERR_SHAPE                       # ldc < N
    assert g(m=-1) == nv.NVFP4_ERR_SHAPE
    assert g(b_=_desc(40, 128, nv.NVFP4_BLOCK2D)) == nv.NVFP4_ERR_SHAPE
    assert g(m=1 << 24, lda=1 << 8) == nv.NVFP4_ERR_SHAPE        # A beyond 32-bit byte offsets
    assert g(a=None) == nv.NVFP4_ERR_NULL
    assert g(c=None) == nv.NVFP4_ERR_NULL
    assert g(a=MIS) == nv.NVFP4_ERR_ALIGN
    assert g(lda=132) == nv.NVFP4_ERR_ALIGN                      # rows of A not 16-byte aligned
    assert g(b_=_desc(32, 128, data=MIS)) == nv.NVFP4_ERR_ALIGN
    assert g(b_=_desc(32, 128, scales=FAKE + 2)) == nv.NVFP4_ERR_ALIGN
    assert g(c=FAKE + 1) == nv.NVFP4_ERR_ALIGN
    assert g(m=0) == nv.NVFP4_OK                                 # empty: no-op
    assert g(b_=_desc(0, 128)) == nv.NVFP4_OK


def test_gemm_nvfp4_out_validation():
    L = nv.lib()
    a, b = _desc(64, 256), _desc(32, 256)
    q = lambda a_=a, b_=b, o=None, amax=FAKE, G=1, offs=None: L.nvfp4_gemm_nvfp4_out(
        ctypes.byref(a_) if a_ else None, ctypes.byref(b_) if b_ else None,
        ctypes.byref(o if o is not None else _desc(64, 32)) if o is not False else None, amax, G, offs, None)
    assert q(o=False) == nv.NVFP4_ERR_NULL
    assert q(a_=None) == nv.NVFP4_ERR_NULL
    assert q(o=_desc(64, 48)) == nv.NVFP4_ERR_SHAPE                      # out must be [M x N]
    assert q(b_=_desc(24, 256), o=_desc(64, 24)) == nv.NVFP4_ERR_SHAPE   # N % 16: blocks of 16 along N
    assert q(o=_desc(64, 32, nv.NVFP4_BLOCK2D)) == nv.NVFP4_ERR_UNSUPPORTED  # row-wise 1D only
    assert q(o=_desc(64, 32, nv.NVFP4_SR)) == nv.NVFP4_ERR_UNSUPPORTED
    assert q(a_=_desc(64, 192), b_=_desc(32, 192)) == nv.NVFP4_ERR_UNSUPPORTED  # K % 256
    assert q(a_=_desc(64, 384), b_=_desc(32, 384), o=_desc(64, 32)) == nv.NVFP4_ERR_UNSUPPORTED
    assert q(a_=_desc(64, 256, scales=FAKE + 8)) == nv.NVFP4_ERR_UNSUPPORTED   # scales 16-byte aligned
    assert q(o=_desc(64, 32, data=0)) == nv.NVFP4_ERR_NULL
    assert q(o=_desc(64, 32, ts=0)) == nv.NVFP4_ERR_NULL
    assert q(o=_desc(64, 32, data=MIS)) == nv.NVFP4_ERR_ALIGN
    assert q(amax=FAKE + 2) == nv.NVFP4_ERR_ALIGN
    assert q(G=2) == nv.NVFP4_ERR_SHAPE                                   # groups without offsets
    assert q(a_=_desc(0, 256), o=_desc(0, 32)) == nv.NVFP4_OK            # empty: no-op
    assert L.nvfp4_scale_from_amax(None, FAKE, None) == nv.NVFP4_ERR_NULL
    assert L.nvfp4_scale_from_amax(FAKE, FAKE + 2, None) == nv.NVFP4_ERR_ALIGN
