"""nvfp4_quantize_noalloc (the entry point that allocates nothing: its amax workspace is the
library's own device array) against nvfp4_quantize with a caller workspace, through the C ABI:
identical codes, scale bytes and tensor scale on two calls in a row, the second on a smaller
input (the array keeps the first call's partial maxima, which the second must not read), in
several modes; plus its host-side argument checks."""
import ctypes

import pytest
import torch

import nvfp4_bit_block_quantize_amd as nv
import synth

FAKE = 0x10000


def _same(a, b, what):
    assert torch.equal(a.data, b.data), f"{what}: codes differ"
    assert torch.equal(a.scales, b.scales), f"{what}: scale bytes differ"
    assert torch.equal(a.tensor_scale, b.tensor_scale), f"{what}: tensor scale differs"


def test_noalloc_validation():
    L = nv.lib()
    d = nv._Tensor(FAKE, FAKE, FAKE, 32, 64, 0)
    q = lambda x=FAKE, out=d, rows=32, cols=64, ldx=64, flags=0: L.nvfp4_quantize_noalloc(
        x, nv.NVFP4_BF16, rows, cols, ldx, flags, 0, 0, ctypes.byref(out) if out is not None else None, None)
    assert q(out=None) == nv.NVFP4_ERR_NULL
    assert q(x=None) == nv.NVFP4_ERR_NULL
    assert q(cols=40, ldx=40) == nv.NVFP4_ERR_SHAPE
    assert q(x=FAKE + 8) == nv.NVFP4_ERR_ALIGN
    assert q(flags=nv.NVFP4_SR | nv.NVFP4_BLOCK2D) == nv.NVFP4_ERR_UNSUPPORTED


CASES = [
    ("row", 0, (1024, 4096), (96, 160)),
    ("row2d", nv.NVFP4_BLOCK2D, (2048, 1024), (48, 64)),
    ("col_sr", nv.NVFP4_COLWISE | nv.NVFP4_SR, (2048, 512), (64, 40)),
    ("row_4over6", nv.NVFP4_FOUR_OVER_SIX, (512, 2048), (16, 32)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,flags,big,small", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_quantize_twice(name, flags, big, small):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for i, shape in enumerate((big, small)):
        # the smaller input has a much smaller maximum: a stale partial maximum left in the array by
        # the first call would show in its tensor scale
        x = synth.normal(shape, 1.0 if i == 0 else 1e-3, seed=40 + i, tensor_id=500, dtype=torch.bfloat16).cuda()
        print(f"[noalloc] {name} call {i} shape={shape} flags={flags}", flush=True)
        ref = nv.nvfp4_quantize(x, flags=flags, seed=11, stream_id=2)
        R, K = (shape[1], shape[0]) if flags & nv.NVFP4_COLWISE else shape
        out = nv.empty_like_quantized(R, K, flags, x.device)
        nv.nvfp4_quantize_noalloc(x, out, flags=flags, seed=11, stream_id=2)
        torch.cuda.synchronize()
        _same(out, ref, f"{name} call {i}")
