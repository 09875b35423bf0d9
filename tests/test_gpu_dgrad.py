"""Backward-data GEMM from the forward weight's 2D quantization (nvfp4_transpose).

transpose(Q2D(W)) must equal the column-wise 2D quantization of W, i.e. Q2D(W^T), bit for bit (the
oracle's own transpose invariance is pinned on the CPU).  dgrad: dX = Q_SR(dY) . Q2D(W) with the
contraction over W's rows (K = 14336), checked on seeded tiles against the oracle.
"""
import numpy as np
import pytest
import torch

import nvfp4_bit_block_quantize_amd as nv
import synth
from tests.gpu_util import assert_quant_equal, gemm_check, oracle_input, seeded_tiles

pytestmark = pytest.mark.gpu
B2 = nv.NVFP4_BLOCK2D


def _host(q):
    return {"data": q.data.cpu().numpy(), "scales": q.scales.cpu().numpy(),
            "ts": q.tensor_scale.cpu().numpy()[0], "flags": q.flags}


# (2000, 464) and (2048, 1024) run the paired tile order (an even number of 128-code tile columns,
# a multiple of 16 tiles), the first with 8-byte pieces and ragged tiles on both axes
@pytest.mark.parametrize("shape", [(16, 16), (48, 80), (64, 64), (1040, 272), (272, 1040), (160, 96), (4128, 288),
                                   (2000, 464), (2048, 1024)])
def test_transpose_equals_colwise_2d_quantization(oracle, shape):
    w = synth.normal(shape, 0.02, seed=3, tensor_id=70, dtype=torch.bfloat16)
    q = nv.nvfp4_quantize(w.cuda(), flags=B2)
    qt = nv.nvfp4_transpose(q)
    torch.cuda.synchronize()
    assert (qt.rows, qt.k) == (shape[1], shape[0])
    ref = oracle.quantize(oracle_input(w), flags=B2 | nv.NVFP4_COLWISE)
    assert_quant_equal(qt, ref, f"transpose {shape}")
    qc = nv.nvfp4_quantize(w.cuda(), flags=B2 | nv.NVFP4_COLWISE)
    assert torch.equal(qt.data, qc.data) and torch.equal(qt.scales, qc.scales)


def test_transpose_empty_copies_tensor_scale():
    src = nv.empty_like_quantized(0, 32, B2, torch.device("cuda"))
    src.tensor_scale.fill_(0.125)
    out = nv.nvfp4_transpose(src)
    torch.cuda.synchronize()
    assert out.tensor_scale.item() == 0.125


def test_transpose_twice_is_identity():
    w = synth.normal((14336, 4096), 0.02, seed=0, tensor_id=4, dtype=torch.bfloat16).cuda()
    q = nv.nvfp4_quantize(w, flags=B2)
    back = nv.nvfp4_transpose(nv.nvfp4_transpose(q))
    torch.cuda.synchronize()
    assert torch.equal(back.data, q.data) and torch.equal(back.scales, q.scales)
    assert torch.equal(back.tensor_scale, q.tensor_scale)


def test_dgrad8b_sampled_tiles(oracle):
    dy, _ = synth.wgrad8b(0)       # dY [8192 x 14336] ~N(0, 1e-3)
    _, w = synth.fprop8b(0)        # W [14336 x 4096] ~N(0, 0.02)
    qdy = nv.nvfp4_quantize(dy.cuda(), flags=nv.NVFP4_SR, seed=7)   # rows of dY, K = 14336
    qw = nv.nvfp4_quantize(w.cuda(), flags=B2)                      # the forward operand
    qwt = nv.nvfp4_transpose(qw)                                    # [4096 x 14336]
    dx = nv.nvfp4_gemm(qdy, qwt, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    M, N, K = qdy.rows, qwt.rows, qdy.k
    assert (M, N, K) == (8192, 4096, 14336)
    tiles = seeded_tiles(M, N, 64, seed=6) + [(0, 0, 1, N), (M - 1, 0, 1, N)]
    cref, bnd = oracle.gemm_ref(_host(qdy), _host(qwt), M, N, K, tiles=tiles)
    rel = gemm_check(dx.float().cpu().numpy(), cref, bnd, True, "dgrad 8192x4096x14336")
    print(f"dgrad max |err|/bound {rel:.2e}")
