"""GPU parity of nvfp4_gemm_w4a16 (bf16 activations x NVFP4 weights) against the oracle's binary64
reference.

Pass condition: |C - C_ref| <= 1e-5 * sum_k |a_ik| |q_jk S_jk| ts (plus 2^-8 |C_ref| for a bf16
output, whose rounding the bound leaves out).  The weights are the library's own quantized tensor
copied back, so the check isolates the multiply.  Also: K = 0 gives C = 0 in both GEMMs, one-hot
activations select decoded weight columns bit for bit, and strided A / C views are honoured."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import gemm_check, seeded_tiles

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_bit_block_quantize_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.lib()


def _host(q):
    return {"data": q.data.cpu().numpy(), "scales": q.scales.cpu().numpy(),
            "ts": q.tensor_scale.cpu().numpy()[0], "flags": q.flags}


def _case(oracle, a, w, b_flags=0, out_dtype=torch.float32, tiles=None, what=""):
    print(f"[w4a16] {what} A={tuple(a.shape)} W={tuple(w.shape)} flags={b_flags} out={out_dtype}", flush=True)
    a = a.cuda()
    qb = nv.nvfp4_quantize(w.cuda(), flags=b_flags)
    c = nv.nvfp4_gemm_w4a16(a, qb, out_dtype=out_dtype)
    torch.cuda.synchronize()
    M, N, K = a.shape[0], qb.rows, qb.k
    cref, bnd = oracle.gemm_w4a16_ref(synth.bf16_bits(a.cpu()), _host(qb), M, N, K, tiles=tiles)
    return gemm_check(c.float().cpu().numpy(), cref, bnd, out_dtype == torch.bfloat16, what)


@pytest.mark.parametrize("M,N,K", [(200, 136, 64), (1, 1, 64), (129, 257, 1088), (256, 256, 4096),
                                   (513, 80, 192)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_w4a16_ragged_shapes(oracle, M, N, K, out_dtype):
    a = synth.normal((M, K), 1.0, seed=5, tensor_id=80, dtype=torch.bfloat16)
    w = synth.normal((N, K), 0.02, seed=5, tensor_id=81, dtype=torch.bfloat16)
    rel = _case(oracle, a, w, out_dtype=out_dtype, what=f"{M}x{N}x{K}")
    print(f"max |err| / bound = {rel:.3e}")


# few activation rows (<= 256) and K % 128 == 0 take the weight-streaming kernel: M tiles 1..4, chunk
# counts that leave waves idle (K = 128) or uneven (K = 1152), ragged N, 1D and 2D scales; above 64
# rows, 64-row activation chunks (a ragged last chunk whose missing rows wrap), and 257 rows, the
# first count past the switch to the tiled kernel
@pytest.mark.parametrize("M,N,K", [(1, 200, 128), (5, 64, 1152), (16, 1000, 512), (17, 130, 2048),
                                   (33, 64, 256), (64, 336, 1024), (65, 96, 256), (100, 200, 512),
                                   (128, 64, 1152), (192, 130, 2048), (193, 64, 256), (256, 80, 512),
                                   (257, 64, 256)])
@pytest.mark.parametrize("b_flags", [0, 2])
def test_w4a16_few_rows(oracle, M, N, K, b_flags):
    if b_flags and N % 16:
        pytest.skip("2D scales need N % 16 == 0")
    a = synth.normal((M, K), 1.0, seed=10, tensor_id=88, dtype=torch.bfloat16)
    w = synth.normal((N, K), 0.02, seed=10, tensor_id=89, dtype=torch.bfloat16)
    for out_dtype in (torch.float32, torch.bfloat16):
        rel = _case(oracle, a, w, b_flags=b_flags, out_dtype=out_dtype, what=f"few rows {M}x{N}x{K}")
    print(f"max |err| / bound = {rel:.3e}")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_w4a16_2d_weight_scales(oracle, out_dtype):
    a = synth.normal((300, 640), 1.0, seed=6, tensor_id=82, dtype=torch.bfloat16)
    synth.outlier_columns(a, 0.01, 20.0, seed=6, tensor_id=82)
    w = synth.normal((272, 640), 0.02, seed=6, tensor_id=83, dtype=torch.bfloat16)
    _case(oracle, a, w, b_flags=nv.NVFP4_BLOCK2D, out_dtype=out_dtype, what="2D W")


def test_w4a16_one_hot_selects_decoded_weight(oracle):
    # C = ts * (q S) for a one-hot row with value 1: one rounding, equal to the fp32 decode
    K, N = 256, 96
    picks = [0, 15, 16, 63, 64, 130, 200, 255]
    a = torch.zeros((len(picks), K), dtype=torch.bfloat16)
    for i, k in enumerate(picks):
        a[i, k] = 1.0
    w = synth.normal((N, K), 1.0, seed=7, tensor_id=84, dtype=torch.float32)
    w[3, 70] = 1e-4  # a small element: a subnormal-range scale product still decodes exactly
    for flags in (0, nv.NVFP4_BLOCK2D):
        qb = nv.nvfp4_quantize(w.cuda(), flags=flags)
        c = nv.nvfp4_gemm_w4a16(a.cuda(), qb, out_dtype=torch.float32).cpu()
        yb = nv.nvfp4_dequantize(qb).cpu()
        for i, k in enumerate(picks):
            assert torch.equal(c[i], yb[:, k]), (flags, k)


def test_w4a16_strided_views(oracle):
    # A a column slice of a wider matrix (lda > K), C a column slice of a wider output (ldc > N)
    M, N, K = 260, 144, 320
    big = synth.normal((M, K + 64), 1.0, seed=8, tensor_id=85, dtype=torch.bfloat16).cuda()
    a = big[:, 32:32 + K]
    w = synth.normal((N, K), 0.05, seed=8, tensor_id=86, dtype=torch.bfloat16)
    qb = nv.nvfp4_quantize(w.cuda())
    cbig = torch.full((M, N + 24), 7.0, dtype=torch.float32, device="cuda")
    nv.nvfp4_gemm_w4a16(a, qb, out=cbig[:, 8:8 + N])
    torch.cuda.synchronize()
    got = cbig.cpu()
    assert torch.all(got[:, :8] == 7.0) and torch.all(got[:, 8 + N:] == 7.0)
    cref, bnd = oracle.gemm_w4a16_ref(synth.bf16_bits(a.cpu()), _host(qb), M, N, K)
    gemm_check(got[:, 8:8 + N].numpy(), cref, bnd, False, "strided")


def test_k_zero_gives_zero_in_both_gemms():
    M, N = 70, 48
    w = torch.empty((N, 0), dtype=torch.bfloat16, device="cuda")
    qb = nv.nvfp4_quantize(w)
    a = torch.empty((M, 0), dtype=torch.bfloat16, device="cuda")
    c = nv.nvfp4_gemm_w4a16(a, qb, out=torch.full((M, N), 3.0, device="cuda"))
    assert torch.all(c.cpu() == 0)
    qa = nv.nvfp4_quantize(a)
    c = nv.nvfp4_gemm(qa, qb, out=torch.full((M, N), 3.0, device="cuda"))
    assert torch.all(c.cpu() == 0)


def test_w4a16_fprop8b_sampled_tiles(oracle):
    # the Llama-3-8B FFN forward shape: X [8192 x 4096] bf16 against the 2D-quantized W [14336 x 4096]
    x, w = synth.fprop8b(0)
    M, N = x.shape[0], w.shape[0]
    tiles = seeded_tiles(M, N, 48, seed=2) + [(0, 0, 1, N), (M - 1, 0, 1, N)]
    rel = _case(oracle, x, w, b_flags=nv.NVFP4_BLOCK2D, out_dtype=torch.bfloat16, tiles=tiles,
                what="fprop 8192x14336x4096")
    print(f"max |err| / bound = {rel:.3e}")


def test_w4a16_decode_shape_full(oracle):
    # a decode-sized batch (16 tokens) against the full 2D-quantized W [14336 x 4096]
    _, w = synth.fprop8b(0)
    a = synth.normal((16, w.shape[1]), 1.0, seed=9, tensor_id=87, dtype=torch.bfloat16)
    rel = _case(oracle, a, w, b_flags=nv.NVFP4_BLOCK2D, out_dtype=torch.bfloat16, what="decode 16x14336x4096")
    print(f"max |err| / bound = {rel:.3e}")
