"""GPU parity of nvfp4_gemm_nvfp4_out: the GEMM whose epilogue quantizes C (row-wise 1D blocks,
nearest-even) with a caller-supplied tensor scale.

Parity chain: the fp32 C of nvfp4_gemm (same operands, same kernel and accumulation order) is
checked against the oracle's binary64 GEMM in test_gpu_gemm.py; here the fused codes and scale bytes
must equal, bit for bit, the oracle quantizing that fp32 C with the same tensor scale
(oracle.quantize_given_ts), and the running amax must equal max |C|.  Tensor scales: the ideal one
(amax / 2688 of this C), a too-small one (block scales clamp at 448, codes saturate at 6), a larger
one, and zero."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_bit_block_quantize_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.lib()


def _fused(qa, qb, ts, group_offsets=None, amax=None):
    out = nv.empty_like_quantized(qa.rows, qb.rows, 0, qa.data.device)
    out.tensor_scale.fill_(float(ts))
    nv.nvfp4_gemm_nvfp4_out(qa, qb, out, amax=amax, group_offsets=group_offsets)
    return out


def _check(oracle, c32, out, ts, what):
    c = c32.cpu().numpy()
    data, scales = oracle.quantize_given_ts(c, np.float32(ts))
    got_s = out.scales.cpu().numpy()
    got_d = out.data.cpu().numpy()
    np.testing.assert_array_equal(got_s, scales, err_msg=f"{what}: scale bytes")
    if not np.array_equal(got_d, data):
        bad = np.argwhere(got_d != data)
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first at {bad[:4].tolist()}")


def _operands(M, N, K, seed, b_flags=0):
    a = synth.normal((M, K), 1.0, seed=seed, tensor_id=90, dtype=torch.bfloat16)
    synth.outlier_columns(a, 0.01, 20.0, seed=seed, tensor_id=90)
    w = synth.normal((N, K), 0.02, seed=seed, tensor_id=91, dtype=torch.bfloat16)
    return nv.nvfp4_quantize(a.cuda()), nv.nvfp4_quantize(w.cuda(), flags=b_flags)


@pytest.mark.parametrize("M,N,K,b_flags", [(200, 272, 256, 2), (256, 256, 1024, 0), (1, 16, 256, 0),
                                           (513, 528, 768, 2)])
def test_fused_out_matches_oracle_quantization_of_fp32_c(oracle, M, N, K, b_flags):
    print(f"[fused] {M}x{N}x{K} b_flags={b_flags}", flush=True)
    qa, qb = _operands(M, N, K, 11, b_flags)
    c32 = nv.nvfp4_gemm(qa, qb, out_dtype=torch.float32)
    amax_c = float(c32.abs().max())
    ideal = np.float32(np.float32(amax_c) / np.float32(2688.0))
    for ts, what in ((ideal, "ideal ts"), (ideal / 8, "ts / 8 (saturating)"), (ideal * 4, "ts * 4"), (0.0, "ts 0")):
        amax = torch.zeros(1, dtype=torch.float32, device="cuda")
        out = _fused(qa, qb, ts, amax=amax)
        torch.cuda.synchronize()
        _check(oracle, c32, out, ts, f"{M}x{N}x{K} {what}")
        assert out.tensor_scale.item() == np.float32(ts)  # the input scale is left in place
        assert amax.item() == np.float32(amax_c), (amax.item(), amax_c)


def test_fused_out_ideal_scale_equals_plain_quantize(oracle):
    # with the tensor scale of this C itself, the fused output is nvfp4_quantize of the fp32 C
    qa, qb = _operands(384, 512, 512, 12)
    c32 = nv.nvfp4_gemm(qa, qb, out_dtype=torch.float32)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    out = nv.empty_like_quantized(384, 512, 0, "cuda")
    nv.nvfp4_gemm_nvfp4_out(qa, qb, out, amax=amax)  # first call: only for the amax
    nv.nvfp4_scale_from_amax(amax, out.tensor_scale)
    nv.nvfp4_gemm_nvfp4_out(qa, qb, out)
    ref = nv.nvfp4_quantize(c32)
    torch.cuda.synchronize()
    assert out.tensor_scale.item() == ref.tensor_scale.item()
    assert torch.equal(out.scales, ref.scales) and torch.equal(out.data, ref.data)
    nv.nvfp4_scale_from_amax(amax, ts)
    assert ts.item() == np.float32(np.float32(amax.item()) / np.float32(2688.0))


def test_fused_out_amax_is_a_running_maximum():
    qa, qb = _operands(64, 64, 256, 13)
    c32 = nv.nvfp4_gemm(qa, qb, out_dtype=torch.float32)
    big = float(c32.abs().max()) * 3
    amax = torch.full((1,), big, dtype=torch.float32, device="cuda")
    _fused(qa, qb, 1e-3, amax=amax)
    assert amax.item() == np.float32(big)
    _fused(qa, qb, 1e-3)  # amax may be omitted


def test_fused_out_grouped(oracle):
    sizes = [37, 0, 256, 100]
    M, N, K = sum(sizes), 144, 256
    offs = np.concatenate([[0], np.cumsum(sizes)]).tolist()
    a = synth.normal((M, K), 1.0, seed=14, tensor_id=92)
    ws = [synth.normal((N, K), 0.05 * (g + 1), seed=14, tensor_id=93 + g) for g in range(len(sizes))]
    qa = nv.nvfp4_quantize(a.cuda())
    qws = [nv.nvfp4_quantize(w.cuda()) for w in ws]
    qb = nv.NVFP4Tensor(torch.cat([q.data for q in qws]), torch.cat([q.scales for q in qws]),
                        torch.cat([q.tensor_scale for q in qws]), N, K, 0, len(sizes))
    c32 = nv.nvfp4_gemm(qa, qb, out_dtype=torch.float32, group_offsets=offs)
    ts = float(c32.abs().max()) / 2688.0
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    out = _fused(qa, qb, ts, group_offsets=offs, amax=amax)
    torch.cuda.synchronize()
    _check(oracle, c32, out, ts, "grouped")
    assert amax.item() == c32.abs().max().item()


def test_fused_out_fprop8b_full(oracle):
    # the Llama-3-8B FFN forward: Y [8192 x 14336] leaves the GEMM as NVFP4, all of it checked
    x, w = synth.fprop8b(0)
    qa = nv.nvfp4_quantize(x.cuda())
    qb = nv.nvfp4_quantize(w.cuda(), flags=nv.NVFP4_BLOCK2D)
    c32 = nv.nvfp4_gemm(qa, qb, out_dtype=torch.float32)
    ts = float(c32.abs().max()) / 2688.0 / 2  # a delayed scale below the ideal one
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    out = _fused(qa, qb, ts, amax=amax)
    torch.cuda.synchronize()
    print("[fused] fprop 8192x14336x4096", flush=True)
    _check(oracle, c32, out, ts, "fprop8b")
    assert amax.item() == c32.abs().max().item()
