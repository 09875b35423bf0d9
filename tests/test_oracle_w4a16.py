"""Pins of the oracle's W4A16 reference (bf16 activations x NVFP4 weights), CPU only: brute force
against a float64 matrix product of the oracle's own dequantized weight on a small case, and
equality with the NVFP4 x NVFP4 reference when the bf16 activations are exactly the values an
NVFP4 activation tensor decodes to."""
import numpy as np
import torch

import synth


def _bf16_bits(x):
    return synth.bf16_bits(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16))


def test_w4a16_brute_force_small(oracle):
    rng = np.random.default_rng(0)
    M, N, K = 5, 7, 48
    a = rng.standard_normal((M, K)).astype(np.float32)
    a_bits = _bf16_bits(a)
    a_vals = torch.from_numpy(a_bits.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    w = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.05)
    qb = oracle.quantize(w)
    b_hat = oracle.dequantize(qb["data"], qb["scales"], qb["ts"], N, K).astype(np.float64)
    # the fp32 dequantized values are RN(q S ts); the reference keeps q S exact and applies ts
    # once, so compare against the exact product with ts factored out
    qs = oracle.dequantize(qb["data"], qb["scales"], np.float32(1.0), N, K).astype(np.float64)
    want = (a_vals @ qs.T) * float(qb["ts"])
    c, bnd = oracle.gemm_w4a16_ref(a_bits, qb, M, N, K)
    np.testing.assert_allclose(c, want, rtol=0, atol=1e-12 * np.abs(want).max())
    np.testing.assert_allclose(bnd, (np.abs(a_vals) @ np.abs(qs).T) * float(qb["ts"]), rtol=1e-15)
    assert np.all(np.abs(c - a_vals @ b_hat.T) <= 1e-6 * bnd)  # and close to the rounded decode


def test_w4a16_equals_nvfp4_gemm_on_exact_activations(oracle):
    # activations quantized to NVFP4 with ts = 1 (tensor maximum 2688): their decoded values have at
    # most 6 significant bits, so the bf16 copy is exact and both references must agree exactly
    rng = np.random.default_rng(1)
    M, N, K = 16, 32, 64
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[0, 0] = 2688.0
    qa = oracle.quantize(a)
    assert qa["ts"] == np.float32(1.0)
    a_dec = oracle.dequantize(qa["data"], qa["scales"], qa["ts"], M, K)
    a_bits = _bf16_bits(a_dec)
    assert np.array_equal(torch.from_numpy(a_bits.view(np.int16)).view(torch.bfloat16).float().numpy(), a_dec)
    qb = oracle.quantize(rng.standard_normal((N, K)).astype(np.float32), flags=oracle.BLOCK2D)
    c4, b4 = oracle.gemm_ref(qa, qb, M, N, K)
    c16, b16 = oracle.gemm_w4a16_ref(a_bits, qb, M, N, K)
    np.testing.assert_array_equal(c16, c4)
    np.testing.assert_array_equal(b16, b4)
