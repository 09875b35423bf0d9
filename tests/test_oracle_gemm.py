"""Pins of the oracle's block-scaled GEMM reference (CPU only): brute force in exact rational
arithmetic on tiny inputs, one-hot rows that select a row of B, an independent decode (E2M1 grid
literal x PyTorch's E4M3 decode) fed to numpy's matmul, and tile-subset consistency."""
from fractions import Fraction

import numpy as np
import pytest
import torch

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _decode_exact(q, blk2d=False):
    """Independent decode: value = grid[code] * E4M3(scale) (exact in float64), no tensor scale."""
    d = q["data"]
    R, K = d.shape[0], d.shape[1] * 2
    codes = np.empty((R, K), dtype=np.uint8)
    codes[:, 0::2] = d & 15
    codes[:, 1::2] = d >> 4
    vals = np.where(codes & 8, -1.0, 1.0) * GRID[codes & 7]
    s = E4M3[q["scales"]]
    if blk2d:
        s = np.repeat(s, 16, axis=0)
    return vals * np.repeat(s, 16, axis=1)


def _quant(oracle, x, flags=0):
    q = oracle.quantize(np.ascontiguousarray(x, dtype=np.float32), flags=flags)
    q["flags"] = flags
    return q


def test_gemm_exact_rational_tiny(oracle):
    rng = np.random.default_rng(0)
    a = rng.standard_normal((4, 32)).astype(np.float32)
    b = rng.standard_normal((3, 32)).astype(np.float32) * 3
    qa, qb = _quant(oracle, a), _quant(oracle, b)
    c, bnd = oracle.gemm_ref(qa, qb, 4, 3, 32)
    da, db = _decode_exact(qa), _decode_exact(qb)
    tsab = Fraction(float(qa["ts"])) * Fraction(float(qb["ts"]))
    for i in range(4):
        for j in range(3):
            exact = sum(Fraction(float(da[i, k])) * Fraction(float(db[j, k])) for k in range(32)) * tsab
            absb = sum(abs(Fraction(float(da[i, k])) * Fraction(float(db[j, k]))) for k in range(32)) * tsab
            assert abs(Fraction(c[i, j]) - exact) <= Fraction(2.0 ** -50) * absb
            assert abs(Fraction(bnd[i, j]) - absb) <= Fraction(2.0 ** -50) * absb


def test_gemm_one_hot_rows_select_b(oracle):
    rng = np.random.default_rng(1)
    K = 64
    b = rng.standard_normal((8, K)).astype(np.float32)
    a = np.zeros((4, K), dtype=np.float32)
    picks = [0, 17, 40, 63]
    for i, k in enumerate(picks):
        a[i, k] = 2.625  # amax 2.625 -> ts = 2^-10, scale 448, code 6.0: the value is exact
    qa, qb = _quant(oracle, a), _quant(oracle, b)
    assert qa["ts"] == np.float32(2.0 ** -10)
    c, _ = oracle.gemm_ref(qa, qb, 4, 8, K)
    yb = oracle.dequantize(qb["data"], qb["scales"], qb["ts"], 8, K).astype(np.float64)
    db = _decode_exact(qb) * float(qb["ts"])
    for i, k in enumerate(picks):
        np.testing.assert_array_equal(c[i], 2.625 * db[:, k])
        np.testing.assert_allclose(c[i], 2.625 * yb[:, k], rtol=2.0 ** -22)


@pytest.mark.parametrize("b2d", [False, True])
def test_gemm_matches_independent_decode_and_matmul(oracle, b2d):
    import synth
    a_t, b_t = synth.tiny(0)
    a, b = a_t.numpy(), b_t.numpy()
    qa = _quant(oracle, a)
    qb = _quant(oracle, b, oracle.BLOCK2D if b2d else 0)
    c, bnd = oracle.gemm_ref(qa, qb, 64, 64, 64)
    da = _decode_exact(qa) * float(qa["ts"])
    db = _decode_exact(qb, b2d) * float(qb["ts"])
    ref = da @ db.T
    assert np.all(np.abs(c - ref) <= 1e-13 * (np.abs(da) @ np.abs(db).T))
    np.testing.assert_allclose(bnd, np.abs(da) @ np.abs(db).T, rtol=1e-14)
    # a transposed operand or a dropped block scale would break this
    assert not np.allclose(c, (da @ db.T).T)


def test_gemm_tiles_match_full(oracle):
    rng = np.random.default_rng(2)
    a = rng.standard_normal((48, 64)).astype(np.float32)
    b = rng.standard_normal((40, 64)).astype(np.float32)
    qa, qb = _quant(oracle, a), _quant(oracle, b)
    full, _ = oracle.gemm_ref(qa, qb, 48, 40, 64)
    tiles = [(0, 0, 16, 16), (16, 24, 32, 16), (47, 39, 1, 1)]
    part, _ = oracle.gemm_ref(qa, qb, 48, 40, 64, tiles=tiles)
    for r0, c0, h, w in tiles:
        np.testing.assert_array_equal(part[r0:r0 + h, c0:c0 + w], full[r0:r0 + h, c0:c0 + w])
    assert np.isnan(part[0, 20])
