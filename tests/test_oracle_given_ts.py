"""Pins of the oracle's quantization with a given tensor scale (the reference for a GEMM epilogue
that quantizes its output under delayed scaling), CPU only.

The format (aissential.tech article, Summary: 16-element blocks, E4M3 block scale, FP32 tensor
scale; E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}) fixes every code once ts is given: block scale
s = RN(RN(a_b / 6) / ts) clamped to 448 and rounded to E4M3, e = 1 / (S * ts), code = nearest grid
value of |y| e (ties to even, saturating at 6), sign copied.  The expected values below are worked
by hand with ts = 0.25 (so that S = 8, e = 1/2 for the first block: every |y| e is exact)."""
import numpy as np

# block 1: a_b = 12 -> s = RN(2 / 0.25) = 8 = E4M3 0x50 (exponent 3 + bias 7, mantissa 0); e = 1/2
BLOCK1 = [12, -6, 3, 1, 0.5, 0.25, 2.5, 5, 7, 9, 11, -12, 0, -0.0, 1.5, 0.6]
# |y| e = 6, 3, 1.5, 0.5, 0.25 (tie 0 / 0.5 -> even 0), 0.125, 1.25 (tie -> 1), 2.5 (tie -> 2),
# 3.5 (tie -> 4), 4.5 (-> 4), 5.5 (-> 6), 6, 0, 0, 0.75 (tie -> 1), 0.3 (-> 0.5)
CODES1 = [7, 8 | 5, 3, 1, 0, 0, 2, 4, 6, 6, 7, 8 | 7, 0, 8, 2, 1]
# block 2: a_b = 3000 -> s = 2000 clamps to 448 = 0x7E; e = 1/112: 3000/112 saturates to 6,
# 672/112 = 6, 336/112 = 3, 56/112 = 0.5; zeros stay +0
BLOCK2 = [3000, 672, 336, 56, -3000] + [0.0] * 11
CODES2 = [7, 7, 5, 1, 8 | 7] + [0] * 11


def test_given_ts_worked_example(oracle):
    y = np.zeros((1, 48), dtype=np.float32)
    y[0, :16] = BLOCK1
    y[0, 16:32] = BLOCK2
    data, scales = oracle.quantize_given_ts(y, 0.25)
    assert scales[0].tolist() == [0x50, 0x7E, 0x00]
    codes = []
    for b in data[0]:
        codes += [int(b & 15), int(b >> 4)]
    assert codes[:16] == CODES1
    assert codes[16:32] == CODES2
    assert codes[32:] == [0] * 16


def test_given_ts_zero_scale_gives_signed_zeros(oracle):
    y = np.array([[1.0, -2.0, 0.0, -0.0] * 4], dtype=np.float32)
    data, scales = oracle.quantize_given_ts(y, 0.0)
    assert scales.tolist() == [[0]]
    codes = []
    for b in data[0]:
        codes += [int(b & 15), int(b >> 4)]
    assert codes == [0, 8, 0, 8] * 4


def test_given_ts_equals_quantize_at_the_amax_scale(oracle):
    # with ts = RN(amax / 2688) the result is the plain row-wise quantization of the same matrix
    rng = np.random.default_rng(3)
    y = (rng.standard_normal((37, 96)) * np.exp(rng.uniform(-6, 6, (37, 1)))).astype(np.float32)
    ref = oracle.quantize(y)
    data, scales = oracle.quantize_given_ts(y, ref["ts"])
    np.testing.assert_array_equal(data, ref["data"])
    np.testing.assert_array_equal(scales, ref["scales"])


def test_given_ts_strided_rows(oracle):
    rng = np.random.default_rng(4)
    big = rng.standard_normal((20, 80)).astype(np.float32)
    d1, s1 = oracle.quantize_given_ts(big[:, 16:64], 0.01)
    d2, s2 = oracle.quantize_given_ts(np.ascontiguousarray(big[:, 16:64]), 0.01)
    np.testing.assert_array_equal(d1, d2)
    np.testing.assert_array_equal(s1, s2)
