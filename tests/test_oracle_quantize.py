"""Pins of the oracle's quantize / dequantize (CPU only): hand-computed worked examples
(tests/golden), invariants and metamorphic relations of the format, statistical unbiasedness of
stochastic rounding, Four-over-Six's per-block optimality, and the format's storage cost."""
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _golden(name):
    return json.load(open(os.path.join(GOLDEN, name)))


def _codes(data):
    """Unpack [R][K/2] bytes into [R][K] codes, low nibble first."""
    d = np.asarray(data, dtype=np.uint8)
    out = np.empty((d.shape[0], d.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = d & 15
    out[:, 1::2] = d >> 4
    return out


def _bf16(x):
    import torch
    return synth.bf16_bits(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16))


# ---- worked examples -------------------------------------------------------------------------

@pytest.mark.parametrize("as_bf16", [False, True])
def test_worked_example_1_exact_round_trip(oracle, as_bf16):
    g = _golden("worked_example_1.json")
    x = np.array(g["x"], dtype=np.float32).reshape(g["rows"], g["cols"])
    x[0, 15] = -0.0
    q = oracle.quantize(_bf16(x) if as_bf16 else x)
    assert q["ts"] == np.float32(g["ts"])
    assert q["scales"].ravel().tolist() == g["scales"]
    assert _codes(q["data"]).ravel().tolist() == g["codes"]
    assert q["data"].tobytes().hex() == g["packed_hex"]
    y = oracle.dequantize(q["data"], q["scales"], q["ts"], 1, 16)
    assert y.tobytes() == x.tobytes()  # bit-exact, including -0


def test_worked_example_2_tie_rules(oracle):
    g = _golden("worked_example_2.json")
    x = np.array(g["x"], dtype=np.float32).reshape(g["rows"], g["cols"])
    q = oracle.quantize(x)
    assert q["ts"] == np.float32(g["ts"])
    assert q["scales"].ravel().tolist() == g["scales"]
    assert _codes(q["data"]).ravel().tolist() == g["codes"]


def test_four_over_six_golden_block(oracle):
    g = _golden("four_over_six_block.json")
    x = np.array(g["x"], dtype=np.float32).reshape(g["rows"], g["cols"])
    q = oracle.quantize(x, flags=oracle.FOUR_OVER_SIX)
    assert q["ts"] == np.float32(g["ts"])
    assert q["scales"].ravel().tolist() == g["scales"]
    assert _codes(q["data"]).ravel().tolist() == g["codes"]
    assert q["sse"] == (g["sse_chosen"], g["sse_plain"])
    plain = oracle.quantize(x)
    assert plain["scales"].ravel().tolist() == [126, 120]


# ---- tensor scale, block scale and element invariants ----------------------------------------

def _random_tensor(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def test_tensor_scale_is_amax_over_2688(oracle):
    for seed, scale in [(0, 1.0), (1, 1e-3), (2, 300.0)]:
        x = _random_tensor((48, 96), seed, scale)
        for flags in [0, oracle.COLWISE, oracle.BLOCK2D]:
            q = oracle.quantize(x, flags=flags)
            assert q["ts"] == np.float32(np.abs(x).max()) / np.float32(2688.0)


def test_block_scale_covers_block_max(oracle):
    # the block maximum maps to the top of the grid (code magnitude 7 = 6.0) whenever the block
    # scale is a normal E4M3 value; scale bytes never exceed 0x7E
    x = _random_tensor((64, 256), 3)
    q = oracle.quantize(x)
    c = _codes(q["data"]).reshape(64, 16, 16)
    xb = x.reshape(64, 16, 16)
    arg = np.abs(xb).argmax(axis=2)
    top = np.take_along_axis(c & 7, arg[..., None], axis=2)[..., 0]
    normal = q["scales"] >= 8
    assert normal.mean() > 0.99
    assert np.all(top[normal] == 7)
    assert q["scales"].max() <= 0x7E


def test_dequant_error_within_half_step(oracle):
    x = _random_tensor((32, 512), 4)
    q = oracle.quantize(x)
    y = oracle.dequantize(q["data"], q["scales"], q["ts"], 32, 512)
    S = np.array([oracle.e4m3_value(b) for b in range(256)], dtype=np.float64)[q["scales"]]
    d = np.repeat(S, 16, axis=1) * np.float64(q["ts"])
    # grid steps are 0.5 below 2, 1 below 4, 2 up to 6: half a step times d, plus fp32 rounding
    v = np.abs(x) / d
    half = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0)) * d
    assert np.all(np.abs(x - y) <= half * (1 + 2.0 ** -20) + 1e-30)


def test_zero_tensor_and_signed_zeros(oracle):
    x = np.zeros((2, 32), dtype=np.float32)
    x[1, 3] = -0.0
    q = oracle.quantize(x)
    assert q["ts"] == 0.0
    assert np.all(q["scales"] == 0)
    c = _codes(q["data"])
    assert c[1, 3] == 8 and c.sum() == 8


def test_format_storage_cost(oracle):
    x = _random_tensor((64, 256), 5)
    q1 = oracle.quantize(x)
    q2 = oracle.quantize(x, flags=oracle.BLOCK2D)
    n = x.size
    assert q1["data"].nbytes == n // 2 and q1["scales"].nbytes == n // 16
    assert q2["data"].nbytes == n // 2 and q2["scales"].nbytes == n // 256
    assert 8 * (q1["data"].nbytes + q1["scales"].nbytes) / n == 4.5
    assert 8 * (q2["data"].nbytes + q2["scales"].nbytes) / n == 4.03125


# ---- metamorphic relations ---------------------------------------------------------------------

@pytest.mark.parametrize("flags_name", ["", "SR", "BLOCK2D", "COLWISE"])
def test_power_of_two_scaling(oracle, flags_name):
    flags = getattr(oracle, flags_name) if flags_name else 0
    x = _random_tensor((32, 64), 6)
    q = oracle.quantize(x, flags=flags, seed=9)
    for k in (-3, 5):
        qk = oracle.quantize((x * np.float32(2.0 ** k)).astype(np.float32), flags=flags, seed=9)
        assert qk["ts"] == q["ts"] * np.float32(2.0 ** k)
        np.testing.assert_array_equal(qk["data"], q["data"])
        np.testing.assert_array_equal(qk["scales"], q["scales"])


@pytest.mark.parametrize("flags_name", ["", "SR", "BLOCK2D", "FOUR_OVER_SIX"])
def test_negation_flips_only_sign_bits(oracle, flags_name):
    flags = getattr(oracle, flags_name) if flags_name else 0
    x = _random_tensor((32, 64), 7)
    q = oracle.quantize(x, flags=flags, seed=3)
    qn = oracle.quantize(-x, flags=flags, seed=3)
    assert qn["ts"] == q["ts"]
    np.testing.assert_array_equal(qn["scales"], q["scales"])
    np.testing.assert_array_equal(qn["data"], q["data"] ^ 0x88)


def test_permutation_inside_block_permutes_codes(oracle):
    x = _random_tensor((8, 64), 8)
    rng = np.random.default_rng(0)
    perm = rng.permutation(16)
    xp = x.reshape(8, 4, 16)[:, :, perm].reshape(8, 64)
    q = oracle.quantize(x)
    qp = oracle.quantize(np.ascontiguousarray(xp))
    np.testing.assert_array_equal(qp["scales"], q["scales"])
    np.testing.assert_array_equal(_codes(qp["data"]).reshape(8, 4, 16),
                                  _codes(q["data"]).reshape(8, 4, 16)[:, :, perm])


@pytest.mark.parametrize("flags_name", ["", "SR", "FOUR_OVER_SIX"])
def test_colwise_is_rowwise_of_transpose(oracle, flags_name):
    flags = getattr(oracle, flags_name) if flags_name else 0
    x = _random_tensor((64, 48), 9)
    qc = oracle.quantize(x, flags=flags | oracle.COLWISE, seed=11, stream_id=2)
    qr = oracle.quantize(np.ascontiguousarray(x.T), flags=flags, seed=11, stream_id=2)
    for key in ("data", "scales"):
        np.testing.assert_array_equal(qc[key], qr[key])
    assert qc["ts"] == qr["ts"]


def test_block2d_is_transpose_invariant(oracle):
    x = _random_tensor((64, 96), 10)
    qr = oracle.quantize(x, flags=oracle.BLOCK2D)
    qc = oracle.quantize(x, flags=oracle.BLOCK2D | oracle.COLWISE)
    np.testing.assert_array_equal(qc["scales"], qr["scales"].T)
    np.testing.assert_array_equal(_codes(qc["data"]), _codes(qr["data"]).T)


def test_block2d_single_nonzero_tile(oracle):
    x = np.zeros((32, 64), dtype=np.float32)
    x[20, 37] = 3.0
    x[0, 0] = 6.0
    q = oracle.quantize(x, flags=oracle.BLOCK2D)
    nz = np.argwhere(q["scales"] != 0).tolist()
    assert nz == [[0, 0], [1, 2]]
    c = _codes(q["data"])
    assert sorted(map(tuple, np.argwhere(c != 0).tolist())) == [(0, 0), (20, 37)]
    assert c[20, 37] == 7  # the tile maximum maps to 6


def test_block2d_matches_1d_on_uniform_rows(oracle):
    # if all 16 rows of a tile are equal, the 2D tile maximum equals each row's block maximum
    row = _random_tensor((1, 128), 12)
    x = np.repeat(row, 32, axis=0)
    q2 = oracle.quantize(x, flags=oracle.BLOCK2D)
    q1 = oracle.quantize(x)
    np.testing.assert_array_equal(q2["data"], q1["data"])
    np.testing.assert_array_equal(np.repeat(q2["scales"], 16, axis=0), q1["scales"])


# ---- stochastic rounding -----------------------------------------------------------------------

def test_sr_unbiased_over_1e6_draws(oracle):
    g = _golden("worked_example_2.json")
    row = np.array(g["x"], dtype=np.float32)
    n = 1_000_000
    x = np.tile(row, (n, 1))
    q = oracle.quantize(x, flags=oracle.SR, seed=7)
    assert q["ts"] == np.float32(2.0 ** -8)
    assert np.all(q["scales"][:, 1] == 120)  # block 1: d = 1, so v = |y| exactly
    c = _codes(q["data"])[:, 16:]
    vals = np.where(c & 8, -1.0, 1.0) * GRID[c & 7]
    mean = vals.mean(axis=0)
    target = row[16:].astype(np.float64)
    step = np.array([1.0 if abs(t) >= 2 else 0.5 for t in target])
    step[np.abs(target) >= 4] = 2.0
    tol = 5 * (step / 2) / np.sqrt(n) + 2.0 ** -16 * step
    assert np.all(np.abs(mean - target) <= tol), (mean - target)
    # exactly representable values never move; every draw is one of the two grid neighbours
    on_grid = np.isin(np.abs(target), GRID)
    assert np.all(vals[:, on_grid] == target[on_grid])
    lo = np.array([GRID[GRID <= abs(t)].max() for t in target])
    mag = np.abs(vals)
    assert np.all((mag >= lo[None, :]) & (mag - lo[None, :] <= step[None, :]))
    # the tie 2.5 goes up with probability exactly 1/2: 32768 of the 65536 16-bit draws
    j = list(target).index(2.5)
    p_up = (np.abs(vals[:, j]) == 3.0).mean()
    assert abs(p_up - 0.5) <= 5 * 0.5 / np.sqrt(n)


def test_sr_is_deterministic_and_seeded(oracle):
    x = _random_tensor((16, 64), 13)
    a = oracle.quantize(x, flags=oracle.SR, seed=7)
    b = oracle.quantize(x, flags=oracle.SR, seed=7)
    c = oracle.quantize(x, flags=oracle.SR, seed=8)
    d = oracle.quantize(x, flags=oracle.SR, seed=7, stream_id=1)
    np.testing.assert_array_equal(a["data"], b["data"])
    assert not np.array_equal(a["data"], c["data"])
    assert not np.array_equal(a["data"], d["data"])
    np.testing.assert_array_equal(a["scales"], c["scales"])  # scales are always round-to-nearest


# ---- Four-over-Six ------------------------------------------------------------------------------

def test_four_over_six_never_worse_per_block(oracle):
    import torch
    w = synth.student_t((256, 512), 4, 0.02, seed=0, tensor_id=77, dtype=torch.float32).numpy()
    plain = oracle.quantize(w)
    fos = oracle.quantize(w, flags=oracle.FOUR_OVER_SIX)
    yp = oracle.dequantize(plain["data"], plain["scales"], plain["ts"], 256, 512).astype(np.float64)
    yf = oracle.dequantize(fos["data"], fos["scales"], fos["ts"], 256, 512).astype(np.float64)
    ep = ((w - yp) ** 2).reshape(256, 32, 16).sum(2)
    ef = ((w - yf) ** 2).reshape(256, 32, 16).sum(2)
    assert np.all(ef <= ep * (1 + 1e-6) + 1e-30)
    assert fos["sse"][0] < fos["sse"][1]
    assert abs(fos["sse"][1] - ep.sum()) <= 1e-5 * ep.sum()
    assert abs(fos["sse"][0] - ef.sum()) <= 1e-5 * ef.sum()
    # blocks that keep target 6 are bit-identical to plain quantization
    same = fos["scales"] == plain["scales"]
    assert same.mean() > 0.3
    cp = _codes(plain["data"]).reshape(256, 32, 16)
    cf = _codes(fos["data"]).reshape(256, 32, 16)
    assert np.all(cp[same] == cf[same])
    assert fos["ts"] == plain["ts"]


# ---- RHT quantize ---------------------------------------------------------------------------------

def test_rht_quantize_equals_quantize_of_transformed(oracle):
    x = _random_tensor((64, 32), 14)
    q = oracle.quantize(x, flags=oracle.COLWISE, rht=True, sign_seed=7, want_rht_out=True)
    # Y = x^T (COLWISE), then each 16-chunk along K transformed
    y = oracle.rht16(np.ascontiguousarray(x.T), oracle.rht_sign_word(7)).reshape(32, 64)
    np.testing.assert_array_equal(q["rht_out"], y)
    q2 = oracle.quantize(y)
    for key in ("data", "scales"):
        np.testing.assert_array_equal(q[key], q2[key])
    assert q["ts"] == q2["ts"]


def test_rht_smooths_channel_outliers(oracle):
    # the RHT spreads a lone outlier over its 16-chunk: the block peak drops by about 4x while the
    # block energy is unchanged (orthogonal transform)
    rng = np.random.default_rng(15)
    x = rng.standard_normal((256, 64)).astype(np.float32)
    x[::16, 5] = 20.0  # an outlier every 16 tokens in channel 5
    q = oracle.quantize(x, flags=oracle.COLWISE, rht=True, sign_seed=7, want_rht_out=True)
    u = np.ascontiguousarray(x.T).reshape(64, 16, 16)
    y = q["rht_out"].reshape(64, 16, 16)
    peak_u = np.abs(u[5]).max(axis=1)
    peak_y = np.abs(y[5]).max(axis=1)
    assert np.all(peak_y < 0.5 * peak_u)
    np.testing.assert_allclose((y.astype(np.float64) ** 2).sum(2), (u.astype(np.float64) ** 2).sum(2),
                               rtol=1e-5)
