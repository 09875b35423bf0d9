"""Pins of the oracle's Four-over-Six variants (CPU only): the tensor scale amax/1792, the scale
search over five targets, and Four-over-Six on 16x16 tiles.  Each is pinned by its closed form,
by the exact ordering of block errors that a minimum over a larger candidate set must satisfy, and
by a hand-built tile where target 4 is exact and target 6 is not."""
import numpy as np
import pytest

from tests.test_oracle_quantize import _codes


def _t(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(4, size=(rows, cols)).astype(np.float32) * np.float32(0.02)
    return x


def test_ts_for_four_is_amax_over_1792(oracle):
    x = _t(48, 64, 1)
    q = oracle.quantize(x, flags=oracle.TS_FOR_FOUR)
    amax = np.float32(np.max(np.abs(x)))
    assert q["ts"] == np.float32(amax / np.float32(1792.0))
    # with targets 6 and 4 the largest possible unclamped block scale is 448 (for the block holding
    # the tensor maximum, at target 4): every scale byte then encodes at most 448
    q46 = oracle.quantize(x, flags=oracle.TS_FOR_FOUR | oracle.FOUR_OVER_SIX)
    assert q46["scales"].max() <= 0x7E


@pytest.mark.parametrize("ts_four", [False, True])
def test_search_never_worse_than_four_over_six_never_worse_than_plain(oracle, ts_four):
    x = _t(64, 256, 2)
    extra = oracle.TS_FOR_FOUR if ts_four else 0
    fos = oracle.quantize(x, flags=oracle.FOUR_OVER_SIX | extra)
    srch = oracle.quantize(x, flags=oracle.SCALE_SEARCH | extra)
    # both start from the same target-6 encoding, so their "plain" sums agree exactly
    assert fos["sse"][1] == srch["sse"][1]
    # per block the search minimises over a superset of {6, 4}: the sums are ordered exactly
    assert srch["sse"][0] <= fos["sse"][0] <= fos["sse"][1]
    assert srch["sse"][0] < fos["sse"][0]  # Student-t blocks do use the intermediate targets


def test_search_choice_is_one_of_the_five_targets(oracle):
    x = _t(16, 512, 3)
    q = oracle.quantize(x, flags=oracle.SCALE_SEARCH)
    ts = q["ts"]
    blocks = np.abs(x).reshape(16, 32, 16).max(axis=2)
    allowed = np.zeros_like(q["scales"], dtype=bool)
    for T in (6.0, 5.5, 5.0, 4.5, 4.0):
        s = np.minimum(np.float32(np.float32(blocks / np.float32(T)) / ts), np.float32(448.0)).astype(np.float32)
        b = np.array([[oracle.lib().or_e4m3_rne(float(v)) for v in row] for row in s], dtype=np.uint8)
        allowed |= (b == q["scales"])
    assert allowed.all()


def test_four_over_six_2d_hand_built_tiles(oracle):
    # tile A (columns 0..15): grid values x 16, exactly representable when the tile maximum 64 maps
    # to 4 (scale 16), not when it maps to 6 (scale RN(64/6) -> E4M3 11); tile B (columns 16..31):
    # 2688 everywhere, so ts = 1 and target 6 is exact there (scale 448, target 4 clamps to the same)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4], dtype=np.float32) * 16
    a = np.resize(grid, (16, 16)).astype(np.float32)
    a[0, 0] = 64.0
    x = np.concatenate([a, np.full((16, 16), 2688.0, dtype=np.float32)], axis=1)
    plain = oracle.quantize(x, flags=oracle.BLOCK2D)
    fos = oracle.quantize(x, flags=oracle.BLOCK2D | oracle.FOUR_OVER_SIX)
    assert plain["ts"] == fos["ts"] == np.float32(1.0)
    e4m3 = oracle.lib().or_e4m3_rne
    assert plain["scales"][0, 0] == e4m3(float(np.float32(64.0) / np.float32(6.0)))
    assert fos["scales"][0, 0] == e4m3(16.0)
    assert plain["scales"][0, 1] == fos["scales"][0, 1] == 0x7E
    back = oracle.dequantize(fos["data"], fos["scales"], fos["ts"], 16, 32, oracle.BLOCK2D)
    np.testing.assert_array_equal(back[:, :16], a)          # exact under target 4
    assert fos["sse"][0] == 0.0 and fos["sse"][1] > 0.0
    np.testing.assert_array_equal(_codes(fos["data"])[:, 16:], _codes(plain["data"])[:, 16:])


def test_four_over_six_2d_never_worse(oracle):
    x = _t(64, 96, 4)
    q = oracle.quantize(x, flags=oracle.BLOCK2D | oracle.FOUR_OVER_SIX)
    assert q["sse"][0] <= q["sse"][1]


def _tile_squares(oracle, tile, ts, T):
    """Rounded squared errors RN(d*d) of a tile under target T, decoded independently of the
    oracle's quantizer (grid literal, the oracle's E4M3 decode of the tile's scale byte)."""
    _, sb = oracle.tile_sse_2d(tile, ts, T)
    S = np.float32(oracle.e4m3_value(sb))
    e = np.float32(1.0) / np.float32(S * ts)
    idx = oracle.e2m1_rne_index((np.abs(tile) * e).astype(np.float32)).reshape(16, 16)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    q = np.where(np.signbit(tile), -grid[idx], grid[idx]).astype(np.float32)
    d = (tile - ((q * S).astype(np.float32) * np.float32(ts)).astype(np.float32)).astype(np.float32)
    return (d * d).astype(np.float32)


def test_tile_error_is_transpose_invariant_sum_of_squares(oracle):
    """The 2D tile error is a sum of the 256 rounded squares (within fp32 summation error of the
    exact sum, so no term is dropped or doubled) and does not change, bit for bit, when the tile is
    transposed, on tiles whose squares span many binades (where the order of additions shows)."""
    rng = np.random.default_rng(11)
    ts = np.float32(2.0 ** -10)
    for trial in range(200):
        mags = np.exp2(rng.uniform(-12, 0, size=(16, 16)))
        tile = (rng.choice([-1.0, 1.0], size=(16, 16)) * mags * 2.0).astype(np.float32)
        for T in (6.0, 4.0):
            s, _ = oracle.tile_sse_2d(tile, ts, T)
            st, _ = oracle.tile_sse_2d(np.ascontiguousarray(tile.T), ts, T)
            assert s.view(np.uint32) == st.view(np.uint32), (trial, T, s, st)
            sq = _tile_squares(oracle, tile, ts, T).astype(np.float64)
            exact = float(np.sum(sq))
            assert abs(float(s) - exact) <= 256 * 2.0 ** -24 * exact, (trial, T, s, exact)


def test_four_over_six_2d_transpose_consistent_on_near_ties(oracle):
    """quantize(W^T) == transpose(quantize(W)) for BLOCK2D | FOUR_OVER_SIX, bit for bit, on random
    Student-t tiles and on tiles built at the crossing of the two candidates' errors, where a
    summation order that changes under transposition would decide differently (the witness below
    counts the tiles a row-major order of the same squares gets wrong)."""
    from tests.gpu_util import codes
    from tests.near_tie import TS, near_tie_tensor
    fl = oracle.BLOCK2D | oracle.FOUR_OVER_SIX
    for x in (_t(64, 96, 4), near_tie_tensor(oracle, 6, 7, 3)):
        q = oracle.quantize(x, flags=fl)
        qt = oracle.quantize(x, flags=fl | oracle.COLWISE)
        assert qt["ts"] == q["ts"]
        np.testing.assert_array_equal(qt["scales"], q["scales"].T)
        np.testing.assert_array_equal(codes(qt["data"]), codes(q["data"]).T)
    # witness: the near-tie tiles are sharp enough to separate summation orders
    x = near_tie_tensor(oracle, 6, 7, 3)
    split = 0
    for a in range(6):
        for b in range(7):
            if a == 0 and b == 0:
                continue
            tile = np.ascontiguousarray(x[16 * a:16 * a + 16, 16 * b:16 * b + 16])
            s6, s4 = _tile_squares(oracle, tile, TS, 6.0), _tile_squares(oracle, tile, TS, 4.0)

            def seq(v):
                acc = np.float32(0.0)
                for t in v.ravel():
                    acc = np.float32(acc + t)
                return acc
            split += (seq(s4) < seq(s6)) != (seq(s4.T) < seq(s6.T))
    assert split >= 5, split


def test_variant_combinations_rejected(oracle):
    x = _t(32, 32, 5)
    for bad in (oracle.SR | oracle.SCALE_SEARCH, oracle.FOUR_OVER_SIX | oracle.SCALE_SEARCH,
                oracle.SCALE_SEARCH | oracle.BLOCK2D, oracle.SR | oracle.FOUR_OVER_SIX):
        with pytest.raises(ValueError):
            oracle.quantize(x, flags=bad)
