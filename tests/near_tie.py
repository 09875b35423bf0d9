"""Near-tie tiles for Four-over-Six on 16x16 tiles.

Each tile is drawn so that one element, bisected over its fp32 values, sits where the oracle's tile
errors for target 6 and target 4 cross.  There the two errors
differ by a few units in the last place, so the choice depends on the order in which the 256
squares are added: exactly the inputs on which a summation order that changes under
transposition would make quantize(W^T) and transpose(quantize(W)) disagree.

The tensor has an anchor tile (the first) holding the tensor maximum 0.65625 = 2688 * 2^-12, so
ts = 2^-12 exactly and every other tile is scaled well below it.
"""
import numpy as np

TS = np.float32(2.0 ** -12)
ANCHOR = np.float32(2688.0 * 2.0 ** -12)


def _ordered(f):
    """fp32 -> integer whose order is the order of the floats (for bisection over fp32 values)."""
    b = int(np.array(f, dtype=np.float32).view(np.uint32))
    return -(b & 0x7FFFFFFF) if b & 0x80000000 else b


def _from_ordered(o):
    b = ((-o) | 0x80000000) if o < 0 else o
    return np.array(b, dtype=np.uint32).view(np.float32)[()]


def _gap(oracle, tile):
    s6, _ = oracle.tile_sse_2d(tile, TS, 6.0)
    s4, _ = oracle.tile_sse_2d(tile, TS, 4.0)
    return float(s6) - float(s4), s6, s4


def near_tie_tile(oracle, rng):
    """One near-tie tile.  A Gaussian tile (target 6 has the lower error) gets elements replaced,
    one at a time, by values at 60-90% of its maximum (which favour target 4) until target 4 wins;
    the last replaced element is then bisected over the fp32 values between its old and new value
    to where the two errors cross (the error is continuous in each element: at a rounding
    boundary both neighbours are equally far)."""
    tile = (rng.standard_normal((16, 16)) * 0.05).astype(np.float32)
    m = float(np.max(np.abs(tile)))
    amax_pos = np.unravel_index(int(np.argmax(np.abs(tile))), tile.shape)
    if _gap(oracle, tile)[0] >= 0:
        return None
    for flat in rng.permutation(256):
        i, j = divmod(int(flat), 16)
        if (i, j) == amax_pos:
            continue
        old = tile[i, j]
        new = np.float32(rng.choice([-1.0, 1.0]) * rng.uniform(0.6, 0.9) * m)
        tile[i, j] = new
        if _gap(oracle, tile)[0] < 0:
            continue
        lo, hi = _ordered(old), _ordered(new)
        sign_old = -1.0
        while abs(hi - lo) > 1:
            mid = (lo + hi) // 2
            tile[i, j] = _from_ordered(mid)
            if np.sign(_gap(oracle, tile)[0]) == sign_old:
                lo = mid
            else:
                hi = mid
        tile[i, j] = _from_ordered(hi if rng.integers(0, 2) else lo)
        return tile
    return None


def near_tie_tensor(oracle, tiles_r, tiles_c, seed):
    """float32 [16 tiles_r x 16 tiles_c]: tile (0, 0) is the anchor (maximum 0.65625 at its
    corner, so ts = 2^-12), every other tile a near tie."""
    rng = np.random.default_rng(seed)
    x = np.zeros((16 * tiles_r, 16 * tiles_c), dtype=np.float32)
    for a in range(tiles_r):
        for b in range(tiles_c):
            if a == 0 and b == 0:
                t = (rng.standard_normal((16, 16)) * 0.02).astype(np.float32)
                t[0, 0] = ANCHOR
            else:
                t = None
                while t is None:
                    t = near_tie_tile(oracle, rng)
            x[16 * a:16 * a + 16, 16 * b:16 * b + 16] = t
    return x
