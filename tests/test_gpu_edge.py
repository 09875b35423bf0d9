"""The format's edge cases through the HIP quantizer (nvfp4_quantize), bit for bit against the
stored golden values and the oracle:

  * the four hand-computed golden files (every E2M1 tie, saturation, signed zero, the exact round
    trip of worked example 1, the Four-over-Six block), row-wise and column-wise, bf16 and fp32;
  * stochastic rounding at an exact tie (v = 2.5 between 2 and 3): rounds up with probability 1/2,
    over 120000 element indices, and bit-exact against the oracle's Philox stream;
  * every finite bf16 value: those with |y| <= 6 in blocks whose encode factor is exactly 1 (so the
    E2M1 rounding sees y itself), larger ones in blocks of 16 consecutive bf16 values anchored at
    their own maximum;
  * every fp32 value within 64 ulp of each E2M1 midpoint, in blocks whose encode factor is 1.

Blocks with encode factor 1: a tensor maximum of 10.5 gives ts = 10.5 / 2688 = 2^-8, and a block
whose maximum is 6 then gets scale RN(RN(6 / 6) / 2^-8) = 256 (an E4M3 value), so
e = RN(1 / RN(256 * 2^-8)) = 1 and v = |y| (worked example 2 of the golden files).
"""
import json
import os

import numpy as np
import pytest
import torch

from tests.gpu_util import assert_quant_equal, codes, oracle_input

pytestmark = pytest.mark.gpu
nv = pytest.importorskip("nvfp4_bit_block_quantize_amd")

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MIDPOINTS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.lib()


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _quantize(y: torch.Tensor, colwise: bool, flags=0, seed=0, stream_id=0):
    """Quantize the logical matrix y [R x K] row-wise, or column-wise from x = y^T."""
    x = y.t().contiguous() if colwise else y.contiguous()
    fl = flags | (nv.NVFP4_COLWISE if colwise else 0)
    print(f"[edge] shape={tuple(x.shape)} dtype={x.dtype} flags={fl}", flush=True)
    q = nv.nvfp4_quantize(x.cuda(), flags=fl, seed=seed, stream_id=stream_id)
    torch.cuda.synchronize()
    return q, x, fl


def _check(oracle, y, colwise, flags=0, what="", seed=0, stream_id=0):
    q, x, fl = _quantize(y, colwise, flags, seed, stream_id)
    ref = oracle.quantize(oracle_input(x), flags=fl, seed=seed, stream_id=stream_id)
    assert_quant_equal(q, ref, what)
    return q, ref


MODES = [(False, torch.float32), (True, torch.float32), (False, torch.bfloat16), (True, torch.bfloat16)]
MODE_IDS = ["row-f32", "col-f32", "row-bf16", "col-bf16"]


@pytest.mark.parametrize("colwise,dtype", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("name,flags", [("worked_example_1.json", 0), ("worked_example_2.json", 0),
                                        ("four_over_six_block.json", nv.NVFP4_FOUR_OVER_SIX)])
def test_golden_files(oracle, name, flags, colwise, dtype):
    g = _golden(name)
    row = torch.tensor(g["x"], dtype=torch.float32)
    for i in g.get("x_negative_zero_at", []):
        row[i] = -0.0
    # 8 copies of the golden row (a column-wise call reads its x^T 8 columns at a time)
    y = row.reshape(1, -1).repeat(8, 1).to(dtype)
    q, _ = _check(oracle, y, colwise, flags, f"{name} colwise={colwise} {dtype}")
    want_codes = np.tile(np.array(g["codes"], dtype=np.uint8), (8, 1))
    np.testing.assert_array_equal(codes(q.data.cpu().numpy()), want_codes)
    np.testing.assert_array_equal(q.scales.cpu().numpy(), np.tile(np.array(g["scales"], dtype=np.uint8), (8, 1)))
    assert q.tensor_scale.item() == g["ts"]
    if "packed_hex" in g:
        assert bytes(q.data.cpu().numpy()[0]).hex() == g["packed_hex"]
        back = nv.nvfp4_dequantize(q, torch.float32).cpu()
        # exact round trip, including the sign of zero
        assert torch.equal(back.view(torch.int32), y.float().view(torch.int32))


def test_e2m1_ties_golden_through_unit_scale_blocks(oracle):
    """tests/golden/e2m1_ties.json (ties, saturation) as values v = |y| of blocks with e = 1."""
    g = _golden("e2m1_ties.json")
    vals = [v for v in g["v"] if v <= 6.0]  # larger v would become the block maximum
    want = [i for v, i in zip(g["v"], g["index"]) if v <= 6.0]
    y = torch.zeros((8, 32), dtype=torch.float32)
    y[:, 0] = 10.5
    y[:, 16] = 6.0
    y[:, 17:17 + len(vals)] = torch.tensor(vals)
    for colwise in (False, True):
        q, _ = _check(oracle, y, colwise, 0, f"ties colwise={colwise}")
        got = codes(q.data.cpu().numpy())[:, 17:17 + len(vals)]
        np.testing.assert_array_equal(got, np.tile(np.array(want, dtype=np.uint8), (8, 1)))


@pytest.mark.parametrize("colwise", [False, True])
def test_stochastic_rounding_tie_is_fair(oracle, colwise):
    rows = 8000
    y = torch.zeros((rows, 32), dtype=torch.float32)
    y[:, 0] = 10.5
    y[:, 16] = 6.0
    y[:, 17:] = 2.5  # v = 2.5: between grid values 2 and 3, f = 1/2
    q, _ = _check(oracle, y, colwise, nv.NVFP4_SR, f"SR tie colwise={colwise}", seed=7, stream_id=0)
    c = codes(q.data.cpu().numpy())[:, 17:]
    assert set(np.unique(c).tolist()) <= {4, 5}
    n = c.size
    up = int(np.sum(c == 5))
    sigma = np.sqrt(0.25 * n)
    assert abs(up - n / 2) <= 5 * sigma, (up, n)


def _unit_scale_blocks(values: np.ndarray, dtype) -> torch.Tensor:
    """Y [R x 256]: row 0 holds the tensor maximum 10.5; every other 16-element block holds the
    anchor 6 and 15 of the given values (|value| <= 6), so every value is encoded with e = 1."""
    per = 15
    nblk = (len(values) + per - 1) // per
    blocks = np.zeros((nblk, 16), dtype=np.float32)
    blocks[:, 0] = 6.0
    flat = np.zeros(nblk * per, dtype=np.float32)
    flat[:len(values)] = values
    blocks[:, 1:] = flat.reshape(nblk, per)
    rows = (nblk + 15) // 16 + 1
    rows = (rows + 7) // 8 * 8
    y = np.zeros((rows, 256), dtype=np.float32)
    y[0, 0] = 10.5
    y.reshape(-1, 16)[16:16 + nblk] = blocks
    return torch.from_numpy(y).to(dtype)


def _all_bf16_below(limit_bits):
    pos = np.arange(0, limit_bits + 1, dtype=np.uint32) << 16
    f = pos.view(np.float32)
    return np.concatenate([f, -f])


@pytest.mark.parametrize("colwise", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_every_bf16_value_up_to_6_at_unit_scale(oracle, colwise, dtype):
    vals = _all_bf16_below(0x40C0)  # 6.0 = 0x40C0
    assert np.max(np.abs(vals)) == 6.0
    y = _unit_scale_blocks(vals, dtype)
    q, ref = _check(oracle, y, colwise, 0, f"bf16 sweep colwise={colwise} {dtype}")
    assert q.tensor_scale.item() == 2.0 ** -8
    assert np.all(ref["scales"].reshape(-1)[16:16 + (len(vals) + 14) // 15] == 0x78)  # S = 256


@pytest.mark.parametrize("colwise", [False, True])
def test_every_large_bf16_value_in_self_anchored_blocks(oracle, colwise):
    """bf16 values above 6 up to the largest finite one, 16 consecutive bit patterns per block (the
    block's maximum is its own last value), split into tensors of 16 binades each so that the block
    scales stay inside the E4M3 range."""
    lo_bits = 0x40C1
    hi_bits = 0x7F7F
    bits = np.arange(lo_bits, hi_bits + 1, dtype=np.uint32)
    exps = bits >> 7
    for e0 in range(int(exps.min()), int(exps.max()) + 1, 16):
        sel = bits[(exps >= e0) & (exps < e0 + 16)]
        vals = (sel << 16).view(np.float32)
        n = (len(vals) + 15) // 16 * 16
        padded = np.zeros(n, dtype=np.float32)
        padded[:len(vals)] = vals
        signs = np.where(np.arange(n) % 3 == 1, -1.0, 1.0).astype(np.float32)
        flat = padded * signs
        rows = (n // 256 + 1 + 7) // 8 * 8
        y = np.zeros((rows, 256), dtype=np.float32)
        y.reshape(-1)[:n] = flat
        _check(oracle, torch.from_numpy(y).to(torch.bfloat16), colwise, 0, f"bf16 large e0={e0} colwise={colwise}")


@pytest.mark.parametrize("colwise", [False, True])
def test_fp32_values_around_every_midpoint(oracle, colwise):
    vals = []
    for m in MIDPOINTS:
        c = np.float32(m)
        lo, hi = c, c
        around = [c]
        for _ in range(64):
            lo = np.nextafter(lo, np.float32(-np.inf), dtype=np.float32)
            hi = np.nextafter(hi, np.float32(np.inf), dtype=np.float32)
            around += [lo, hi]
        vals += around
    vals = np.array(vals, dtype=np.float32)
    vals = np.concatenate([vals, -vals])
    y = _unit_scale_blocks(vals, torch.float32)
    q, _ = _check(oracle, y, colwise, 0, f"midpoints colwise={colwise}")
    # the rule itself: v below a midpoint rounds down, above rounds up, on it to the even code
    got = codes(q.data.cpu().numpy()).reshape(-1, 16)[16:, 1:].reshape(-1)[:len(vals)]
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mag = grid[got & 7]
    v = np.abs(vals).astype(np.float64)
    nearest = np.abs(v[:, None] - grid[None, :])
    dmin = nearest.min(axis=1)
    assert np.all(np.abs(v - mag) == dmin)
    tie = np.sum(nearest == dmin[:, None], axis=1) > 1
    assert np.all((got[tie] & 7) % 2 == 0)
    assert np.all(((got >> 3) & 1) == np.signbit(vals))
