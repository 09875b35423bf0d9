"""Stochastic rounding at the boundaries of the encode's shortcuts, bit for bit against the oracle.

The library's stochastic-rounding encode (i) takes each block's encode factor e from a
per-workgroup table of the 127 scale bytes, (ii) when e is 0 or in [2^-14, 2^100] (bf16 input;
[1, 2^100] for fp32) feeds the converter ceil(RN(|y| e 2^23)) from one multiply instead of
ceil(RN(RN(|y| e) 2^23)), and (iii) divides the block maximum by 6 and by ts through reciprocals
when ts is in [2^-100, 2^100] and the block maximum is 0 or in [2^-90, 2^100].  Where (ii) could
differ from the two-step product at all, the operand is 0 or 1 before the ceil, and an operand of 1
rounds up only for r16 = 0.  So the first test puts the smallest nonzero values exactly at the
elements whose r16 is 0 (the oracle's Philox4x32-10 at the element's index), in blocks whose maxima
put e on both sides of the threshold; the others put ts and the block maxima on both sides of the
reciprocal ranges.
"""
import numpy as np
import pytest
import torch

from tests.gpu_util import assert_quant_equal

pytestmark = pytest.mark.gpu
nv = pytest.importorskip("nvfp4_bit_block_quantize_amd")

SEED, STREAM = 11, 2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.lib()


def _r16(oracle, idx):
    """The 16 random bits of logical elements idx: word (i & 7) >> 1, half i & 1, of Philox4x32-10
    keyed by (SEED, 0) at counter (i >> 3, 0, STREAM, 0)."""
    calls = np.unique(idx >> 3)
    ctr = np.zeros((len(calls), 4), dtype=np.uint32)
    ctr[:, 0] = (calls & 0xFFFFFFFF).astype(np.uint32)
    ctr[:, 1] = (calls >> 32).astype(np.uint32)
    ctr[:, 2] = STREAM
    key = np.zeros((len(calls), 2), dtype=np.uint32)
    key[:, 0] = SEED
    words = oracle.philox(ctr, key)
    pos = np.searchsorted(calls, idx >> 3)
    w = words[pos, (idx & 7) >> 1]
    return ((w >> (16 * (idx & 1).astype(np.uint32))) & 0xFFFF).astype(np.int64)


def _quantize_both(oracle, y, colwise, what):
    """Quantize logical Y [R x K] (row-wise, or column-wise from x = Y^T) on the GPU and in the oracle."""
    x = y.t().contiguous() if colwise else y
    flags = nv.NVFP4_SR | (nv.NVFP4_COLWISE if colwise else 0)
    print(f"[sr paths] {what} Y={tuple(y.shape)} dtype={y.dtype} colwise={colwise}", flush=True)
    q = nv.nvfp4_quantize(x.cuda(), flags=flags, seed=SEED, stream_id=STREAM)
    torch.cuda.synchronize()
    xo = x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()
    ref = oracle.quantize(xo, flags=flags, seed=SEED, stream_id=STREAM)
    assert_quant_equal(q, ref, f"{what} colwise={colwise} {y.dtype}")
    return q


def _tiny_at_zero_r16(oracle, dtype, R=8192, K=1024):
    """Y with the smallest nonzero magnitudes at every element whose r16 is 0.  Block b of each row
    has maximum 1.5 * 2^k (one anchor element), k stepping through a range that puts the block's
    encode factor e ~ 6 / max on both sides of the fold threshold; the other elements are uniform
    in +-max / 8.  Returns Y and the exponents k of the blocks that hold a tiny element."""
    rng = np.random.default_rng(5)
    if dtype == torch.bfloat16:
        amax, klo, khi = 2.0 ** 22, 8, 21   # e from ~2^-19 to ~2^-6 (threshold 2^-14)
        tiny = np.array([2.0 ** -133, 3 * 2.0 ** -133, 2.0 ** -130, 2.0 ** -126, 1.5 * 2.0 ** -120, 2.0 ** -100])
    else:
        amax, klo, khi = 2.0 ** 12, -4, 11  # e from ~2^-8 to ~2^6 (threshold 1)
        tiny = np.array([2.0 ** -149, 2.0 ** -148, 3 * 2.0 ** -149, 2.0 ** -140, 2.0 ** -126, 2.0 ** -110])
    nb = K // 16
    kexp = klo + (np.arange(R * nb) % (khi - klo + 1))
    kexp = rng.permutation(kexp).reshape(R, nb)
    bmax = 1.5 * np.exp2(kexp.astype(np.float64))
    y = rng.uniform(-0.125, 0.125, size=(R, K)) * np.repeat(bmax, 16, axis=1)
    idx = np.arange(R * K, dtype=np.uint64)
    zero_r16 = (_r16(oracle, idx) == 0).reshape(R, K)
    # anchor: the first element of each block whose r16 is not 0
    blk = zero_r16.reshape(R, nb, 16)
    first_free = np.argmax(~blk, axis=2)
    rows = np.repeat(np.arange(R), nb)
    cols = (np.tile(np.arange(nb), R) * 16 + first_free.reshape(-1))
    y[rows, cols] = np.where(rng.random(R * nb) < 0.5, -1.0, 1.0) * bmax.reshape(-1)
    zr, zc = np.nonzero(zero_r16)
    y[zr, zc] = tiny[np.arange(len(zr)) % len(tiny)] * np.where(np.arange(len(zr)) % 2 == 0, 1.0, -1.0)
    y[0, 1:16] = 0.0
    y[0, 0] = amax
    y[0, 16 + (zero_r16[0, 16:32].argmin())] = amax  # tensor maximum also in a regular block
    return torch.from_numpy(y.astype(np.float32)).to(dtype), kexp[zr, zc // 16]


@pytest.mark.parametrize("colwise", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_smallest_values_at_zero_r16_across_the_fold_threshold(oracle, dtype, colwise):
    y, ks = _tiny_at_zero_r16(oracle, dtype)
    # both sides of the threshold hold tiny elements (e ~ 6 / (1.5 * 2^k))
    thr = 14 + 2 if dtype == torch.bfloat16 else 2
    assert np.sum(ks <= thr - 2) >= 8 and np.sum(ks >= thr + 2) >= 8, ks
    _quantize_both(oracle, y, colwise, "tiny at r16 = 0")


@pytest.mark.parametrize("amax", [1e-33, 1e35])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("colwise", [False, True])
def test_tensor_scale_outside_the_reciprocal_range(oracle, amax, dtype, colwise):
    # ts = amax / 2688: about 2^-121 and 2^105
    rng = np.random.default_rng(6)
    y = rng.standard_normal((256, 512)) * (amax / 5.0)
    y[3, 7] = amax
    y[9, 16:32] = amax * 2.0 ** -20 * rng.standard_normal(16)
    _quantize_both(oracle, torch.from_numpy(y.astype(np.float32)).to(dtype), colwise, f"amax {amax:g}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("colwise", [False, True])
def test_block_maxima_around_the_reciprocal_lower_bound(oracle, dtype, colwise):
    # ts ~ 1 / 2688 (tensor maximum 1); block maxima from 2^-100 to 2^-80, zero blocks, and a block
    # with values right at 2^-90
    rng = np.random.default_rng(7)
    R, K = 128, 512
    nb = K // 16
    kexp = -100 + (np.arange(R * nb) % 21)
    bmax = np.exp2(rng.permutation(kexp).astype(np.float64)).reshape(R, nb)
    y = rng.uniform(-1.0, 1.0, size=(R, K)) * np.repeat(bmax, 16, axis=1)
    y[:, ::16] = np.repeat(bmax, 1, axis=1)
    y[5, 32:48] = 0.0
    y[6, 64:80] = 2.0 ** -90 * np.array([1.0, -1.0] * 8)
    y[0, 0] = 1.0
    _quantize_both(oracle, torch.from_numpy(y.astype(np.float32)).to(dtype), colwise, "block maxima near 2^-90")
