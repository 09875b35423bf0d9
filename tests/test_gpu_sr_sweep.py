"""Stochastic rounding through nvfp4_quantize on a structured sweep of (v, r16), bit for bit against
the oracle.

The rule (round up iff r16 < f * 65536, f the position of v between its two E2M1 neighbours) is
taken on the GPU by the hardware converter with r16 mapped into its random operand.  This test
puts, for every 16-bit value r16 and each of the seven grid intervals [0, 0.5) ... [4, 6), values v
at 64 r16 + d units of 2^-22 of the interval's step, d in {-2, -1, -0.5, -0.25, 0, 0.25, 0.5, 1, 2}
(fractional d matter below 1, where f * 2^22 need not be an integer), into elements whose Philox
bits are that r16: every element's r16 is known (the oracle's Philox4x32-10 at the element's
index), and element positions are assigned to (r16, interval, offset) combinations so that every
combination occurs.  The blocks have encode factor exactly 1 (tensor maximum 10.5, ts = 2^-8, an
anchor 6 in every block, scale 256), so the converter sees v itself.
"""
import numpy as np
import pytest
import torch

from tests.gpu_util import assert_quant_equal, codes

pytestmark = pytest.mark.gpu
nv = pytest.importorskip("nvfp4_bit_block_quantize_amd")

LOS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0])
STEPS = np.array([0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0])
DELTAS = np.array([-2.0, -1.0, -0.5, -0.25, 0.0, 0.25, 0.5, 1.0, 2.0])
SEED, STREAM = 7, 0


def _r16(oracle, idx):
    """The 16 random bits of logical elements idx (uint64): word (i & 7) >> 1, half i & 1, of
    Philox4x32-10 keyed by (SEED, 0) at counter (i >> 3, 0, STREAM, 0)."""
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


def _sweep_tensor(oracle, K=256):
    ncomb = len(LOS) * len(DELTAS)           # 63 (interval, offset) combinations
    per_row = K - K // 16                    # elements per row that are not block anchors
    rows = 1 + int(np.ceil(65536 * 150 / per_row))  # ~150 elements per r16 value: every r16 gets all 63
    R = (rows + 7) // 8 * 8
    r, k = np.meshgrid(np.arange(R, dtype=np.int64), np.arange(K, dtype=np.int64), indexing="ij")
    free = (k % 16 != 0) & (r > 0)
    idx = (r * K + k)[free]
    r16 = _r16(oracle, idx.astype(np.uint64))
    # rank of each element among the elements with the same r16 -> its combination
    order = np.argsort(r16, kind="stable")
    sorted_r = r16[order]
    first = np.searchsorted(sorted_r, sorted_r, side="left")
    rank = np.empty_like(order)
    rank[order] = np.arange(len(order)) - first
    comb = rank % ncomb
    iv, di = comb // len(DELTAS), comb % len(DELTAS)
    v = LOS[iv] + (64.0 * r16 + DELTAS[di]) * STEPS[iv] / 4194304.0
    v = np.maximum(v, 0.0)
    sign = np.where((rank // ncomb) % 2 == 1, -1.0, 1.0)
    y = np.zeros((R, K), dtype=np.float32)
    y[:, 0::16] = 6.0
    y[0, :] = 0.0
    y[0, 0] = 10.5
    y[free] = (sign * v).astype(np.float32)
    # every (r16, combination) pair occurs
    seen = np.zeros((65536, ncomb), dtype=bool)
    seen[r16, comb] = True
    assert seen.all(), f"{(~seen).sum()} (r16, combination) pairs missing"
    return torch.from_numpy(y)


@pytest.mark.parametrize("colwise", [False, True])
def test_stochastic_rounding_structured_sweep(oracle, colwise):
    y = _sweep_tensor(oracle)
    x = y.t().contiguous() if colwise else y
    flags = nv.NVFP4_SR | (nv.NVFP4_COLWISE if colwise else 0)
    print(f"[sr sweep] Y={tuple(y.shape)} colwise={colwise}", flush=True)
    q = nv.nvfp4_quantize(x.cuda(), flags=flags, seed=SEED, stream_id=STREAM)
    torch.cuda.synchronize()
    assert q.tensor_scale.item() == 2.0 ** -8
    ref = oracle.quantize(x.numpy(), flags=flags, seed=SEED, stream_id=STREAM)
    assert_quant_equal(q, ref, f"SR sweep colwise={colwise}")
    # both outcomes occur in every interval (the sweep sits on the decision boundary)
    c = codes(q.data.cpu().numpy()) & 7
    assert len(np.unique(c)) == 8
