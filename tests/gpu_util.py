"""Helpers shared by the GPU parity tests: move synthetic inputs to the device and to the oracle,
and compare library outputs with the oracle's."""
import numpy as np
import torch

import synth

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def oracle_input(x: torch.Tensor) -> np.ndarray:
    """The same values the GPU sees, as the oracle takes them (fp32, or bf16 bit patterns)."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return synth.bf16_bits(x)
    return x.numpy()


def codes(data: np.ndarray) -> np.ndarray:
    d = np.asarray(data, dtype=np.uint8)
    out = np.empty((d.shape[0], d.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = d & 15
    out[:, 1::2] = d >> 4
    return out


def assert_quant_equal(q, ref, what=""):
    """Bit-exact comparison of a library NVFP4Tensor with an oracle result."""
    d = q.data.cpu().numpy()
    s = q.scales.cpu().numpy()
    ts = q.tensor_scale.cpu().numpy()[0]
    assert ts.view(np.uint32) == np.float32(ref["ts"]).view(np.uint32), (what, ts, ref["ts"])
    np.testing.assert_array_equal(s, ref["scales"], err_msg=f"{what}: scale bytes")
    if not np.array_equal(d, ref["data"]):
        cg, cr = codes(d), codes(ref["data"])
        bad = np.argwhere(cg != cr)
        raise AssertionError(f"{what}: {len(bad)} codes differ, first at {bad[:5].tolist()}: "
                             f"gpu {cg[tuple(bad[0])]} oracle {cr[tuple(bad[0])]}")


def code_value(c):
    return np.where(c & 8, -1.0, 1.0) * GRID[c & 7]


def gemm_check(c_gpu: np.ndarray, c_ref: np.ndarray, bound: np.ndarray, bf16_out: bool, what=""):
    """|C - C_ref| <= 1e-5 * sum_k |a||b|  (+ 2^-8 |C_ref| for a bf16 output) on every cell that
    the oracle computed (non-NaN)."""
    m = ~np.isnan(c_ref)
    err = np.abs(c_gpu.astype(np.float64)[m] - c_ref[m])
    tol = 1e-5 * bound[m] + (2.0 ** -8 * np.abs(c_ref[m]) if bf16_out else 0.0)
    worst = np.max(err - tol) if err.size else -1
    assert np.all(err <= tol), f"{what}: {np.sum(err > tol)} of {err.size} cells out of tolerance (worst excess {worst})"
    return float(np.max(err / np.maximum(bound[m], 1e-300))) if err.size else 0.0


def seeded_tiles(M, N, n, seed, tile=128):
    """n distinct tile-aligned rectangles (row0, col0, h, w) chosen by a seeded generator, plus the
    first and last full rows' tiles, clipped to the matrix."""
    tm, tn = (M + tile - 1) // tile, (N + tile - 1) // tile
    rng = np.random.default_rng(seed)
    pick = rng.choice(tm * tn, size=min(n, tm * tn), replace=False)
    out = []
    for p in pick:
        i, j = divmod(int(p), tn)
        out.append((i * tile, j * tile, min(tile, M - i * tile), min(tile, N - j * tile)))
    return out
