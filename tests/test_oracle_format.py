"""Pins of the oracle's format primitives (CPU only).

Each test fixes one primitive against something other than the oracle itself: the format's own
grid and tie rule (tests/golden), an independent closed-form threshold ladder, PyTorch's
float8_e4m3fn cast and its header-only Philox4_32 engine (library routines), and the algebra of
the Sylvester Hadamard matrix.
"""
import json
import os
import subprocess

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


# ---- E2M1 ------------------------------------------------------------------------------------

def test_e2m1_decode_is_the_grid(oracle):
    vals = [oracle.e2m1_value(c) for c in range(16)]
    assert vals[:8] == GRID
    assert vals[8:] == [-g for g in GRID]
    assert np.signbit(np.float32(vals[8]))  # code 0x8 is -0


def test_e2m1_ties_golden(oracle):
    g = json.load(open(os.path.join(GOLDEN, "e2m1_ties.json")))
    idx = oracle.e2m1_rne_index(np.array(g["v"], dtype=np.float32))
    assert idx.tolist() == g["index"]
    assert [GRID[i] for i in idx] == g["value"]


def _ladder(v):
    """Closed-form round-to-nearest-even onto the E2M1 grid: count the midpoints passed, with
    each midpoint counted as passed only when the upper neighbour has the even code."""
    v = v.astype(np.float64)
    return ((v > 0.25).astype(int) + (v >= 0.75) + (v > 1.25) + (v >= 1.75) + (v > 2.5)
            + (v >= 3.5) + (v > 5.0)).astype(np.uint8)


def test_e2m1_rne_exhaustive(oracle):
    # every non-negative fp32 value, +0 up to +inf (2^31 - 2^23 + 1 bit patterns), in chunks on
    # threads (numpy and the oracle's array call release the GIL)
    from concurrent.futures import ThreadPoolExecutor
    top = int(np.array([np.inf], dtype=np.float32).view(np.uint32)[0])
    chunk = 1 << 24

    def check(b0):
        bits = np.arange(b0, min(b0 + chunk, top + 1), dtype=np.uint32)
        v = bits.view(np.float32)
        ref = ((v > 0.25).astype(np.uint8) + (v >= 0.75) + (v > 1.25) + (v >= 1.75) + (v > 2.5)
               + (v >= 3.5) + (v > 5.0)).astype(np.uint8)
        got = oracle.e2m1_rne_index(v)
        bad = np.flatnonzero(got != ref)
        return (b0, int(bits[bad[0]]), int(got[bad[0]]), int(ref[bad[0]])) if bad.size else None

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        fails = [f for f in ex.map(check, range(0, top + 1, chunk)) if f is not None]
    assert not fails, f"first mismatches (chunk, bits, oracle, ladder): {fails[:4]}"


def test_e2m1_rne_matches_threshold_ladder(oracle):
    # a strided sweep over every fp32 bit pattern in [0, 8) plus +-64 ulps around each midpoint
    # and grid point
    top = np.array([8.0], dtype=np.float32).view(np.uint32)[0]
    bits = np.arange(0, top, 241, dtype=np.uint32)
    pts = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] + GRID + [6.0], dtype=np.float32)
    near = (pts.view(np.uint32)[:, None].astype(np.int64) + np.arange(-64, 65)[None, :]).ravel()
    near = near[near >= 0].astype(np.uint32)
    v = np.concatenate([bits, near]).view(np.float32)
    v = np.concatenate([v, np.array([np.inf, 6.5, 1e30, 7.0, 1e-45], dtype=np.float32)])
    got = oracle.e2m1_rne_index(v)
    np.testing.assert_array_equal(got, _ladder(v))


# ---- E4M3 ------------------------------------------------------------------------------------

def _torch_e4m3_decode():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()


def test_e4m3_decode_matches_torch(oracle):
    ref = _torch_e4m3_decode()
    for b in range(256):
        v = oracle.e4m3_value(b)
        if np.isnan(ref[b]):
            assert np.isnan(v), b
        else:
            assert v == ref[b] and np.signbit(v) == np.signbit(ref[b]), b
    finite_nonneg = [b for b in range(128) if not np.isnan(ref[b])]
    assert len(finite_nonneg) == 127
    assert oracle.e4m3_value(0x7E) == 448.0


def _torch_e4m3_rne(s):
    return torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_rne_matches_torch_cast(oracle):
    vals = np.array([oracle.e4m3_value(b) for b in range(0x7F)], dtype=np.float64)
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    # every fp32 value within 4096 ulps of each midpoint and each E4M3 value, plus a strided sweep
    near = (np.concatenate([mids, vals.astype(np.float32)]).view(np.uint32)[:, None].astype(np.int64)
            + np.arange(-4096, 4097)[None, :]).ravel()
    top = np.array([448.0], dtype=np.float32).view(np.uint32)[0]
    bits = np.arange(0, top + 1, 997, dtype=np.int64)
    allb = np.concatenate([bits, near])
    allb = allb[(allb >= 0) & (allb <= top)].astype(np.uint32)
    s = allb.view(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_rne(s), _torch_e4m3_rne(s))


def test_e4m3_rne_spot_values(oracle):
    # observed with the PyTorch cast on this image: 17->16, 19->20, 2^-10->0, 1.5*2^-10->2^-9;
    # values above 448 clamp to 448 (0x7E) in the oracle
    s = np.array([17.0, 19.0, 2.0 ** -10, 1.5 * 2.0 ** -10, 464.0, 448.0, 0.0], dtype=np.float32)
    got = [oracle.e4m3_value(b) for b in oracle.e4m3_rne(s)]
    assert got == [16.0, 20.0, 0.0, 2.0 ** -9, 448.0, 448.0, 0.0]


# ---- Philox4x32-10 ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def torch_philox(tmp_path_factory):
    import torch.utils.cpp_extension as ce
    src = os.path.join(os.path.dirname(__file__), "helpers", "philox_torch.cpp")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_torch")
    inc = sum((["-I", p] for p in ce.include_paths()), [])
    subprocess.run(["g++", "-O1", "-std=c++17", *inc, src, "-o", exe], check=True)

    def run(triples):
        inp = "".join(f"{s} {q} {o}\n" for s, q, o in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return np.array([[int(w) for w in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64).astype(np.uint32)
    return run


def test_philox_matches_torch_engine(oracle, torch_philox):
    rng = np.random.default_rng(1234)
    triples = [(0, 0, 0), (7, 0, 0), (7, 0, 1), (2 ** 64 - 1, 2 ** 64 - 1, 2 ** 64 - 1), (7, 1 << 32, 0)]
    for _ in range(200):
        triples.append((int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 40)),
                        int(rng.integers(0, 2 ** 50))))
    ref = torch_philox(triples)
    ctr = np.array([[o & 0xFFFFFFFF, o >> 32, q & 0xFFFFFFFF, q >> 32] for s, q, o in triples],
                   dtype=np.uint64).astype(np.uint32)
    key = np.array([[s & 0xFFFFFFFF, s >> 32] for s, q, o in triples], dtype=np.uint64).astype(np.uint32)
    np.testing.assert_array_equal(oracle.philox(ctr, key), ref)


def test_rht_sign_word_is_philox_block(oracle, torch_philox):
    # the sign word is word 0 (low 16 bits) of the block at counter (0, 0, 0, 1) keyed by the seed
    for seed in [0, 7, 123456789, 2 ** 63 + 5]:
        ref = torch_philox([(seed, 1 << 32, 0)])[0]
        assert oracle.rht_sign_word(seed) == int(ref[0]) & 0xFFFF


# ---- 16x16 random Hadamard transform ---------------------------------------------------------

def _sylvester(n):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.kron(np.array([[1, 1], [1, -1]], dtype=np.int64), h)
    return h


def test_rht_matrix_is_sylvester_hadamard(oracle):
    cols = []
    for j in range(16):
        e = np.zeros(16, dtype=np.float32)
        e[j] = 1.0
        cols.append(oracle.rht16(e, 0) * 4.0)  # exact: entries +-1/4
    Hc = np.stack(cols, axis=1)
    assert np.all(np.abs(Hc) == 1.0)
    Hi = Hc.astype(np.int64)
    np.testing.assert_array_equal(Hi @ Hi.T, 16 * np.eye(16, dtype=np.int64))
    np.testing.assert_array_equal(Hi, _sylvester(16))


def test_rht_equals_quarter_H_D_u(oracle):
    rng = np.random.default_rng(5)
    H = _sylvester(16).astype(np.float64)
    for trial in range(200):
        sw = int(rng.integers(0, 1 << 16))
        u = (rng.standard_normal(16) * 10.0 ** rng.integers(-3, 4)).astype(np.float32)
        d = np.array([-1.0 if (sw >> t) & 1 else 1.0 for t in range(16)])
        ref = 0.25 * (H @ (d * u.astype(np.float64)))
        got = oracle.rht16(u, sw).astype(np.float64)
        # four butterfly stages, one fp32 rounding per output per stage
        bound = 4 * 2.0 ** -24 * np.abs(u).astype(np.float64).sum()
        assert np.all(np.abs(got - ref) <= bound), trial


def test_rht_parseval_and_inverse(oracle):
    rng = np.random.default_rng(6)
    u = rng.standard_normal(16 * 64).astype(np.float32)
    sw = oracle.rht_sign_word(7)
    y = oracle.rht16(u, sw)
    n_u = (u.astype(np.float64) ** 2).reshape(-1, 16).sum(1)
    n_y = (y.astype(np.float64) ** 2).reshape(-1, 16).sum(1)
    np.testing.assert_allclose(n_y, n_u, rtol=1e-6)
    back = oracle.rht16(y, 0)  # (1/4) H (1/4) H D u = D u
    d = np.array([-1.0 if (sw >> t) & 1 else 1.0 for t in range(16)], dtype=np.float32)
    np.testing.assert_allclose(back.reshape(-1, 16) * d, u.reshape(-1, 16), atol=1e-6)
