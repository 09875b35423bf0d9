"""The synthetic input generator (synth/gen.c): its Philox stream, normals, Student-t draws and
permutations.  CPU only."""
import ctypes

import numpy as np
import pytest
import torch
from scipy import stats

import synth


def test_philox_words_match_the_oracle(oracle):
    # the generator's counter is (call, 0, stream, 0x5EED5EED) under key (seed, tensor id); the
    # oracle's Philox4x32-10 is pinned to PyTorch's Philox engine in test_oracle_format.py
    for seed, tid, stream in ((0, 0, 0), (7, 3, 1), (2**32 + 5, 1000, 4)):
        w = synth.philox_words(64, seed, tid, stream).reshape(-1, 4)
        ctr = np.array([[c, 0, stream, 0x5EED5EED] for c in range(64)], dtype=np.uint32)
        key = np.array([[seed & 0xFFFFFFFF, tid]] * 64, dtype=np.uint32)
        np.testing.assert_array_equal(w, oracle.philox(ctr, key))


def test_normal_is_box_muller_of_the_stream():
    w = synth.philox_words(8, 3, 11).astype(np.float64).reshape(-1, 4)
    u = (w + 0.5) / 2.0**32
    z = np.empty((8, 4))
    for p in range(2):
        r = np.sqrt(-2.0 * np.log(u[:, 2 * p]))
        z[:, 2 * p] = r * np.cos(2 * np.pi * u[:, 2 * p + 1])
        z[:, 2 * p + 1] = r * np.sin(2 * np.pi * u[:, 2 * p + 1])
    got = synth.normal((32,), 0.5, seed=3, tensor_id=11, dtype=torch.float32).numpy()
    np.testing.assert_allclose(got, (0.5 * z.reshape(-1)).astype(np.float32), rtol=2e-7, atol=0)


def test_element_depends_only_on_its_index():
    big = synth.normal((64, 1000), 1.0, seed=1, tensor_id=2, dtype=torch.float32)
    small = synth.normal((7, 1000), 1.0, seed=1, tensor_id=2, dtype=torch.float32)
    assert torch.equal(big[:7], small)
    L = synth._lib()
    one = np.empty(100_003, dtype=np.float32)
    many = np.empty(100_003, dtype=np.float32)
    L.sg_normal(one.ctypes.data, one.size, 5, 9, ctypes.c_double(1.0), 0, 1)
    L.sg_normal(many.ctypes.data, many.size, 5, 9, ctypes.c_double(1.0), 0, 7)
    np.testing.assert_array_equal(one, many)


def test_bf16_output_is_the_rounded_fp32_output():
    f = synth.normal((1000, 257), 0.02, seed=4, tensor_id=8, dtype=torch.float32)
    b = synth.normal((1000, 257), 0.02, seed=4, tensor_id=8, dtype=torch.bfloat16)
    assert torch.equal(f.to(torch.bfloat16), b)


def test_normal_distribution():
    z = synth.normal((1 << 20,), 1.0, seed=0, tensor_id=12, dtype=torch.float32).double().numpy()
    n = z.size
    assert abs(z.mean()) < 5 / np.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * np.sqrt(2.0 / n)
    assert stats.kstest(z, "norm").pvalue > 1e-4
    # different tensor ids and seeds give uncorrelated streams
    z2 = synth.normal((1 << 20,), 1.0, seed=0, tensor_id=13, dtype=torch.float32).double().numpy()
    z3 = synth.normal((1 << 20,), 1.0, seed=1, tensor_id=12, dtype=torch.float32).double().numpy()
    assert abs(np.corrcoef(z, z2)[0, 1]) < 5 / np.sqrt(n)
    assert abs(np.corrcoef(z, z3)[0, 1]) < 5 / np.sqrt(n)


def test_student_t_distribution():
    t = synth.student_t((1 << 19,), nu=4, scale=1.0, seed=0, tensor_id=1000, dtype=torch.float32).double().numpy()
    assert stats.kstest(t, "t", args=(4,)).pvalue > 1e-4
    scaled = synth.student_t((1 << 10,), nu=4, scale=0.02, seed=0, tensor_id=1000, dtype=torch.float32).double().numpy()
    np.testing.assert_allclose(scaled, (t[:1 << 10] * 0.02).astype(np.float32), rtol=2e-7)


def test_permutation():
    for n in (1, 2, 10, 4096, 100_003):
        p = synth.permutation(n, seed=0, tensor_id=3)
        assert np.array_equal(np.sort(p), np.arange(n))
    # position of element 0 over many seeds is uniform over 8 places (chi-square)
    pos = [int(np.argmax(synth.permutation(8, seed=s, tensor_id=1) == 0)) for s in range(4000)]
    counts = np.bincount(pos, minlength=8)
    assert stats.chisquare(counts).pvalue > 1e-4


def test_moe_routing_is_top2_over_distinct_experts():
    loads, slot_token = synth.moe_routing()
    assert loads.sum() == 32768 and loads.min() >= 85 and loads.max() <= 8210
    off = np.concatenate([[0], np.cumsum(loads)])
    expert_of_slot = np.repeat(np.arange(64), loads)
    # each token appears in exactly two slots, of two different experts
    order = np.argsort(slot_token, kind="stable")
    assert np.array_equal(np.bincount(slot_token, minlength=16384), np.full(16384, 2))
    e = expert_of_slot[order].reshape(-1, 2)
    assert np.all(e[:, 0] != e[:, 1])
    assert off[-1] == 32768
