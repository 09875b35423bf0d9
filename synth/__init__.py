"""Seeded synthetic inputs for the NVFP4 quantize / GEMM workloads.

This module holds no part of the quantization method: it only draws the input tensors (shapes,
value distributions, outlier structure and MoE routing) that both the HIP library and the CPU
oracle are fed with.  Every random number comes from its own C generator (synth/gen.c, built into
synth/libsynth.so): Philox4x32-10 keyed by (seed, tensor id), Box-Muller in double, Fisher-Yates
permutations.  No torch or numpy random generator is used, so the inputs depend only on the seed,
the tensor id and the element index (and the C library's log, sin, cos and sqrt).

Workloads (shapes stand in for the Llama-3-8B / Llama-3.1-405B FFN and the MoE expert layers that
the pages' throughput and checkpoint results are quoted on; no dataset or trained weight is used):
  tiny      A, B [64 x 64] fp32 ~N(0,1), 1% of entries x50
  fprop8b   X [8192 x 4096] bf16 ~N(0,1), 0.1% of channels (columns) x20; W [14336 x 4096] ~N(0,0.02)
  wgrad8b   dY [8192 x 14336] bf16 ~N(0,1e-3); X [8192 x 4096] ~N(0,1)
  moe       64 experts W_e [4096 x 1536] = 0.02 * Student-t(nu=4); X [16384 x 4096] ~N(0,1);
            top-2 routing with Zipf(1.1) expert loads
  fprop405b X [8192 x 16384] ~N(0,1), 0.1% channels x20; W [53248 x 16384] ~N(0,0.01)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "libsynth.so")
        src = os.path.join(_HERE, "gen.c")
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
            _build.build()
        L = ctypes.CDLL(path)
        P, i64, u64, u32, i32, dbl = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                      ctypes.c_int, ctypes.c_double)
        L.sg_normal.argtypes = [P, i64, u64, u32, dbl, i32, i32]
        L.sg_normal.restype = None
        L.sg_student_t.argtypes = [P, i64, i32, dbl, u64, u32, i32, i32]
        L.sg_student_t.restype = None
        L.sg_permutation.argtypes = [P, i64, u64, u32, u32]
        L.sg_permutation.restype = None
        L.sg_words.argtypes = [P, i64, u64, u32, u32]
        L.sg_words.restype = None
        _LIB = L
    return _LIB


def _empty(shape, dtype) -> torch.Tensor:
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"synthetic inputs are float32 or bfloat16, not {dtype}")
    return torch.empty(shape, dtype=dtype)


def permutation(n: int, seed=0, tensor_id=0, stream=0) -> np.ndarray:
    """A seeded uniformly drawn permutation of range(n) (int64)."""
    out = np.empty(n, dtype=np.int64)
    _lib().sg_permutation(out.ctypes.data, n, int(seed) & (2**64 - 1), int(tensor_id) & 0xFFFFFFFF, stream)
    return out


def philox_words(ncalls: int, seed=0, tensor_id=0, stream=0) -> np.ndarray:
    """The generator's raw Philox4x32-10 output words (4 per call), for its own tests."""
    out = np.empty(4 * ncalls, dtype=np.uint32)
    _lib().sg_words(out.ctypes.data, ncalls, int(seed) & (2**64 - 1), int(tensor_id) & 0xFFFFFFFF, stream)
    return out


def normal(shape, std=1.0, seed=0, tensor_id=0, dtype=torch.bfloat16) -> torch.Tensor:
    """i.i.d. N(0, std^2): element i is Box-Muller normal i of the (seed, tensor_id) stream times std,
    rounded to fp32 and then (RNE) to `dtype`."""
    out = _empty(shape, dtype)
    _lib().sg_normal(out.data_ptr(), out.numel(), int(seed) & (2**64 - 1), int(tensor_id) & 0xFFFFFFFF,
                     float(std), 1 if dtype == torch.bfloat16 else 0, _THREADS)
    return out


def outlier_columns(x: torch.Tensor, frac: float, factor: float, seed=0, tensor_id=0) -> torch.Tensor:
    """Scale round(frac * ncols) seeded columns (channels) of x by `factor` (in place, fp32 math)."""
    ncol = x.shape[1]
    n = int(round(frac * ncol))
    if n == 0:
        return x
    cols = torch.from_numpy(permutation(ncol, seed, tensor_id + 100)[:n])
    x[:, cols] = (x[:, cols].float() * factor).to(x.dtype)
    return x


def outlier_entries(x: torch.Tensor, frac: float, factor: float, seed=0, tensor_id=0) -> torch.Tensor:
    """Scale round(frac * numel) seeded entries of x by `factor` (in place)."""
    n = int(round(frac * x.numel()))
    idx = torch.from_numpy(permutation(x.numel(), seed, tensor_id + 200)[:n])
    flat = x.view(-1)
    flat[idx] = (flat[idx].float() * factor).to(x.dtype)
    return x


def student_t(shape, nu=4, scale=1.0, seed=0, tensor_id=0, dtype=torch.bfloat16) -> torch.Tensor:
    """scale * t_nu with t = z0 / sqrt(sum_{s=1..nu} z_s^2 / nu), z_s the element's normal of stream s;
    computed in double, rounded to fp32, then (RNE) to `dtype`."""
    out = _empty(shape, dtype)
    _lib().sg_student_t(out.data_ptr(), out.numel(), int(nu), float(scale), int(seed) & (2**64 - 1),
                        int(tensor_id) & 0xFFFFFFFF, 1 if dtype == torch.bfloat16 else 0, _THREADS)
    return out


def zipf_loads(n_experts=64, total=32768, s=1.1, seed=0) -> np.ndarray:
    """Per-expert row counts: Zipf(s) probabilities over expert ranks, ranks mapped to experts by a
    seeded permutation, counts by largest-remainder rounding of total * p (sum == total)."""
    ranks = np.arange(1, n_experts + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    raw = total * p
    m = np.floor(raw).astype(np.int64)
    rem = total - int(m.sum())
    order = np.argsort(-(raw - m), kind="stable")
    m[order[:rem]] += 1
    perm = permutation(n_experts, seed, 900)
    loads = np.zeros(n_experts, dtype=np.int64)
    loads[perm] = m  # rank r -> expert perm[r]
    return loads


def moe_routing(n_tokens=16384, n_experts=64, topk=2, s=1.1, seed=0):
    """Top-2 routing with Zipf loads.  Returns (loads[E], slot_token[n_tokens*topk]) where the slots
    are expert-sorted: rows offsets[e]:offsets[e+1] of the grouped activation matrix belong to
    expert e and slot_token[j] is the token feeding row j.  Token t takes slots t and t + n_tokens
    of the expert-sorted slot list (always two distinct experts when every load < n_tokens), then
    tokens are relabelled by a seeded permutation."""
    total = n_tokens * topk
    loads = zipf_loads(n_experts, total, s, seed)
    assert loads.max() < n_tokens
    slot_token = np.empty(total, dtype=np.int64)
    base = np.arange(n_tokens, dtype=np.int64)
    for k in range(topk):
        slot_token[k * n_tokens:(k + 1) * n_tokens] = base
    relabel = permutation(n_tokens, seed, 901)
    slot_token = relabel[slot_token]
    return loads, slot_token


# ---- the workloads ---------------------------------------------------------------------------

def tiny(seed=0):
    a = normal((64, 64), 1.0, seed, 1, torch.float32)
    b = normal((64, 64), 1.0, seed, 2, torch.float32)
    outlier_entries(a, 0.01, 50.0, seed, 1)
    outlier_entries(b, 0.01, 50.0, seed, 2)
    return a, b


def fprop8b(seed=0, m=8192, n=14336, k=4096):
    x = normal((m, k), 1.0, seed, 3)
    outlier_columns(x, 0.001, 20.0, seed, 3)
    w = normal((n, k), 0.02, seed, 4)
    return x, w


def wgrad8b(seed=0, tokens=8192, n_out=14336, n_in=4096):
    dy = normal((tokens, n_out), 1e-3, seed, 5)
    x = normal((tokens, n_in), 1.0, seed, 6)
    return dy, x


def moe_experts(seed=0, n_experts=64, k=4096, n=1536, workers=1):
    """Expert weights [k x n] bf16, Student-t(4) x 0.02; expert e draws from its own generator, so
    the result does not depend on `workers` (threads that generate experts concurrently)."""
    make = lambda e: student_t((k, n), 4, 0.02, seed, 1000 + e)
    if workers <= 1:
        return [make(e) for e in range(n_experts)]
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(make, range(n_experts)))


def moe_tokens(seed=0, n_tokens=16384, k=4096):
    return normal((n_tokens, k), 1.0, seed, 7)


def fprop405b(seed=0, m=8192, n=53248, k=16384):
    x = normal((m, k), 1.0, seed, 8)
    outlier_columns(x, 0.001, 20.0, seed, 8)
    w = normal((n, k), 0.01, seed, 9)
    return x, w


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16 CPU tensor (what the oracle takes for bf16 inputs)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
