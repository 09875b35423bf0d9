"""The GEMM design probe (libnvfp4_probe.so, measurement only): both inner steps it times compute
the same 128 x 128 tile of one 16-element NVFP4 block product, and it is the product the oracle
defines (binary64, tensor scales 1), within the GEMM tolerance 1e-5 * sum_k |a||b|."""
import ctypes
import os

import numpy as np
import pytest
import torch

from tests.gpu_util import gemm_check

pytestmark = pytest.mark.gpu
PROBE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "nvfp4_bit_block_quantize_amd",
                     "libnvfp4_probe.so")


@pytest.mark.parametrize("design", [0, 1, 2])
def test_design_probe_computes_the_block_product(oracle, design):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = ctypes.CDLL(PROBE)
    P = ctypes.c_void_p
    L.nvfp4_probe_design.argtypes = [ctypes.c_int, P, P, P, P, P, ctypes.c_int, ctypes.c_int, P]
    rng = np.random.default_rng(3 + design)
    a = (rng.standard_normal((128, 16)) * np.exp2(rng.integers(-4, 4, (128, 1)))).astype(np.float32)
    b = (rng.standard_normal((128, 16)) * 0.02).astype(np.float32)
    qa, qb = oracle.quantize(a), oracle.quantize(b)
    for q in (qa, qb):
        q["ts"] = np.float32(1.0)  # the probe multiplies codes and block scales only
    dev = [torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in (qa["data"], qa["scales"], qb["data"], qb["scales"])]
    c = torch.zeros((128, 128), dtype=torch.float32, device="cuda")
    print(f"[probe] design {design}", flush=True)
    st = L.nvfp4_probe_design(design, *[ctypes.c_void_p(t.data_ptr()) for t in dev], ctypes.c_void_p(c.data_ptr()), 1, 1,
                              None)
    torch.cuda.synchronize()
    assert st == 0
    cref, bnd = oracle.gemm_ref(qa, qb, 128, 128, 16)
    gemm_check(c.cpu().numpy(), cref, bnd, False, f"design {design}")
