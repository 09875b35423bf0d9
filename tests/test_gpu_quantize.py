"""GPU parity of nvfp4_quantize / nvfp4_rht_quantize / nvfp4_dequantize against the CPU oracle.

Quantize is bit-exact (packed codes, E4M3 scale bytes and the FP32 tensor scale), including
stochastic rounding with the same Philox stream.  With the Hadamard transform the transformed
values must agree within 2 ulp, at most 1e-4 of the codes may differ and only by one grid step,
and scales / tensor scale must equal the oracle's quantization of the GPU's own transformed
values bit for bit."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import assert_quant_equal, codes, oracle_input

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_bit_block_quantize_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.lib()


def _run(x, flags, seed=0, stream_id=0, rht=False, sign_seed=0, want_rht=False):
    xd = x.cuda()
    R, K = (x.shape[1], x.shape[0]) if flags & nv.NVFP4_COLWISE else tuple(x.shape)
    rht_out = torch.empty((R, K), dtype=torch.float32, device="cuda") if want_rht else None
    print(f"[quantize] shape={tuple(x.shape)} dtype={x.dtype} flags={flags} rht={rht}", flush=True)
    if rht:
        q = nv.nvfp4_rht_quantize(xd, sign_seed, flags=flags, seed=seed, stream_id=stream_id, rht_out=rht_out)
    else:
        q = nv.nvfp4_quantize(xd, flags=flags, seed=seed, stream_id=stream_id)
    torch.cuda.synchronize()
    return q, rht_out


def _gauss(shape, seed, dtype=torch.bfloat16, std=1.0):
    return synth.normal(shape, std, seed=seed, tensor_id=50, dtype=dtype)


CASES = [
    # (name, shape of x, dtype, flags)
    ("row_rne_ragged", (300, 1040), torch.bfloat16, 0),
    ("row_rne_f32", (64, 64), torch.float32, 0),
    ("row_sr", (300, 1040), torch.bfloat16, nv.NVFP4_SR),
    ("row_4over6", (300, 1040), torch.bfloat16, nv.NVFP4_FOUR_OVER_SIX),
    ("row_2d", (208, 1056), torch.bfloat16, nv.NVFP4_BLOCK2D),
    ("row_2d_f32", (48, 80), torch.float32, nv.NVFP4_BLOCK2D),
    ("col_rne_ragged", (528, 392), torch.bfloat16, nv.NVFP4_COLWISE),
    ("col_rne_aligned", (512, 256), torch.bfloat16, nv.NVFP4_COLWISE),
    ("col_rne_f32", (48, 40), torch.float32, nv.NVFP4_COLWISE),
    ("col_sr", (528, 392), torch.bfloat16, nv.NVFP4_COLWISE | nv.NVFP4_SR),
    ("col_4over6", (528, 392), torch.bfloat16, nv.NVFP4_COLWISE | nv.NVFP4_FOUR_OVER_SIX),
    ("col_2d", (528, 400), torch.bfloat16, nv.NVFP4_COLWISE | nv.NVFP4_BLOCK2D),
    # Shapes on which both passes take the XCD order (pass-1 grid and pass-2 grid multiples of 8;
    # for 16x16 tiles, rows of 1024-byte multiples), with a band or slab count that is not a
    # multiple of 8, so some XCDs own one band or slab fewer than others:
    # 1D: 32670 blocks, pass-2 grid 128, 8 pass-1 parts, 63.8 slabs of 512 blocks
    ("row_rne_xcd_order", (495, 1056), torch.bfloat16, 0),
    ("row_sr_xcd_order", (495, 1056), torch.bfloat16, nv.NVFP4_SR),
    ("row_4over6_xcd_order", (495, 1056), torch.bfloat16, nv.NVFP4_FOUR_OVER_SIX),
    # 2D: 63 bands of one 1024-chunk slab each (8 pass-1 parts, pass-2 grid 16), bf16 and fp32
    ("row_2d_xcd_order", (1008, 512), torch.bfloat16, nv.NVFP4_BLOCK2D),
    ("row_2d_xcd_order_f32", (1008, 256), torch.float32, nv.NVFP4_BLOCK2D),
    ("row_2d_4over6_xcd_order", (1008, 512), torch.bfloat16, nv.NVFP4_BLOCK2D | nv.NVFP4_FOUR_OVER_SIX),
    # 2D: 260 bands of 8 slabs (256 pass-1 parts, pass-2 grid 520)
    ("row_2d_xcd_order_wide", (4160, 4096), torch.bfloat16, nv.NVFP4_BLOCK2D),
]


@pytest.mark.parametrize("name,shape,dtype,flags", CASES, ids=[c[0] for c in CASES])
def test_quantize_matches_oracle(oracle, name, shape, dtype, flags):
    if flags & nv.NVFP4_FOUR_OVER_SIX:
        x = synth.student_t(shape, 4, 0.02, seed=1, tensor_id=51, dtype=dtype)
    else:
        x = _gauss(shape, 2, dtype)
        synth.outlier_entries(x, 0.01, 30.0, seed=2, tensor_id=52)
    q, _ = _run(x, flags, seed=7, stream_id=3)
    ref = oracle.quantize(oracle_input(x), flags=flags, seed=7, stream_id=3)
    assert_quant_equal(q, ref, name)


@pytest.mark.parametrize("flags", [0, nv.NVFP4_COLWISE, nv.NVFP4_BLOCK2D, nv.NVFP4_COLWISE | nv.NVFP4_SR])
def test_quantize_strided_input(oracle, flags):
    base = _gauss((256, 160), 3)
    x = base[:, :144]  # leading dimension 160 > 144 columns
    q, _ = _run(x, flags, seed=5)
    ref = oracle.quantize(oracle_input(x.contiguous()), flags=flags, seed=5)
    assert_quant_equal(q, ref, f"strided flags={flags}")


@pytest.mark.parametrize("kind", ["zeros", "signed_zeros", "tiny", "one_hot", "huge_range"])
def test_quantize_degenerate_inputs(oracle, kind):
    x = torch.zeros((32, 64), dtype=torch.float32)
    if kind == "signed_zeros":
        x[3, 5] = -0.0
        x[7, :] = -0.0
    elif kind == "tiny":
        x = _gauss((32, 64), 4, torch.float32) * 1e-38  # ts is subnormal
    elif kind == "one_hot":
        x[5, 17] = -3.0
    elif kind == "huge_range":
        x = _gauss((32, 64), 5, torch.float32)
        x[0, 0] = 3e38
        x[1, :16] = 1e-30
    for flags in (0, nv.NVFP4_COLWISE, nv.NVFP4_BLOCK2D, nv.NVFP4_SR, nv.NVFP4_FOUR_OVER_SIX):
        q, _ = _run(x, flags, seed=1)
        ref = oracle.quantize(oracle_input(x), flags=flags, seed=1)
        assert_quant_equal(q, ref, f"{kind} flags={flags}")


def test_quantize_empty():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    q = nv.nvfp4_quantize(x)
    torch.cuda.synchronize()
    assert q.tensor_scale.item() == 0.0 and q.data.numel() == 0


def test_quantize_repeatable():
    x = _gauss((512, 2048), 6).cuda()
    a = nv.nvfp4_quantize(x, flags=nv.NVFP4_SR, seed=7)
    b = nv.nvfp4_quantize(x, flags=nv.NVFP4_SR, seed=7)
    torch.cuda.synchronize()
    assert torch.equal(a.data, b.data) and torch.equal(a.scales, b.scales)


# ---- random Hadamard transform -----------------------------------------------------------------------

def _check_rht(oracle, x, flags, sign_seed, seed=0, stream_id=0, name=""):
    q, rht_gpu = _run(x, flags, seed=seed, stream_id=stream_id, rht=True, sign_seed=sign_seed, want_rht=True)
    ref = oracle.quantize(oracle_input(x), flags=flags, seed=seed, stream_id=stream_id, rht=True,
                          sign_seed=sign_seed, want_rht_out=True)
    rg = rht_gpu.cpu().numpy()
    ulp = np.spacing(np.abs(ref["rht_out"]).astype(np.float32))
    assert np.all(np.abs(rg - ref["rht_out"]) <= 2 * ulp), f"{name}: transform beyond 2 ulp"
    # scales / ts / codes must equal the oracle's quantization of the GPU's own transformed values
    re = oracle.quantize(rg, flags=flags & ~nv.NVFP4_COLWISE, seed=seed, stream_id=stream_id)
    assert_quant_equal(q, re, f"{name} (on the GPU transform)")
    cg, cr = codes(q.data.cpu().numpy()), codes(ref["data"])
    diff = cg != cr
    assert diff.mean() <= 1e-4, f"{name}: {diff.mean():.2e} of codes differ"
    if diff.any():
        steps = np.abs((cg[diff] & 7).astype(int) - (cr[diff] & 7).astype(int))
        assert np.all(steps <= 1)
    return float(diff.mean())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("flags", [nv.NVFP4_COLWISE, nv.NVFP4_COLWISE | nv.NVFP4_SR, 0, nv.NVFP4_SR,
                                   nv.NVFP4_COLWISE | nv.NVFP4_FOUR_OVER_SIX, nv.NVFP4_FOUR_OVER_SIX])
def test_rht_quantize_matches_oracle(oracle, flags, dtype):
    x = _gauss((528, 400), 7, dtype)
    synth.outlier_columns(x, 0.02, 20.0, seed=7, tensor_id=53)
    frac = _check_rht(oracle, x, flags, sign_seed=7, seed=7, name=f"rht flags={flags} {dtype}")
    assert frac == 0.0  # same butterfly order as the oracle: identical


@pytest.mark.parametrize("flags", [0, nv.NVFP4_SR])
def test_rht_row_xcd_order(oracle, flags):
    # row-wise transform with both passes in XCD order: 32670 blocks, pass-1 grid 32, pass-2 grid 128,
    # 127.6 slabs of 256 blocks
    x = _gauss((495, 1056), 11)
    frac = _check_rht(oracle, x, flags, sign_seed=3, seed=5, name=f"rht rows xcd order flags={flags}")
    assert frac == 0.0


def test_rht_sign_seed_changes_transform(oracle):
    x = _gauss((64, 64), 8)
    _, a = _run(x, nv.NVFP4_COLWISE, rht=True, sign_seed=1, want_rht=True)
    _, b = _run(x, nv.NVFP4_COLWISE, rht=True, sign_seed=2, want_rht=True)
    assert not torch.equal(a, b)


# ---- dequantize ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("flags", [0, nv.NVFP4_BLOCK2D])
def test_dequantize_matches_oracle(oracle, flags):
    x = _gauss((208, 1056), 9)
    q, _ = _run(x, flags)
    y32 = nv.nvfp4_dequantize(q, torch.float32)
    y16 = nv.nvfp4_dequantize(q, torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.dequantize(q.data.cpu().numpy(), q.scales.cpu().numpy(), q.tensor_scale.item(), 208, 1056, flags)
    g = y32.cpu().numpy()
    assert g.tobytes() == ref.tobytes()
    np.testing.assert_array_equal(y16.cpu().view(torch.int16).numpy(),
                                  torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy())


def test_dequantize_strided_output_and_full_weight(oracle):
    # into a column window of a wider output (ldy > K), both dtypes: the columns outside stay
    x = _gauss((48, 160), 10)
    q, _ = _run(x, 0)
    ref = oracle.dequantize(q.data.cpu().numpy(), q.scales.cpu().numpy(), q.tensor_scale.item(), 48, 160, 0)
    for dt in (torch.float32, torch.bfloat16):
        big = torch.full((48, 160 + 24), 7.0, dtype=dt, device="cuda")
        nv.nvfp4_dequantize(q, out=big[:, 8:168])
        got = big.cpu()
        assert torch.all(got[:, :8] == 7.0) and torch.all(got[:, 168:] == 7.0)
        want = torch.from_numpy(ref).to(dt)
        assert torch.equal(got[:, 8:168].view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           want.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
    # the decode of the full 2D-quantized fprop weight [14336 x 4096], as the bench times it
    _, w = synth.fprop8b(0)
    qw = nv.nvfp4_quantize(w.cuda(), flags=nv.NVFP4_BLOCK2D)
    y16 = nv.nvfp4_dequantize(qw, torch.bfloat16).cpu()
    ref = oracle.dequantize(qw.data.cpu().numpy(), qw.scales.cpu().numpy(), qw.tensor_scale.item(),
                            qw.rows, qw.k, nv.NVFP4_BLOCK2D)
    assert torch.equal(y16.view(torch.int16), torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16))


def test_round_trip_tiny_workload(oracle):
    a, b = synth.tiny(0)
    for t in (a, b):
        q, _ = _run(t, 0)
        y = nv.nvfp4_dequantize(q).cpu().numpy()
        ref = oracle.quantize(t.numpy())
        assert_quant_equal(q, ref, "tiny")
        err = np.abs(y - t.numpy())
        assert err.max() <= 0.25 * np.abs(t.numpy()).max() / 6 * 2


# ---- full-size workloads ---------------------------------------------------------------------------------

def test_fprop8b_quantize_full(oracle):
    x, w = synth.fprop8b(0)
    qx, _ = _run(x, 0)
    assert_quant_equal(qx, oracle.quantize(oracle_input(x)), "X [8192x4096] 1D")
    qw, _ = _run(w, nv.NVFP4_BLOCK2D)
    assert_quant_equal(qw, oracle.quantize(oracle_input(w), flags=nv.NVFP4_BLOCK2D), "W [14336x4096] 2D")


def test_wgrad8b_rht_quantize_full(oracle):
    dy, x = synth.wgrad8b(0)
    f = _check_rht(oracle, dy, nv.NVFP4_COLWISE | nv.NVFP4_SR, sign_seed=7, seed=7, name="dY^T RHT+SR")
    g = _check_rht(oracle, x, nv.NVFP4_COLWISE, sign_seed=7, name="X^T RHT")
    print(f"code mismatch fraction dY {f:.2e} X {g:.2e}")


def test_moe_expert_four_over_six(oracle):
    w = synth.moe_experts(0, n_experts=1)[0]
    q, _ = _run(w, nv.NVFP4_COLWISE | nv.NVFP4_FOUR_OVER_SIX)
    ref = oracle.quantize(oracle_input(w), flags=nv.NVFP4_COLWISE | nv.NVFP4_FOUR_OVER_SIX)
    assert_quant_equal(q, ref, "W_e^T 4/6")
    chosen, plain = ref["sse"]
    print(f"4/6 MSE reduction on one Student-t expert: {100 * (1 - chosen / plain):.2f}%")
    assert chosen < plain
