"""GPU parity of nvfp4_gemm against the oracle's binary64 block-scaled GEMM.

Pass condition: |C - C_ref| <= 1e-5 * sum_k |a_ik||b_jk| per output cell (plus 2^-8 |C_ref| for a
bf16 output, whose rounding the bound leaves out).  The GEMM inputs are the library's own
quantized operands copied back, so the check isolates the multiply (quantize parity is tested
separately)."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import gemm_check, seeded_tiles

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_bit_block_quantize_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.lib()


def _host(q):
    return {"data": q.data.cpu().numpy(), "scales": q.scales.cpu().numpy(),
            "ts": q.tensor_scale.cpu().numpy()[0], "flags": q.flags}


def _gemm_case(oracle, a, b, a_flags=0, b_flags=0, out_dtype=torch.float32, tiles=None, what=""):
    print(f"[gemm] {what} A={tuple(a.shape)} B={tuple(b.shape)} out={out_dtype}", flush=True)
    qa = nv.nvfp4_quantize(a.cuda(), flags=a_flags)
    qb = nv.nvfp4_quantize(b.cuda(), flags=b_flags)
    c = nv.nvfp4_gemm(qa, qb, out_dtype=out_dtype)
    torch.cuda.synchronize()
    M, N, K = qa.rows, qb.rows, qa.k
    cref, bnd = oracle.gemm_ref(_host(qa), _host(qb), M, N, K, tiles=tiles)
    return gemm_check(c.float().cpu().numpy(), cref, bnd, out_dtype == torch.bfloat16, what)


def test_gemm_tiny_full(oracle):
    a, b = synth.tiny(0)
    rel = _gemm_case(oracle, a, b, what="tiny 64x64x64")
    print(f"max |err| / bound = {rel:.3e}")


@pytest.mark.parametrize("M,N,K", [(200, 136, 80), (1, 1, 16), (129, 257, 1040), (256, 256, 4096)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gemm_ragged_shapes(oracle, M, N, K, out_dtype):
    a = synth.normal((M, K), 1.0, seed=1, tensor_id=60, dtype=torch.bfloat16)
    b = synth.normal((N, K), 0.02, seed=1, tensor_id=61, dtype=torch.bfloat16)
    _gemm_case(oracle, a, b, out_dtype=out_dtype, what=f"{M}x{N}x{K}")


# the pipelined kernel moves block scales two K steps at a time: K = 256 (one pair, later pairs
# clamped), 768 (three pairs), 1280; K = 384 (an odd number of steps) takes the guarded kernel
@pytest.mark.parametrize("K", [256, 384, 768, 1280])
@pytest.mark.parametrize("flags", [(0, 0), (2, 2), (0, 2)])
def test_gemm_k_pairs(oracle, K, flags):
    a = synth.normal((272, K), 1.0, seed=9, tensor_id=70, dtype=torch.bfloat16)
    b = synth.normal((528, K), 0.05, seed=9, tensor_id=71, dtype=torch.bfloat16)
    _gemm_case(oracle, a, b, a_flags=flags[0], b_flags=flags[1], out_dtype=torch.float32,
               what=f"K={K} flags={flags}")


def test_gemm_2d_weight_scales(oracle):
    a = synth.normal((96, 512), 1.0, seed=2, tensor_id=62)
    b = synth.normal((160, 512), 0.02, seed=2, tensor_id=63)
    _gemm_case(oracle, a, b, b_flags=nv.NVFP4_BLOCK2D, out_dtype=torch.bfloat16, what="2D B")
    _gemm_case(oracle, a, b, a_flags=nv.NVFP4_BLOCK2D, b_flags=nv.NVFP4_BLOCK2D, what="2D A and B")


def test_gemm_one_hot_selects_weight_row(oracle):
    # A rows with one element 2.625 (-> ts 2^-10, scale 448, code 6: exact) pick columns of B_hat
    K = 256
    a = torch.zeros((8, K), dtype=torch.float32)
    picks = [0, 31, 100, 255, 17, 64, 128, 200]
    for i, k in enumerate(picks):
        a[i, k] = 2.625
    b = synth.normal((48, K), 1.0, seed=3, tensor_id=64, dtype=torch.float32)
    qa, qb = nv.nvfp4_quantize(a.cuda()), nv.nvfp4_quantize(b.cuda())
    c = nv.nvfp4_gemm(qa, qb, out_dtype=torch.float32).cpu()
    yb = nv.nvfp4_dequantize(qb).cpu()
    for i, k in enumerate(picks):
        torch.testing.assert_close(c[i], 2.625 * yb[:, k], rtol=2 ** -22, atol=0)


def test_gemm_grouped_small(oracle):
    sizes = [0, 37, 128, 1, 90, 300]
    M, N, K = sum(sizes), 96, 160
    offs = np.concatenate([[0], np.cumsum(sizes)]).tolist()
    a = synth.normal((M, K), 1.0, seed=4, tensor_id=65)
    ws = [synth.normal((N, K), 0.05 * (g + 1), seed=4, tensor_id=66 + g) for g in range(len(sizes))]
    qa = nv.nvfp4_quantize(a.cuda())
    qws = [nv.nvfp4_quantize(w.cuda()) for w in ws]
    G = len(sizes)
    qb = nv.NVFP4Tensor(torch.cat([q.data for q in qws]), torch.cat([q.scales for q in qws]),
                        torch.cat([q.tensor_scale for q in qws]), N, K, 0, G)
    c = nv.nvfp4_gemm(qa, qb, out_dtype=torch.float32, group_offsets=offs).cpu().numpy()
    ha = _host(qa)
    for g in range(G):
        r0, r1 = offs[g], offs[g + 1]
        if r1 == r0:
            continue
        sub = {"data": ha["data"][r0:r1], "scales": ha["scales"][r0:r1], "ts": ha["ts"], "flags": 0}
        cref, bnd = oracle.gemm_ref(sub, _host(qws[g]), r1 - r0, N, K)
        gemm_check(c[r0:r1], cref, bnd, False, f"group {g}")


def test_gemm_fprop8b_sampled_tiles(oracle):
    x, w = synth.fprop8b(0)
    M, N = x.shape[0], w.shape[0]
    tiles = seeded_tiles(M, N, 64, seed=0) + [(0, 0, 1, N), (M - 1, 0, 1, N)]
    rel = _gemm_case(oracle, x, w, b_flags=nv.NVFP4_BLOCK2D, out_dtype=torch.bfloat16, tiles=tiles,
                     what="fprop 8192x14336x4096")
    print(f"max |err| / bound = {rel:.3e}")


def test_gemm_wgrad8b_rht_sampled_tiles(oracle):
    dy, x = synth.wgrad8b(0)
    qa = nv.nvfp4_rht_quantize(dy.cuda(), 7, flags=nv.NVFP4_COLWISE | nv.NVFP4_SR, seed=7)
    qb = nv.nvfp4_rht_quantize(x.cuda(), 7, flags=nv.NVFP4_COLWISE)
    c = nv.nvfp4_gemm(qa, qb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    M, N, K = qa.rows, qb.rows, qa.k
    tiles = seeded_tiles(M, N, 64, seed=1) + [(0, 0, 1, N), (M - 1, 0, 1, N)]
    cref, bnd = oracle.gemm_ref(_host(qa), _host(qb), M, N, K, tiles=tiles)
    gemm_check(c.cpu().numpy(), cref, bnd, False, "wgrad 14336x4096x8192")
    # the transforms cancel in the product: dW stays close to the unquantized dY^T X
    r0, c0, h, w_ = tiles[0]
    exact = (dy[:, r0:r0 + h].double().T @ x[:, c0:c0 + w_].double()).numpy()
    got = c.cpu().numpy()[r0:r0 + h, c0:c0 + w_]
    rel = np.linalg.norm(got - exact) / np.linalg.norm(exact)
    print(f"relative error of NVFP4 wgrad vs bf16 inputs on one tile: {rel:.3f}")
    assert rel < 0.35


@pytest.mark.parametrize("K", [80, 256])
@pytest.mark.parametrize("case", ["tiny_scales", "huge_spikes"])
def test_gemm_degenerate_tensor_scales(oracle, case, K):
    """Tensor scales whose product under- or overflows fp32 while C itself is representable: the
    epilogue multiplies by ts_a and then by ts_b, never by RN(ts_a * ts_b).  tiny_scales: inputs
    ~N(0, 2^-116), so ts_a * ts_b falls below the smallest normal fp32 (the product would carry ~15
    bits); huge_spikes: one 2^76 entry per operand at different k (ts ~ 2^64.6 each, so ts_a * ts_b
    overflows to inf), every other block's scale underflows to zero and C is exactly 0 (inf * 0
    would be NaN)."""
    if case == "tiny_scales":
        a = synth.normal((96, K), 2.0 ** -58, seed=5, tensor_id=90, dtype=torch.float32)
        b = synth.normal((80, K), 2.0 ** -58, seed=5, tensor_id=91, dtype=torch.float32)
    else:
        a = synth.normal((96, K), 1.0, seed=5, tensor_id=92, dtype=torch.float32)
        b = synth.normal((80, K), 1.0, seed=5, tensor_id=93, dtype=torch.float32)
        a[0, 0] = 2.0 ** 76
        b[0, 1] = 2.0 ** 76
    ts_a = np.float32(a.abs().max().item()) / np.float32(2688.0)
    ts_b = np.float32(b.abs().max().item()) / np.float32(2688.0)
    with np.errstate(over="ignore", under="ignore"):
        prod = np.float32(ts_a * ts_b)
    assert (prod < np.float32(2.0 ** -126)) if case == "tiny_scales" else np.isinf(prod)
    for out_dtype in (torch.float32, torch.bfloat16):
        _gemm_case(oracle, a, b, out_dtype=out_dtype, what=f"degenerate {case} K={K}")


def test_gemm_grouped_beyond_one_launch(oracle):
    # 200 expert groups (more than one launch's group table holds), empty groups included, weights
    # from one grouped quantize call; every group checked against the oracle, both output types
    rng = np.random.default_rng(31)
    sizes = rng.integers(0, 40, 200)
    sizes[[0, 127, 128, 199]] = [0, 0, 33, 5]
    G, N, K = len(sizes), 48, 256
    M = int(sizes.sum())
    offs = np.concatenate([[0], np.cumsum(sizes)]).tolist()
    a = synth.normal((M, K), 1.0, seed=31, tensor_id=400)
    w = torch.stack([synth.normal((N, K), 0.02 * (1 + g % 7), seed=31, tensor_id=401 + g) for g in range(G)])
    qa = nv.nvfp4_quantize(a.cuda())
    qb = nv.nvfp4_quantize_grouped(w.cuda())
    ha, hb = _host(qa), _host(qb)
    ts_b = qb.tensor_scale.cpu().numpy()
    for out_dtype in (torch.float32, torch.bfloat16):
        print(f"[gemm] 200 groups out={out_dtype}", flush=True)
        c = nv.nvfp4_gemm(qa, qb, out_dtype=out_dtype, group_offsets=offs).float().cpu().numpy()
        for g in range(G):
            r0, r1 = offs[g], offs[g + 1]
            if r1 == r0:
                continue
            sub_a = {"data": ha["data"][r0:r1], "scales": ha["scales"][r0:r1], "ts": ha["ts"], "flags": 0}
            sub_b = {"data": hb["data"][g * N:(g + 1) * N], "scales": hb["scales"][g * N:(g + 1) * N],
                     "ts": ts_b[g], "flags": 0}
            cref, bnd = oracle.gemm_ref(sub_a, sub_b, r1 - r0, N, K)
            gemm_check(c[r0:r1], cref, bnd, out_dtype == torch.bfloat16, f"group {g}")
    # the same groups with the output quantized in the epilogue: the oracle's quantization of the
    # fp32 C with the given tensor scale
    c32 = nv.nvfp4_gemm(qa, qb, out_dtype=torch.float32, group_offsets=offs)
    ts = float(c32.abs().max()) / 2688.0
    out = nv.empty_like_quantized(M, N, 0, "cuda")
    out.tensor_scale.fill_(ts)
    nv.nvfp4_gemm_nvfp4_out(qa, qb, out, group_offsets=offs)
    data, scales = oracle.quantize_given_ts(c32.cpu().numpy(), np.float32(ts))
    np.testing.assert_array_equal(out.scales.cpu().numpy(), scales)
    np.testing.assert_array_equal(out.data.cpu().numpy(), data)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gemm_grouped_half_tiles(oracle, out_dtype):
    """Grouped GEMM whose groups end in bands of 1..128 rows (computed as 128 x 256 tiles in a launch
    of their own) next to groups ending in 129..256 rows (full tiles): remainders at the boundaries
    (1, 127, 128, 129, 255, 256, 257, 384, 385, 512), and more half tiles than compute units, so that
    with bf16 C each workgroup of the half launch runs several tiles.  Every output is checked."""
    rng = np.random.default_rng(41)
    edge = [1, 127, 128, 129, 255, 256, 257, 384, 385, 512, 0, 2]
    sizes = np.concatenate([edge, rng.integers(1, 129, 120)])
    G, N, K = len(sizes), 768, 512
    M = int(sizes.sum())
    offs = np.concatenate([[0], np.cumsum(sizes)]).tolist()
    print(f"[gemm] {G} groups, {M} rows, half tiles {3 * int(np.sum((sizes % 256 > 0) & (sizes % 256 <= 128)))}, "
          f"out={out_dtype}", flush=True)
    a = synth.normal((M, K), 1.0, seed=41, tensor_id=600)
    w = torch.stack([synth.normal((N, K), 0.02 * (1 + g % 5), seed=41, tensor_id=601 + g) for g in range(G)])
    qa = nv.nvfp4_quantize(a.cuda())
    qb = nv.nvfp4_quantize_grouped(w.cuda())
    ha, hb = _host(qa), _host(qb)
    ts_b = qb.tensor_scale.cpu().numpy()
    c = nv.nvfp4_gemm(qa, qb, out_dtype=out_dtype, group_offsets=offs).float().cpu().numpy()
    worst = 0.0
    for g in range(G):
        r0, r1 = offs[g], offs[g + 1]
        if r1 == r0:
            continue
        sub_a = {"data": ha["data"][r0:r1], "scales": ha["scales"][r0:r1], "ts": ha["ts"], "flags": 0}
        sub_b = {"data": hb["data"][g * N:(g + 1) * N], "scales": hb["scales"][g * N:(g + 1) * N],
                 "ts": ts_b[g], "flags": 0}
        cref, bnd = oracle.gemm_ref(sub_a, sub_b, r1 - r0, N, K)
        worst = max(worst, gemm_check(c[r0:r1], cref, bnd, out_dtype == torch.bfloat16, f"group {g} ({r1 - r0} rows)"))
    print(f"max |err| / bound = {worst:.3e}")
