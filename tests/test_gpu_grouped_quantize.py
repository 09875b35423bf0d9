"""GPU parity of nvfp4_quantize_grouped: G equally shaped tensors quantized by one call, each with
its own tensor scale, group g drawing stochastic rounding from stream stream_id + g, into one
group-contiguous NVFP4 tensor.

Pass condition (bit-exact): every group equals the oracle's quantization of that group's tensor
with stream id stream_id + g (codes, scale bytes, tensor scale), and equals the library's own
single-tensor call on it.  Groups differ in magnitude by powers of ten, so a tensor scale taken from
the wrong group changes every code."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import assert_quant_equal, oracle_input

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_bit_block_quantize_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.lib()


def _group(q, g):
    rows_s = q.scales.shape[0] // q.groups
    return nv.NVFP4Tensor(q.data[g * q.rows:(g + 1) * q.rows], q.scales[g * rows_s:(g + 1) * rows_s],
                          q.tensor_scale[g:g + 1], q.rows, q.k, q.flags)


def _groups_input(G, rows, cols, dtype, seed, pad_rows=0, pad_cols=0):
    x = torch.empty((G, rows + pad_rows, cols + pad_cols), dtype=dtype)
    for g in range(G):
        t = synth.normal((rows + pad_rows, cols + pad_cols), 10.0 ** (g % 5 - 2), seed=seed, tensor_id=300 + g,
                         dtype=torch.float32)
        synth.outlier_entries(t, 0.01, 30.0, seed, 300 + g)
        x[g] = t.to(dtype)
    return x


F = nv
CASES = [
    (0, "1D rows"), (F.NVFP4_COLWISE, "1D cols"), (F.NVFP4_BLOCK2D, "2D rows"),
    (F.NVFP4_COLWISE | F.NVFP4_BLOCK2D, "2D cols"), (F.NVFP4_FOUR_OVER_SIX, "4/6 rows"),
    (F.NVFP4_COLWISE | F.NVFP4_FOUR_OVER_SIX, "4/6 cols"), (F.NVFP4_BLOCK2D | F.NVFP4_FOUR_OVER_SIX, "4/6 2D"),
    (F.NVFP4_SR, "SR rows"), (F.NVFP4_COLWISE | F.NVFP4_SR, "SR cols"),
    (F.NVFP4_SCALE_SEARCH, "search rows"), (F.NVFP4_FOUR_OVER_SIX | F.NVFP4_TS_FOR_FOUR, "4/6 ts/1792"),
]


@pytest.mark.parametrize("flags,what", CASES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_grouped_quantize_matches_oracle_per_group(oracle, flags, what, dtype):
    G, rows, cols = 5, 272, 400  # several column tiles and pass-2 chunks, ragged against every tile size
    print(f"[grouped quantize] {what} {dtype} G={G} [{rows}x{cols}]", flush=True)
    x = _groups_input(G, rows, cols, dtype, seed=21)
    xd = x.cuda()
    q = nv.nvfp4_quantize_grouped(xd, flags=flags, seed=99, stream_id=3)
    torch.cuda.synchronize()
    for g in range(G):
        ref = oracle.quantize(oracle_input(x[g]), flags=flags, seed=99, stream_id=3 + g)
        assert_quant_equal(_group(q, g), ref, f"{what} group {g}")
        single = nv.nvfp4_quantize(xd[g], flags=flags, seed=99, stream_id=3 + g)
        assert torch.equal(single.data, _group(q, g).data) and torch.equal(single.scales, _group(q, g).scales)


def test_grouped_quantize_strided_groups(oracle):
    # each group a [rows x cols] window of a larger [rows+8 x cols+32] slab: ldx > cols and a group
    # stride beyond rows * ldx
    G, rows, cols = 3, 64, 96
    x = _groups_input(G, rows, cols, torch.bfloat16, seed=22, pad_rows=8, pad_cols=32)
    xd = x.cuda()[:, 4:4 + rows, 16:16 + cols]
    for flags in (0, nv.NVFP4_COLWISE | nv.NVFP4_FOUR_OVER_SIX, nv.NVFP4_BLOCK2D):
        q = nv.nvfp4_quantize_grouped(xd, flags=flags)
        torch.cuda.synchronize()
        for g in range(G):
            ref = oracle.quantize(oracle_input(x[g, 4:4 + rows, 16:16 + cols].contiguous()), flags=flags)
            assert_quant_equal(_group(q, g), ref, f"strided flags={flags} group {g}")


def test_grouped_quantize_one_group_and_empty():
    x = synth.normal((1, 48, 64), 1.0, seed=23, tensor_id=310).cuda()
    q = nv.nvfp4_quantize_grouped(x)
    single = nv.nvfp4_quantize(x[0])
    assert torch.equal(q.data, single.data) and torch.equal(q.scales, single.scales)
    assert torch.equal(q.tensor_scale, single.tensor_scale)
    # zero rows: every group's tensor scale is written as 0
    e = torch.empty((4, 0, 64), dtype=torch.bfloat16, device="cuda")
    out = nv.empty_like_quantized(0, 64, 0, "cuda", groups=4)
    out.tensor_scale.fill_(5.0)
    nv.nvfp4_quantize_grouped(e, out=out)
    assert torch.all(out.tensor_scale.cpu() == 0)


def test_grouped_quantize_moe_experts_feed_grouped_gemm(oracle):
    # 64 experts [4096 x 1536] column-wise with Four-over-Six, as the MoE expert layer quantizes them:
    # equal to 64 separate calls; two experts against the oracle in full
    E, K, N = 64, 4096, 1536
    experts = synth.moe_experts(0, E, K, N, workers=16)
    w = torch.stack(experts).cuda()
    fl = nv.NVFP4_COLWISE | nv.NVFP4_FOUR_OVER_SIX
    print("[grouped quantize] 64 MoE experts", flush=True)
    q = nv.nvfp4_quantize_grouped(w, flags=fl)
    for e in range(E):
        single = nv.nvfp4_quantize(w[e], flags=fl)
        g = _group(q, e)
        assert torch.equal(single.data, g.data) and torch.equal(single.scales, g.scales), e
        assert torch.equal(single.tensor_scale, g.tensor_scale), e
    for e in (0, 37):
        assert_quant_equal(_group(q, e), oracle.quantize(oracle_input(experts[e]), flags=fl), f"expert {e}")
