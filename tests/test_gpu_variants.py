"""Four-over-Six variants on the GPU against the oracle (bit-exact codes, scale bytes and tensor
scale): the tensor scale amax/1792, the five-target scale search, and Four-over-Six on 16x16
tiles (row-wise and column-wise), with ragged shapes and the transform; plus the block-error
report of each variant on Student-t expert weights of the MoE workload."""
import numpy as np
import pytest
import torch

import nvfp4_bit_block_quantize_amd as nv
import synth
from tests.gpu_util import assert_quant_equal, oracle_input

pytestmark = pytest.mark.gpu
F46, TS4, SRCH = nv.NVFP4_FOUR_OVER_SIX, nv.NVFP4_TS_FOR_FOUR, nv.NVFP4_SCALE_SEARCH
COL, B2 = nv.NVFP4_COLWISE, nv.NVFP4_BLOCK2D

CASES = [
    ("row_ts4", (96, 528), TS4),
    ("row_ts4_sr", (96, 528), TS4 | nv.NVFP4_SR),
    ("row_4over6_ts4", (300, 1040), F46 | TS4),
    ("row_search", (300, 1040), SRCH),
    ("row_search_ts4", (64, 4096), SRCH | TS4),
    ("col_search", (528, 392), COL | SRCH),
    ("row2d_ts4", (272, 1040), B2 | TS4),
    ("row2d_4over6", (272, 1040), B2 | F46),
    ("row2d_4over6_wide", (48, 4112), B2 | F46),
    ("row2d_4over6_ts4", (272, 1040), B2 | F46 | TS4),
    ("col2d_4over6", (528, 400), COL | B2 | F46),
    ("col2d_4over6_ragged", (1040, 272), COL | B2 | F46),
]


@pytest.mark.parametrize("name,shape,flags", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_variant_matches_oracle(oracle, name, shape, flags, dtype):
    x = synth.student_t(shape, 4, 0.02, seed=8, tensor_id=80, dtype=dtype)
    q = nv.nvfp4_quantize(x.cuda(), flags=flags, seed=5, stream_id=1)
    torch.cuda.synchronize()
    ref = oracle.quantize(oracle_input(x), flags=flags, seed=5, stream_id=1)
    assert_quant_equal(q, ref, f"{name} {dtype}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("flags", [SRCH, F46 | TS4, SRCH | TS4, COL | SRCH])
def test_variant_with_transform(oracle, flags, dtype):
    x = synth.normal((128, 1024), 1.0, seed=9, tensor_id=81, dtype=dtype)
    q = nv.nvfp4_rht_quantize(x.cuda(), 7, flags=flags)
    torch.cuda.synchronize()
    ref = oracle.quantize(oracle_input(x), flags=flags, rht=True, sign_seed=7)
    # the transform adds in the same order on both sides here (same butterfly): codes agree exactly
    assert_quant_equal(q, ref, f"RHT flags {flags}")


def test_c4_expert_block_error_report(oracle):
    """Block squared error of each variant relative to plain max-to-6 scaling, summed over 8 of
    the 64 Student-t(4) x 0.02 experts [4096 x 1536] (quantized column-wise, blocks along 4096);
    the GPU codes are checked bit-exactly against the oracle, whose per-block errors are summed."""
    experts = synth.moe_experts(0, n_experts=8, workers=8)
    variants = [("4/6", F46), ("4/6, ts=amax/1792", F46 | TS4), ("search {6..4}", SRCH),
                ("search, ts=amax/1792", SRCH | TS4), ("2D 4/6 (vs plain 2D)", B2 | F46)]
    tot = {name: [0.0, 0.0] for name, _ in variants}
    for w in experts:
        xw = oracle_input(w)
        for name, fl in variants:
            flags = COL | fl
            q = nv.nvfp4_quantize(w.cuda(), flags=flags)
            ref = oracle.quantize(xw, flags=flags)
            assert_quant_equal(q, ref, f"expert {name}")
            tot[name][0] += ref["sse"][0]
            tot[name][1] += ref["sse"][1]
    lines = []
    for name, _ in variants:
        chosen, plain = tot[name]
        assert chosen <= plain
        lines.append(f"{name}: {100 * (1 - chosen / plain):.2f}% lower block error than plain")
    print("\n" + "\n".join(lines))
    # the search can only improve on Four-over-Six (same tensor scale, superset of targets)
    assert tot["search {6..4}"][0] <= tot["4/6"][0]
    assert tot["search, ts=amax/1792"][0] <= tot["4/6, ts=amax/1792"][0]


def test_four_over_six_2d_transpose_on_near_ties(oracle):
    """Row-wise and column-wise 16x16-tile Four-over-Six on tiles built at the crossing of the two
    candidates' errors (tests/near_tie.py), bit-exact against the oracle; nvfp4_transpose of the
    row-wise result equals the column-wise quantization (quantize(W^T) == quantize(W)^T)."""
    from tests.near_tie import near_tie_tensor
    x = torch.from_numpy(near_tie_tensor(oracle, 8, 12, seed=5))  # fp32 [128 x 192]: bf16 would round the ties away
    xd = x.cuda()
    q = nv.nvfp4_quantize(xd, flags=B2 | F46)
    qc = nv.nvfp4_quantize(xd, flags=COL | B2 | F46)
    qt = nv.nvfp4_transpose(q)
    torch.cuda.synchronize()
    assert_quant_equal(q, oracle.quantize(x.numpy(), flags=B2 | F46), "row2d 4/6 near ties")
    assert_quant_equal(qc, oracle.quantize(x.numpy(), flags=COL | B2 | F46), "col2d 4/6 near ties")
    assert torch.equal(qt.data.cpu(), qc.data.cpu())
    assert torch.equal(qt.scales.cpu(), qc.scales.cpu())
    assert torch.equal(qt.tensor_scale.cpu(), qc.tensor_scale.cpu())
