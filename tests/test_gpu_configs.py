"""Parity at the full sizes of the MoE and 405B-shaped workloads (GPU against the oracle).

MoE (64 experts [4096 x 1536] Student-t(4) x 0.02, 16384 tokens ~N(0,1) routed top-2 with
Zipf(1.1) expert loads): experts quantized column-wise with Four-over-Six, the routed tokens
row-wise, then the grouped GEMM; every group's first and last 128-row tile (a seeded 128-column
window) is checked against the oracle's double-precision product of the GPU's own operands.

405B-shaped FFN forward (X [8192 x 16384] ~N(0,1) with 0.1% outlier channels x20, W [53248 x
16384] ~N(0,0.01) with 16x16 scaling): both quantizations checked bit-exactly in full, and 64
seeded 128 x 128 tiles of Y = X W^T (bf16 out) against the oracle; then the W4A16 GEMM of 16 and
40 tokens against the same weight (2D and 1D scales), 48 seeded column windows each.
"""
import os

import numpy as np
import pytest
import torch

import nvfp4_bit_block_quantize_amd as nv
import synth
from tests.gpu_util import assert_quant_equal, gemm_check, oracle_input, seeded_tiles

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

WORKERS = min(16, os.cpu_count() or 1)


def _host_rows(q, r0, r1, block2d=False):
    """Host copy of rows [r0, r1) of a quantized tensor (r0, r1 multiples of 16 for 2D scales)."""
    sc = q.scales[r0 // 16:(r1 + 15) // 16] if block2d else q.scales[r0:r1]
    return {"data": q.data[r0:r1].cpu().numpy(), "scales": sc.cpu().numpy(),
            "ts": q.tensor_scale.cpu().numpy()[0], "flags": nv.NVFP4_BLOCK2D if block2d else 0}


def test_moe_grouped_gemm_full(oracle):
    E, K, N, T = 64, 4096, 1536, 16384
    print("[moe] generating experts and tokens", flush=True)
    experts = synth.moe_experts(0, E, K, N, workers=WORKERS)
    tokens = synth.moe_tokens(0, T, K).cuda()
    loads, slot_token = synth.moe_routing(T, E, 2, 1.1, 0)
    offs = np.concatenate([[0], np.cumsum(loads)]).tolist()
    assert offs[-1] == 2 * T and loads.min() >= 1

    # experts: W_e [K x N] quantized along K (COLWISE) with Four-over-Six into one group-contiguous B
    dev = tokens.device
    qb = nv.NVFP4Tensor(torch.empty((E * N, K // 2), dtype=torch.uint8, device=dev),
                        torch.empty((E * N, K // 16), dtype=torch.uint8, device=dev),
                        torch.empty(E, dtype=torch.float32, device=dev), N, K,
                        nv.NVFP4_COLWISE | nv.NVFP4_FOUR_OVER_SIX, E)
    fl = nv.NVFP4_COLWISE | nv.NVFP4_FOUR_OVER_SIX
    for e in range(E):
        view = nv.NVFP4Tensor(qb.data[e * N:(e + 1) * N], qb.scales[e * N:(e + 1) * N],
                              qb.tensor_scale[e:e + 1], N, K, fl)
        nv.nvfp4_quantize(experts[e].cuda(), flags=fl, out=view)
    # quantize parity of the lightest and the heaviest expert (full tensors)
    for e in (int(np.argmin(loads)), int(np.argmax(loads))):
        ref = oracle.quantize(oracle_input(experts[e]), flags=fl)
        view = nv.NVFP4Tensor(qb.data[e * N:(e + 1) * N], qb.scales[e * N:(e + 1) * N],
                              qb.tensor_scale[e:e + 1], N, K, fl)
        assert_quant_equal(view, ref, f"expert {e} (load {loads[e]}) 4/6")
        chosen, plain = ref["sse"]
        assert chosen <= plain
        print(f"[moe] expert {e}: 4/6 block-MSE reduction {100 * (1 - chosen / plain):.2f}%", flush=True)

    # routed activations: rows grouped by expert, one tensor scale for all tokens
    xg = tokens[torch.from_numpy(slot_token).to(dev)]
    qa = nv.nvfp4_quantize(xg)
    c = nv.nvfp4_gemm(qa, qb, out_dtype=torch.float32, group_offsets=offs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    worst = 0.0
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        starts = sorted({0, max(0, (r1 - r0 - 1) // 128 * 128)})
        c0 = int(rng.integers(0, N // 128)) * 128
        a_e = _host_rows(qa, r0, r1)
        b_e = _host_rows(qb, e * N, (e + 1) * N)
        b_e["ts"] = qb.tensor_scale[e].item()
        tiles = [(s, c0, min(128, r1 - r0 - s), 128) for s in starts]
        cref, bnd = oracle.gemm_ref(a_e, b_e, r1 - r0, N, K, tiles=tiles)
        got = c[r0:r1].cpu().numpy()
        worst = max(worst, gemm_check(got, cref, bnd, False, f"expert {e} rows {r0}:{r1}"))
    print(f"[moe] grouped GEMM: 64 groups x first/last tiles, max |err|/bound {worst:.2e}", flush=True)


def test_fprop405b_quantize_full_and_gemm_tiles(oracle):
    print("[405b] generating X [8192 x 16384], W [53248 x 16384]", flush=True)
    x, w = synth.fprop405b(0)
    qx = nv.nvfp4_quantize(x.cuda())
    qw = nv.nvfp4_quantize(w.cuda(), flags=nv.NVFP4_BLOCK2D)
    y = nv.nvfp4_gemm(qx, qw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    print("[405b] oracle quantize X", flush=True)
    assert_quant_equal(qx, oracle.quantize(oracle_input(x)), "405B X 1D")
    print("[405b] oracle quantize W", flush=True)
    assert_quant_equal(qw, oracle.quantize(oracle_input(w), flags=nv.NVFP4_BLOCK2D), "405B W 2D")
    x_dec = x[:40].clone()  # decode-sized activation batches for the W4A16 checks below
    del x
    M, N, K = qx.rows, qw.rows, qx.k
    worst = 0.0
    for (r0, c0, h, wd) in seeded_tiles(M, N, 64, seed=5):
        a_t = _host_rows(qx, r0, r0 + h)
        b_t = _host_rows(qw, c0, c0 + wd, block2d=True)
        cref, bnd = oracle.gemm_ref(a_t, b_t, h, wd, K)
        got = y[r0:r0 + h, c0:c0 + wd].float().cpu().numpy()
        worst = max(worst, gemm_check(got, cref, bnd, True, f"405B tile ({r0},{c0})"))
    print(f"[405b] 64 tiles of 8192x53248x16384: max |err|/bound {worst:.2e}", flush=True)

    # W4A16 at the same weight size: 16 tokens against the 2D-quantized W (weight streaming, one
    # M tile), 40 tokens against W quantized with 1D blocks (three M tiles); 48 seeded windows of
    # 128 output columns each against the oracle
    windows = [(0, c0, 1, 128) for (_, c0, _, _) in seeded_tiles(1, N, 48, seed=6)]
    for rows, flags in ((16, nv.NVFP4_BLOCK2D), (40, 0)):
        qw_w = qw if flags else nv.nvfp4_quantize(w.cuda())
        a16 = x_dec[:rows].to(torch.bfloat16)
        yw = nv.nvfp4_gemm_w4a16(a16.cuda(), qw_w, out_dtype=torch.float32)
        torch.cuda.synchronize()
        a_bits = synth.bf16_bits(a16)
        worst = 0.0
        for (_, c0, _, wd) in windows:
            b_t = _host_rows(qw_w, c0, c0 + wd, block2d=bool(flags))
            cref, bnd = oracle.gemm_w4a16_ref(a_bits, b_t, rows, wd, K)
            worst = max(worst, gemm_check(yw[:, c0:c0 + wd].cpu().numpy(), cref, bnd, False,
                                          f"405B W4A16 {rows} rows flags={flags} cols {c0}"))
        print(f"[405b] W4A16 {rows}x53248x16384 (flags {flags}), 48 windows: max |err|/bound {worst:.2e}", flush=True)
        del qw_w
