"""The library's calls launch kernels only (no memsets, arguments by value), so a quantize +
quantize + GEMM step can be captured in a HIP graph.  Every replay, with unrelated eager work and
cleared outputs in between, must reproduce the eager results bit for bit."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_bit_block_quantize_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.lib()


@pytest.mark.parametrize("rht", [False, True])
def test_graph_replays_match_eager(rht):
    dev = torch.device("cuda")
    x = synth.normal((512, 1024), 1.0, seed=1, tensor_id=70).to(dev)
    w = synth.normal((384, 1024), 0.02, seed=1, tensor_id=71).to(dev)
    fa = nv.NVFP4_COLWISE | nv.NVFP4_SR if rht else 0
    fb = nv.NVFP4_COLWISE if rht else nv.NVFP4_BLOCK2D
    Ra, Ka = (x.shape[1], x.shape[0]) if rht else tuple(x.shape)
    Rb, Kb = (w.shape[1], w.shape[0]) if rht else tuple(w.shape)
    if rht:  # wgrad-like: transform both operands along the shared dimension
        w = synth.normal((512, 384), 0.02, seed=1, tensor_id=72).to(dev)
        Rb, Kb = w.shape[1], w.shape[0]
    qa = nv.empty_like_quantized(Ra, Ka, fa, dev)
    qb = nv.empty_like_quantized(Rb, Kb, fb, dev)
    wsa = torch.empty(nv.nvfp4_workspace_size(*x.shape, fa) // 4, dtype=torch.int32, device=dev)
    wsb = torch.empty(nv.nvfp4_workspace_size(*w.shape, fb) // 4, dtype=torch.int32, device=dev)
    y = torch.empty((Ra, Rb), dtype=torch.float32, device=dev)

    def step():
        if rht:
            nv.nvfp4_rht_quantize(x, 7, flags=fa, seed=7, out=qa, workspace=wsa)
            nv.nvfp4_rht_quantize(w, 7, flags=fb, out=qb, workspace=wsb)
        else:
            nv.nvfp4_quantize(x, flags=fa, out=qa, workspace=wsa)
            nv.nvfp4_quantize(w, flags=fb, out=qb, workspace=wsb)
        nv.nvfp4_gemm(qa, qb, out=y)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (qa.data, qa.scales, qa.tensor_scale, qb.data, qb.scales, qb.tensor_scale, y)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = synth.normal((256, 256), 1.0, seed=2, tensor_id=73).to(dev)
    for r in range(4):
        for t in (qa.data, qa.scales, qa.tensor_scale, qb.data, qb.scales, qb.tensor_scale, y):
            t.zero_()
        nv.nvfp4_quantize(other)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (qa.data, qa.scales, qa.tensor_scale, qb.data, qb.scales, qb.tensor_scale, y)
        for a_, b_ in zip(got, ref):
            assert torch.equal(a_, b_), f"replay {r} differs from the eager result"
