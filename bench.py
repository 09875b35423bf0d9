#!/usr/bin/env python3
"""Benchmark of the NVFP4 quantize-and-multiply path on one MI355X.

Default workload (the Llama-3-8B FFN forward shape): X [8192 x 4096] bf16 ~N(0,1) with 0.1% outlier
channels x20, W [14336 x 4096] bf16 ~N(0,0.02).  One step = nvfp4_quantize(X) (1D blocks) +
nvfp4_quantize(W) (16x16 tiles) + nvfp4_gemm(X_q, W_q) -> Y [8192 x 14336] bf16, FP32 accumulate.
Inputs are generated once and resident in HBM before the timed region.

Prints one JSON line.  `value` is the whole step's throughput in TFLOP/s (2*M*N*K per step / step
time, the step replayed as one HIP graph); the components object carries the quantize GB/s (algorithmic bytes: both passes' reads plus
the codes and scales written) and the GEMM-only TFLOP/s; `roofline` describes the dominant kernel
(the GEMM) against the MI355X dense fp16 MFMA peak; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME] [--no-cpu]

Other workloads (--workload): fprop8b_q (the GEMM output quantized in the epilogue), dgrad8b,
wgrad8b (RHT + stochastic rounding), w4a16_8b and w4a16_decode (bf16 activations x NVFP4 weights),
fprop405b (the Llama-3.1-405B FFN forward, 8192x53248x16384), moe (64 experts [4096x1536],
Zipf(1.1) top-2 loads over 16384 tokens, grouped GEMM) and dequant8b (NVFP4 -> bf16 / fp32 decode of
the fprop weight and activations, HBM GB/s).  The CPU oracle baseline is timed on the
default workload only.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
METRIC = "NVFP4 quantize HBM GB/s + NVFP4 GEMM TFLOP/s (8192x14336x4096)"


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="fprop8b",
                   choices=["fprop8b", "fprop8b_q", "wgrad8b", "dgrad8b", "w4a16_8b", "w4a16_decode",
                            "fprop405b", "moe", "dequant8b", "gemm_designs"])
    p.add_argument("--decode-tokens", type=int, default=16, help="rows of X in the w4a16_decode workload")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-rows", type=int, default=8192, help="rows of X and W in the CPU sample (about 10 s on 16 cores)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run 5 device-to-device copies of MIB MiB (a known-size kernel for scaling "
                        "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    p.add_argument("--traffic-summary", metavar="DIR", default=None,
                   help="no GPU: read the rocprofv3 counter CSVs under DIR (pmc_FETCH_SIZE, pmc_WRITE_SIZE "
                        "of a bench run; cpy_FETCH_SIZE, cpy_WRITE_SIZE of --copy-calibration 1024), write "
                        "profiles/gemm_fprop8b_traffic.json and exit")
    return p.parse_args()


def quant_bytes(rows, cols, block2d):
    """Algorithmic HBM bytes of one quantize of a bf16 tensor: two reads (amax pass, encode pass),
    the packed codes and the scale bytes."""
    n = rows * cols
    return n * 2 + n * 2 + n // 2 + (n // 256 if block2d else n // 16)


def gemm_source_digest():
    """sha256 over the GEMM kernel sources (the counters below are only valid for this source)."""
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "gemm_kernels.hpp", "gemm_variant.hip", "gemm_common.hpp", "nvfp4_device.hpp"):
        with open(os.path.join(ROOT, "nvfp4_bit_block_quantize_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_gemm_counters():
    """The committed rocprofv3 counter summary of the GEMM (profiles/gemm_fprop8b_traffic.json: HBM
    bytes per launch from FETCH_SIZE / WRITE_SIZE scaled by the copy-kernel calibration, MFMA busy
    fraction and shader clock); None when it is missing or was taken on other sources."""
    path = os.path.join(ROOT, "profiles", "gemm_fprop8b_traffic.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256") != gemm_source_digest():
        return None
    return t


def _counter_per_dispatch(csv_path, name_part, counter):
    """Mean over the dispatches of kernels whose name contains name_part of the counter's value
    summed over all its instances (KiB for FETCH_SIZE / WRITE_SIZE)."""
    import csv
    per = {}
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for '{name_part}' in {csv_path}")
    return sum(per.values()) / len(per), len(per)


def _mfma_per_dispatch(csv_path, name_part):
    """Per dispatch of kernels whose name contains name_part: MFMA busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs), shader clock
    (GRBM_GUI_ACTIVE / 8 over the dispatch's duration) and VALU instructions per MFMA."""
    import csv
    per, span = {}, {}
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            if name_part not in r["Kernel_Name"]:
                continue
            d = per.setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            span[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = []
    for k, c in per.items():
        g = c["GRBM_GUI_ACTIVE"] / 8
        out.append((c["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * 1024), g / span[k], c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"] - 1))
    if not out:
        raise SystemExit(f"no counter rows for '{name_part}' in {csv_path}")
    return out


def traffic_summary(d):
    copy_kib = 1024 * 1024  # --copy-calibration 1024: 1 GiB read and 1 GiB written per launch
    cf, _ = _counter_per_dispatch(os.path.join(d, "cpy_FETCH_SIZE", "p_counter_collection.csv"), "copyBuffer", "FETCH_SIZE")
    cw, _ = _counter_per_dispatch(os.path.join(d, "cpy_WRITE_SIZE", "p_counter_collection.csv"), "copyBuffer", "WRITE_SIZE")
    gf, nf = _counter_per_dispatch(os.path.join(d, "pmc_FETCH_SIZE", "p_counter_collection.csv"), "gemm", "FETCH_SIZE")
    gw, nw = _counter_per_dispatch(os.path.join(d, "pmc_WRITE_SIZE", "p_counter_collection.csv"), "gemm", "WRITE_SIZE")
    fs, ws = copy_kib / cf, copy_kib / cw
    # MFMA pass: the dispatches after the first few (clocks settle over the warm-up)
    mf = _mfma_per_dispatch(os.path.join(d, "pmc_MFMA", "p_counter_collection.csv"), "gemm")
    mf = mf[len(mf) // 2:]
    M, N, K = 8192, 14336, 4096
    cmd = "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} --output-format csv -d $OUT/{d} -o p -- python3 $REPO/bench.py {a}"
    out = {
        "what": "HBM-side traffic per launch of the NVFP4 GEMM (fprop 8192x14336x4096, bf16 out), from rocprofv3 "
                "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over the dispatches), each scaled by the "
                "same counter's reading for a device-to-device copy of 1024 MiB; and the MFMA busy fraction "
                "(SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs)) at the shader clock "
                "(GRBM_GUI_ACTIVE / 8 over the dispatch's duration), over the later half of the dispatches",
        "commands": [cmd.format(c="FETCH_SIZE", d="pmc_FETCH_SIZE", a="--steps 2 --warmup 1 --no-cpu"),
                     cmd.format(c="WRITE_SIZE", d="pmc_WRITE_SIZE", a="--steps 2 --warmup 1 --no-cpu"),
                     cmd.format(c="FETCH_SIZE", d="cpy_FETCH_SIZE", a="--copy-calibration 1024"),
                     cmd.format(c="WRITE_SIZE", d="cpy_WRITE_SIZE", a="--copy-calibration 1024"),
                     cmd.format(c="SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU GRBM_GUI_ACTIVE", d="pmc_MFMA",
                                a="--steps 10 --warmup 5 --no-cpu"),
                     "python3 bench.py --traffic-summary $OUT"],
        "mfma_busy_frac": round(sum(x[0] for x in mf) / len(mf), 4),
        "sclk_ghz": round(sum(x[1] for x in mf) / len(mf), 3),
        "valu_per_mfma": round(sum(x[2] for x in mf) / len(mf), 3),
        "mfma_dispatches": len(mf),
        "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1), "copy_true_kib_each_way": copy_kib,
        "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
        "gemm_dispatches": [nf, nw],
        "gemm_fetch_kib_per_launch": round(gf, 1), "gemm_write_kib_per_launch": round(gw, 1),
        "traffic_bytes_per_launch": int(round((gf * fs + gw * ws) * 1024)),
        "algorithmic_operand_bytes": M * K // 2 + N * K // 2 + M * K // 16 + N * K // 256,
        "output_bytes": M * N * 2,
        "gemm_source_sha256": gemm_source_digest(),
    }
    path = os.path.join(ROOT, "profiles", "gemm_fprop8b_traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def main():
    a = _args()
    if a.traffic_summary:
        traffic_summary(a.traffic_summary)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        sys.exit(2)
    import torch
    import nvfp4_bit_block_quantize_amd as nv
    import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    nv.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.copy_calibration:
        n = a.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}))
        return

    if a.workload == "moe":
        run_moe(a, nv, torch, synth, dev)
        return
    if a.workload == "dequant8b":
        run_dequant(a, nv, torch, synth, dev)
        return
    if a.workload == "gemm_designs":
        run_gemm_designs(a, torch, dev)
        return
    if a.workload in ("fprop8b", "fprop8b_q"):
        x_cpu, w_cpu = synth.fprop8b(0)
        M, K = x_cpu.shape
        N = w_cpu.shape[0]
        fa, fb, rht = 0, nv.NVFP4_BLOCK2D, False
        out_dtype = torch.bfloat16
        workload = "Llama-3-8B FFN fprop: X[8192x4096] bf16 1D blocks, W[14336x4096] bf16 16x16 tiles, Y bf16"
        if a.workload == "fprop8b_q":
            workload = ("Llama-3-8B FFN fprop: X[8192x4096] bf16 1D blocks, W[14336x4096] bf16 16x16 tiles, "
                        "Y quantized to NVFP4 (1D) in the GEMM epilogue, tensor scale from the previous step's amax")
        qbytes = quant_bytes(M, K, False) + quant_bytes(N, K, True)
    elif a.workload == "fprop405b":
        x_cpu, w_cpu = synth.fprop405b(0)
        M, K = x_cpu.shape
        N = w_cpu.shape[0]
        fa, fb, rht = 0, nv.NVFP4_BLOCK2D, False
        out_dtype = torch.bfloat16
        workload = "Llama-3.1-405B FFN fprop: X[8192x16384] bf16 1D blocks, W[53248x16384] bf16 16x16 tiles, Y bf16"
        qbytes = quant_bytes(M, K, False) + quant_bytes(N, K, True)
    elif a.workload == "dgrad8b":
        dy_cpu, _ = synth.wgrad8b(0)
        _, w_cpu = synth.fprop8b(0)
        x_cpu = dy_cpu  # A = dY (rows, K = 14336, stochastic rounding); B = transpose of Q2D(W)
        M, K = x_cpu.shape
        N = w_cpu.shape[1]
        fa, fb, rht = nv.NVFP4_SR, nv.NVFP4_BLOCK2D, False
        out_dtype = torch.bfloat16
        workload = "Llama-3-8B FFN dgrad: dY[8192x14336] SR rows, W[14336x4096] 16x16 tiles transposed, dX bf16"
        # the B side of a step moves the 2D-quantized W through nvfp4_transpose (codes + scales, both ways)
        qbytes = quant_bytes(M, K, False) + 2 * (N * K // 2 + N * K // 256)
    elif a.workload in ("w4a16_8b", "w4a16_decode"):
        # weight-only 4-bit: bf16 activations against the 16x16-tile NVFP4 weight, which a serving
        # stack quantizes once (outside the step); the step is the GEMM alone
        x_cpu, w_cpu = synth.fprop8b(0)
        if a.workload == "w4a16_decode":
            x_cpu = x_cpu[:a.decode_tokens].contiguous()
        M, K = x_cpu.shape
        N = w_cpu.shape[0]
        fa, fb, rht = 0, nv.NVFP4_BLOCK2D, False
        out_dtype = torch.bfloat16
        workload = (f"Llama-3-8B FFN fprop, W4A16: X[{M}x4096] bf16 (not quantized), W[14336x4096] NVFP4 "
                    "16x16 tiles (quantized once, outside the step), Y bf16")
        qbytes = 0
    else:
        dy_cpu, xx_cpu = synth.wgrad8b(0)
        x_cpu, w_cpu = dy_cpu, xx_cpu  # A = dY^T, B = X^T
        K, M = x_cpu.shape
        N = w_cpu.shape[1]
        fa, fb, rht = nv.NVFP4_COLWISE | nv.NVFP4_SR, nv.NVFP4_COLWISE, True
        out_dtype = torch.float32
        workload = "Llama-3-8B FFN wgrad: RHT(dY)[8192x14336] SR, RHT(X)[8192x4096], dW fp32"
        qbytes = quant_bytes(K, M, False) + quant_bytes(K, N, False)
    x = x_cpu.to(dev)
    w = w_cpu.to(dev)
    del x_cpu, w_cpu
    R_a, K_a = (x.shape[1], x.shape[0]) if fa & nv.NVFP4_COLWISE else tuple(x.shape)
    R_b, K_b = (w.shape[1], w.shape[0]) if fb & nv.NVFP4_COLWISE else tuple(w.shape)
    qa = nv.empty_like_quantized(R_a, K_a, fa, dev)
    qb = nv.empty_like_quantized(R_b, K_b, fb, dev)
    qw_fwd = None
    if a.workload == "dgrad8b":
        # the forward pass's 2D quantization of W (not part of the dgrad step); the step's B operand
        # is its transpose [4096 x 14336]
        qw_fwd = nv.nvfp4_quantize(w, flags=nv.NVFP4_BLOCK2D)
        qb = nv.empty_like_quantized(w.shape[1], w.shape[0], nv.NVFP4_BLOCK2D, dev)
    ws_a = torch.empty(nv.nvfp4_workspace_size(*x.shape, fa) // 4, dtype=torch.int32, device=dev)
    ws_b = torch.empty(nv.nvfp4_workspace_size(*w.shape, fb) // 4, dtype=torch.int32, device=dev)
    y = torch.empty((M, N), dtype=out_dtype, device=dev)

    w4a16 = a.workload.startswith("w4a16")
    fused = a.workload == "fprop8b_q"
    if fused:
        y_q = nv.empty_like_quantized(M, N, 0, dev)
        amax = torch.zeros(1, dtype=torch.float32, device=dev)
    if w4a16:
        qb = nv.nvfp4_quantize(w, flags=fb, workspace=ws_b)

    def q_a(src=None):
        if w4a16:
            return
        src = x if src is None else src
        if rht:
            nv.nvfp4_rht_quantize(src, 7, flags=fa, seed=7, out=qa, workspace=ws_a)
        else:
            nv.nvfp4_quantize(src, flags=fa, seed=7, out=qa, workspace=ws_a)

    def q_b(src=None):
        if w4a16:
            return
        if qw_fwd is not None:
            nv.nvfp4_transpose(qw_fwd if src is None else src, out=qb)
        elif rht:
            nv.nvfp4_rht_quantize(w if src is None else src, 7, flags=fb, out=qb, workspace=ws_b)
        else:
            nv.nvfp4_quantize(w if src is None else src, flags=fb, out=qb, workspace=ws_b)

    def mm():
        if fused:
            nv.nvfp4_gemm_nvfp4_out(qa, qb, y_q, amax=amax)
        elif w4a16:
            nv.nvfp4_gemm_w4a16(x, qb, out=y)
        else:
            nv.nvfp4_gemm(qa, qb, out=y)

    def step():
        q_a(); q_b()
        if fused:
            # delayed scaling: this step's tensor scale from the previous step's amax
            nv.nvfp4_scale_from_amax(amax, y_q.tensor_scale)
            amax.zero_()
        mm()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    # per-call times of each library call: `steps` back-to-back launches on the launch stream
    # bracketed by two events (the library launches on torch's current stream); a GEMM queued first
    # keeps the GPU busy while the host enqueues them, so host launch overhead is not timed
    def per_call_ms(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        mm()  # ~0.7 ms of queued GPU work, so that the launches below are enqueued ahead of the GPU
        e0.record()
        for _ in range(a.steps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / a.steps

    unfused_ms = None
    if fused:
        # the same output the unfused way: bf16 Y, then its two-pass quantization
        ws_y = torch.empty(nv.nvfp4_workspace_size(M, N, 0) // 4, dtype=torch.int32, device=dev)
        y_q2 = nv.empty_like_quantized(M, N, 0, dev)

        def unfused():
            nv.nvfp4_gemm(qa, qb, out=y)
            nv.nvfp4_quantize(y, out=y_q2, workspace=ws_y)
        unfused_ms = per_call_ms(unfused)
    qa_ms = per_call_ms(q_a) if not w4a16 else 0.0
    qb_ms = per_call_ms(q_b) if not w4a16 else 0.0

    # the same calls with the input out of the caches: back-to-back calls re-read a tensor that fits
    # the 256 MB Infinity Cache from there; here 1 GiB is read before each call (a read, so no dirty
    # lines are written back inside the timed call) and each call is timed alone between two events
    def cold_ms(fn, reps=5):
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        total = 0.0
        for _ in range(reps):
            flush.max()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            total += e0.elapsed_time(e1)
        del flush
        return total / reps
    qa_cold = cold_ms(q_a) if qbytes else 0.0
    qb_cold = cold_ms(q_b) if qbytes else 0.0

    # The same calls streamed: back to back, each on its own copy of the input, with enough copies
    # (512 MiB or more in all) that every call reads an input last touched more than the Infinity
    # Cache's 256 MB ago, so each input comes from HBM.  A call timed alone after the flush above also
    # carries the ~6 us between the flush kernel's end and the call's first kernel (event and
    # dispatch; profiles/quantize_cold_fprop8b.md), which a call queued behind other work does not.
    def stream_cold_ms(fn, src):
        if torch.is_tensor(src):
            nbytes = src.numel() * src.element_size()
            copy = src.clone
        else:  # a quantized tensor (the dgrad step's transpose input)
            nbytes = src.data.numel() + src.scales.numel()
            copy = lambda: nv.NVFP4Tensor(src.data.clone(), src.scales.clone(), src.tensor_scale.clone(),
                                          src.rows, src.k, src.flags)
        ncopy = 1 if nbytes >= (512 << 20) else -(-(512 << 20) // nbytes) + 1
        copies = [copy() for _ in range(ncopy)]
        reps = max(a.steps, 2 * ncopy)
        for c in copies:
            fn(c)
        mm()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(copies[i % ncopy])
        e1.record()
        e1.synchronize()
        del copies
        return e0.elapsed_time(e1) / reps
    qa_stream = stream_cold_ms(q_a, x) if qbytes else 0.0
    qb_stream = stream_cold_ms(q_b, qw_fwd if qw_fwd is not None else w) if qbytes else 0.0

    # copy ceiling: a device-to-device copy of the bf16 X (read + write, the same buffer sizes as the
    # quantize inputs), back to back like the quantize calls
    copy_dst = torch.empty_like(x)
    copy_ms = per_call_ms(lambda: copy_dst.copy_(x))
    copy_gbps = 2 * x.numel() * x.element_size() / (copy_ms * 1e-3) / 1e9
    del copy_dst
    mm_ms = per_call_ms(mm)
    step()
    torch.cuda.synchronize()
    y_eager = y.clone() if not fused else torch.cat([y_q.data.view(-1), y_q.scales.view(-1)])

    # the step as one HIP graph (every library call is capturable: kernels only, no memsets)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm the side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    graph_ok = bool(torch.equal(y, y_eager)) if not fused else bool(
        torch.equal(torch.cat([y_q.data.view(-1), y_q.scales.view(-1)]), y_eager))
    if not graph_ok:
        print(json.dumps({"error": "graph replay differs from eager result"}))
        sys.exit(1)
    for _ in range(a.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_step = wall * 1e3 / a.steps
    flops = 2.0 * M * N * K
    gemm_tflops = flops / (mm_ms * 1e-3) / 1e12
    quant_gbps = qbytes / ((qa_ms + qb_ms) * 1e-3) / 1e9 if qbytes else 0.0
    # HBM bytes a W4A16 GEMM must move at least once: bf16 A, the weight's codes and scales, C
    w4_bytes = M * K * 2 + N * K // 2 + N * K // 256 + M * N * 2
    value = flops / (ms_step * 1e-3) / 1e12

    counters = measured_gemm_counters() if a.workload == "fprop8b" else None
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1 x e4m3) -> exact f16 operands, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": workload, "M": M, "N": N, "K": K, "out": str(out_dtype).replace("torch.", "")},
        "components": {
            "quantize_warm_gbps": round(quant_gbps, 1),
            # cold: every input read from HBM (calls back to back, each on an input copy last touched
            # more than the Infinity Cache's size ago), as a training step meets them
            "quantize_cold_gbps": round(qbytes / ((qa_stream + qb_stream) * 1e-3) / 1e9, 1) if qbytes else None,
            "quantize_hbm_frac": round(qbytes / ((qa_stream + qb_stream) * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4) if qbytes else None,
            # each call alone after a 1 GiB flush read, between two events (includes the gap before
            # the first kernel)
            "quantize_cold_single_call_gbps": round(qbytes / ((qa_cold + qb_cold) * 1e-3) / 1e9, 1) if qbytes else None,
            "copy_ceiling_gbps": round(copy_gbps, 1),
            "quantize_frac_of_copy": round(quant_gbps / copy_gbps, 4) if qbytes else None,
            "quantize_cold_a_ms": round(qa_stream, 4),
            "quantize_cold_b_ms": round(qb_stream, 4),
            "quantize_cold_single_call_a_ms": round(qa_cold, 4),
            "quantize_cold_single_call_b_ms": round(qb_cold, 4),
            "quantize_a_ms": round(qa_ms, 4),
            "quantize_b_ms": round(qb_ms, 4),
            "quantize_algorithmic_bytes": qbytes,
            "gemm_ms": round(mm_ms, 4),
            "gemm_tflops": round(gemm_tflops, 1),
            "step_timing": "HIP graph replay of quantize(A) + quantize(B) + GEMM; components: mean of back-to-back launches of each call",
        },
        "roofline": {
            "kernel": "nvfp4 gemm",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 1),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_F16_TFLOPS, 4),
            "traffic": counters.get("traffic_bytes_per_launch") if counters else None,
        },
    }
    if counters:
        # MFMA busy fraction and shader clock of the committed counter run of this source: the
        # peak at that clock is 2.5 PFLOP/s x sclk / 2.4 GHz
        sclk = counters["sclk_ghz"]
        result["roofline"].update({"mfma_busy": counters["mfma_busy_frac"], "sclk_ghz": sclk,
                                   "frac_at_sclk": round(gemm_tflops / (PEAK_F16_TFLOPS * sclk / 2.4), 4)})
    if fused:
        result["components"]["unfused_gemm_bf16_plus_quantize_ms"] = round(unfused_ms, 4)
        result["components"]["step_timing"] = ("HIP graph replay of quantize(A) + quantize(B) + tensor scale from "
                                               "the previous amax + GEMM with NVFP4 output")
    if w4a16:
        result["dtype"] = "bf16 x nvfp4 (e2m1 x e4m3) -> exact bf16 operands, f32 accumulate"
        result["components"] = {"gemm_ms": round(mm_ms, 4), "gemm_tflops": round(gemm_tflops, 1),
                                "gemm_min_hbm_bytes": w4_bytes,
                                "gemm_gbps": round(w4_bytes / (mm_ms * 1e-3) / 1e9, 1),
                                "step_timing": "HIP graph replay of the W4A16 GEMM; gemm_ms: mean of back-to-back launches"}
        result["roofline"]["kernel"] = "nvfp4 w4a16 gemm"
        if a.workload == "w4a16_decode":
            gbps = w4_bytes / (mm_ms * 1e-3) / 1e9
            result["roofline"].update({"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                                       "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4)})
    if not a.no_cpu and a.workload == "fprop8b":
        result["cpu_baseline"] = cpu_baseline(a, nv)
    print(json.dumps(result), flush=True)


def run_gemm_designs(a, torch, dev):
    """The GEMM design probe (libnvfp4_probe.so): the inner step of each way of putting the NVFP4
    block-scaled product on the matrix cores, timed on its own (operands in registers, no memory
    traffic) on every SIMD of the GPU: one wave computes a 128 x 128 tile over one 16-element block,
    repeated.  Design 0 (the library's): exact fp16 decode with the scale folded in +
    v_mfma_f32_32x32x16_f16.  Design 1: fp4 operands of v_mfma_scale_f32_32x32x64_f8f6f4 (the block
    zero-padded to 64 K) into a fresh accumulator, rescaled by S_a * S_b per output element.
    Also design 0's MFMAs alone (operands decoded once), which separates the decode's cost from the
    matrix cores' own rate.  Useful work: 2 * 128 * 128 * 16 flops per wave per repetition."""
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "nvfp4_bit_block_quantize_amd", "libnvfp4_probe.so"))
    P = ctypes.c_void_p
    L.nvfp4_probe_design.argtypes = [ctypes.c_int, P, P, P, P, P, ctypes.c_int, ctypes.c_int, P]
    g = torch.Generator(device="cpu").manual_seed(1)
    codes = [torch.randint(0, 256, (128, 8), dtype=torch.uint8, generator=g).to(dev) for _ in range(2)]
    scales = [torch.randint(0x30, 0x50, (128, 1), dtype=torch.uint8, generator=g).to(dev) for _ in range(2)]
    c = torch.zeros((128, 128), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in (codes[0], scales[0], codes[1], scales[1])]
    workgroups, reps = 1024, 2000  # 4 waves each: 4096 waves, 16 per CU
    out = {}
    # 0-2: 4 x 4 tiles per wave, 4 waves per workgroup; 3, 5: 2 x 4 tiles, 8 waves (two per SIMD);
    # 4: 2 x 4 tiles, 4 waves
    # 6: 4 x 4 tiles, one wave per SIMD, design 2 plus decode work the MFMAs do not read
    # 7: design 0 with the decode of the next block interleaved with the MFMAs of this one
    # 8: design 6 with conversions only (independent VALU instructions)
    waves = {0: 4, 1: 4, 2: 4, 3: 8, 4: 4, 5: 8, 6: 4, 7: 4, 8: 4}
    tile_flops = {0: 2 * 128 * 128 * 16, 1: 2 * 128 * 128 * 16, 2: 2 * 128 * 128 * 16,
                  3: 2 * 64 * 128 * 16, 4: 2 * 64 * 128 * 16, 5: 2 * 64 * 128 * 16, 6: 2 * 128 * 128 * 16,
                  7: 2 * 128 * 128 * 16, 8: 2 * 128 * 128 * 16}
    for design in (0, 1, 2, 3, 4, 5, 6, 7, 8):
        for _ in range(a.warmup):
            L.nvfp4_probe_design(design, *ptrs, ctypes.c_void_p(c.data_ptr()), reps, workgroups, stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(a.steps):
            st = L.nvfp4_probe_design(design, *ptrs, ctypes.c_void_p(c.data_ptr()), reps, workgroups, stream)
        e1.record()
        e1.synchronize()
        if st != 0:
            raise SystemExit(f"probe launch failed: {st}")
        ms = e0.elapsed_time(e1) / a.steps
        flops = float(waves[design]) * workgroups * reps * tile_flops[design]
        out[design] = (ms, flops / (ms * 1e-3) / 1e12)
    print(json.dumps({
        "metric": "GEMM design probe: inner-step TFLOP/s of useful work (one 16-element block per step)",
        "value": round(out[0][1], 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(out[0][0], 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4 codes", "data": "synthetic",
        "config": {"workload": "GEMM design probe: 4096 waves x 2000 repetitions of a 128x128x16 block step"},
        "components": {"design0_fp16_decode_ms": round(out[0][0], 4), "design0_tflops": round(out[0][1], 1),
                       "design1_fp4_rescale_ms": round(out[1][0], 4), "design1_tflops": round(out[1][1], 1),
                       "design0_over_design1": round(out[1][0] / out[0][0], 2),
                       "mfma_alone_ms": round(out[2][0], 4), "mfma_alone_tflops": round(out[2][1], 1),
                       "tile64x128_two_waves_per_simd_tflops": round(out[3][1], 1),
                       "tile64x128_one_wave_per_simd_tflops": round(out[4][1], 1),
                       "tile64x128_mfma_alone_two_waves_tflops": round(out[5][1], 1),
                       "independent_decode_one_wave_tflops": round(out[6][1], 1),
                       "pipelined_decode_one_wave_tflops": round(out[7][1], 1),
                       "independent_conversions_one_wave_tflops": round(out[8][1], 1)},
    }), flush=True)


def run_dequant(a, nv, torch, synth, dev):
    """nvfp4_dequantize of the fprop shapes: W [14336 x 4096] (16x16 tiles) and X [8192 x 4096] (1D)
    to bf16, and W to fp32.  One step = the three decodes; algorithmic bytes = codes + scale bytes
    read, the decoded tensor written."""
    x_cpu, w_cpu = synth.fprop8b(0)
    qx = nv.nvfp4_quantize(x_cpu.to(dev))
    qw = nv.nvfp4_quantize(w_cpu.to(dev), flags=nv.NVFP4_BLOCK2D)
    del x_cpu, w_cpu
    yw16 = torch.empty((qw.rows, qw.k), dtype=torch.bfloat16, device=dev)
    yw32 = torch.empty((qw.rows, qw.k), dtype=torch.float32, device=dev)
    yx16 = torch.empty((qx.rows, qx.k), dtype=torch.bfloat16, device=dev)
    calls = [("w_2d_bf16", lambda: nv.nvfp4_dequantize(qw, out=yw16), qw, 2),
             ("x_1d_bf16", lambda: nv.nvfp4_dequantize(qx, out=yx16), qx, 2),
             ("w_2d_f32", lambda: nv.nvfp4_dequantize(qw, out=yw32), qw, 4)]

    def nbytes(q, es):
        return q.data.numel() + q.scales.numel() + q.rows * q.k * es

    def step():
        for _, fn, _, _ in calls:
            fn()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    comp = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, fn, q, es in calls:
        e0.record()
        for _ in range(a.steps):
            fn()
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / a.steps
        comp[name + "_ms"] = round(ms, 4)
        comp[name + "_gbps"] = round(nbytes(q, es) / (ms * 1e-3) / 1e9, 1)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for _ in range(a.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / a.steps
    total = sum(nbytes(q, es) for _, _, q, es in calls)
    gbps = total / (ms_step * 1e-3) / 1e9
    w16 = comp["w_2d_bf16_gbps"]
    result = {
        "metric": "NVFP4 dequantize HBM GB/s",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1 x e4m3) -> bf16 / f32",
        "data": "synthetic",
        "config": {"workload": "decode of Llama-3-8B FFN fprop operands: W[14336x4096] 16x16 tiles -> bf16 and f32, "
                               "X[8192x4096] 1D -> bf16"},
        "components": dict(comp, algorithmic_bytes=total,
                           step_timing="HIP graph replay of the three decodes; components: mean of back-to-back launches"),
        "roofline": {"kernel": "nvfp4 dequantize (W 2D -> bf16)", "bound": "hbm", "achieved": w16,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(w16 / PEAK_HBM_GBPS, 4), "traffic": None},
    }
    print(json.dumps(result), flush=True)


def run_moe(a, nv, torch, synth, dev):
    """MoE expert layer, one step: nvfp4_quantize of the routed activations X_sorted [32768 x 4096]
    (rows already in expert order: the token gather / dispatch happens before the step),
    nvfp4_quantize_grouped of the 64 expert weights W_e [4096 x 1536] (column-wise, so blocks run
    along K = 4096, with Four-over-Six, each expert its own tensor scale) into one group-contiguous
    B, then the grouped GEMM Y_e = X_e W_e^T, bf16 out.  For comparison the experts are also
    quantized by 64 separate nvfp4_quantize calls (captured as one graph)."""
    import numpy as np
    E, K, N, T = 64, 4096, 1536, 16384
    experts = synth.moe_experts(0, E, K, N, workers=max(1, min(16, os.cpu_count() or 1)))
    w_all = torch.stack(experts).to(dev)  # [E, K, N]
    del experts
    tokens = synth.moe_tokens(0, T, K)
    loads, slot_token = synth.moe_routing(T, E, 2, 1.1, 0)
    offs = [int(v) for v in np.concatenate([[0], np.cumsum(loads)])]
    M = offs[-1]
    xg = tokens[torch.from_numpy(slot_token)].to(dev)  # [32768, 4096]
    del tokens
    fl = nv.NVFP4_COLWISE | nv.NVFP4_FOUR_OVER_SIX
    qa = nv.empty_like_quantized(M, K, 0, dev)
    qb = nv.NVFP4Tensor(torch.empty((E * N, K // 2), dtype=torch.uint8, device=dev),
                        torch.empty((E * N, K // 16), dtype=torch.uint8, device=dev),
                        torch.empty(E, dtype=torch.float32, device=dev), N, K, fl, E)
    views = [nv.NVFP4Tensor(qb.data[e * N:(e + 1) * N], qb.scales[e * N:(e + 1) * N],
                            qb.tensor_scale[e:e + 1], N, K, fl) for e in range(E)]
    ws_a = torch.empty(nv.nvfp4_workspace_size(M, K, 0) // 4, dtype=torch.int32, device=dev)
    ws_b = torch.empty(nv.nvfp4_workspace_size(K, N, fl) // 4, dtype=torch.int32, device=dev)
    ws_bg = torch.empty(E * nv.nvfp4_workspace_size(K, N, fl) // 4, dtype=torch.int32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def q_a():
        nv.nvfp4_quantize(xg, out=qa, workspace=ws_a)

    def q_b():
        nv.nvfp4_quantize_grouped(w_all, flags=fl, out=qb, workspace=ws_bg)

    def q_b_separate():
        for e in range(E):
            nv.nvfp4_quantize(w_all[e], flags=fl, out=views[e], workspace=ws_b)

    def mm():
        nv.nvfp4_gemm(qa, qb, out=y, group_offsets=offs)

    def step():
        q_a(); q_b(); mm()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    def per_call_ms(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        mm()
        e0.record()
        for _ in range(a.steps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / a.steps

    qa_ms, qb_ms, mm_ms = per_call_ms(q_a), per_call_ms(q_b), per_call_ms(mm)
    step()
    torch.cuda.synchronize()
    y_eager = y.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(y, y_eager):
        print(json.dumps({"error": "graph replay differs from eager result"}))
        sys.exit(1)
    # the experts as 64 separate calls, as one graph: 128 short kernels, launch gaps included
    g_b = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_b):
        q_b_separate()
    for _ in range(a.warmup):
        graph.replay()
        g_b.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(a.steps):
        g_b.replay()
    e1.record()
    e1.synchronize()
    qb_graph_ms = e0.elapsed_time(e1) / a.steps
    t0 = time.perf_counter()
    for _ in range(a.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / a.steps

    flops = 2.0 * M * N * K
    gemm_tflops = flops / (mm_ms * 1e-3) / 1e12
    qa_bytes = quant_bytes(M, K, False)
    qb_bytes = E * quant_bytes(N, K, False)
    # tiles of the grouped call: 256 x 256, except a group's last band when it holds at most 128 rows
    # (a 128 x 256 tile of half the work, in a launch of its own)
    half_bands = int(sum(1 for m in loads if 0 < int(m) % 256 <= 128))
    full_bands = int(sum((int(m) + 255) // 256 for m in loads)) - half_bands
    tiles = (full_bands + half_bands) * (N // 256)
    padded_rows = 256 * full_bands + 128 * half_bands
    result = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1 x e4m3) -> exact f16 operands, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "MoE experts: 64 x W_e[4096x1536] Student-t(4) col-wise 4/6, X_sorted[32768x4096] "
                               "(16384 tokens, top-2, Zipf(1.1) loads) 1D, grouped Y_e = X_e W_e^T bf16",
                   "M": M, "N": N, "K": K, "groups": E, "out": "bfloat16",
                   "loads_min_max": [int(loads.min()), int(loads.max())]},
        "components": {
            "quantize_x_ms": round(qa_ms, 4),
            "quantize_x_gbps": round(qa_bytes / (qa_ms * 1e-3) / 1e9, 1),
            "quantize_experts_ms": round(qb_ms, 4),
            "quantize_experts_gbps": round(qb_bytes / (qb_ms * 1e-3) / 1e9, 1),
            "quantize_experts_frac_hbm": round(qb_bytes / (qb_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "quantize_experts_separate_calls_graph_ms": round(qb_graph_ms, 4),
            "quantize_algorithmic_bytes": qa_bytes + qb_bytes,
            "gemm_ms": round(mm_ms, 4),
            "gemm_tflops": round(gemm_tflops, 1),
            "gemm_tiles": tiles,
            "gemm_half_tiles": half_bands * (N // 256),
            "gemm_tile_fill": round(M / padded_rows, 4),
            "step_timing": "HIP graph replay of quantize(X_sorted) + grouped quantize(64 W_e) + grouped GEMM; "
                           "components: mean of back-to-back launches",
        },
        "roofline": {
            "kernel": "nvfp4 grouped gemm",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 1),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_F16_TFLOPS, 4),
            "traffic": None,
        },
    }
    print(json.dumps(result), flush=True)


def cpu_baseline(a, nv):
    """The CPU oracle (as it stands) on bounded samples of the workloads, on the host's cores.

    Main sample (the `value`, in the step's unit: TFLOP/s of 2*m*n*K per second of quantize + GEMM):
    quantize the first rows of X (1D) and of W (16x16 tiles), then the binary64 GEMM of the two
    samples over the full K, handed to the oracle as 128 x 128 output tiles (its GEMM runs one tile
    per thread).  Also: the same on one core (an eighth of the rows), the full tiny 64 x 64 x 64
    round trip, and 64 output tiles of 128 x 128 with the 405B FFN's K = 16384 (operands drawn
    like that workload's, 1024 rows each)."""
    import numpy as np
    import oracle
    import synth
    threads = max(1, min(16, os.cpu_count() or 1))

    def tiles_of(m, n, t=128):
        return [(i, j, min(t, m - i), min(t, n - j)) for i in range(0, m, t) for j in range(0, n, t)]

    rows = a.cpu_rows
    x_cpu, w_cpu = synth.fprop8b(0)
    xs = synth.bf16_bits(x_cpu[:rows].contiguous())
    wsmp = synth.bf16_bits(w_cpu[:rows].contiguous())
    del x_cpu, w_cpu
    K = xs.shape[1]
    t0 = time.perf_counter()
    qx = oracle.quantize(xs, nthreads=threads)
    qw = oracle.quantize(wsmp, flags=oracle.BLOCK2D, nthreads=threads)
    t1 = time.perf_counter()
    oracle.gemm_ref(qx, qw, rows, rows, K, tiles=tiles_of(rows, rows), nthreads=threads)
    t2 = time.perf_counter()
    flops = 2.0 * rows * rows * K
    qbytes = quant_bytes(rows, K, False) + quant_bytes(rows, K, True)
    # one core, on an eighth of the sample
    r1 = max(16, rows // 8)
    s0 = time.perf_counter()
    qx1 = oracle.quantize(xs[:r1], nthreads=1)
    qw1 = oracle.quantize(wsmp[:r1], flags=oracle.BLOCK2D, nthreads=1)
    s1 = time.perf_counter()
    oracle.gemm_ref(qx1, qw1, r1, r1, K, tiles=tiles_of(r1, r1), nthreads=1)
    s2 = time.perf_counter()
    # the tiny round trip, in full: quantize A and B (fp32 64 x 64), dequantize, GEMM
    ta, tb = synth.tiny(0)
    u0 = time.perf_counter()
    qa, qb = oracle.quantize(ta.numpy(), nthreads=threads), oracle.quantize(tb.numpy(), nthreads=threads)
    oracle.dequantize(qa["data"], qa["scales"], qa["ts"], 64, 64)
    oracle.dequantize(qb["data"], qb["scales"], qb["ts"], 64, 64)
    oracle.gemm_ref(qa, qb, 64, 64, 64, nthreads=threads)
    u1 = time.perf_counter()
    # 64 tiles of 128 x 128 with K = 16384 (the 405B FFN's contraction), operands of that workload's
    # distributions: X ~N(0,1) with 0.1% outlier channels x20, W ~N(0,0.01) in 16x16 tiles
    xa = synth.normal((1024, 16384), 1.0, seed=0, tensor_id=8)
    synth.outlier_columns(xa, 0.001, 20.0, seed=0, tensor_id=8)
    wb = synth.normal((1024, 16384), 0.01, seed=0, tensor_id=9)
    q5a = oracle.quantize(synth.bf16_bits(xa), nthreads=threads)
    q5b = oracle.quantize(synth.bf16_bits(wb), flags=oracle.BLOCK2D, nthreads=threads)
    v0 = time.perf_counter()
    oracle.gemm_ref(q5a, q5b, 1024, 1024, 16384, tiles=tiles_of(1024, 1024), nthreads=threads)
    v1 = time.perf_counter()
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(flops / (t2 - t0) / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"quantize X[:{rows}] (1D) and W[:{rows}] (2D), binary64 GEMM {rows}x{rows}x{K} as 128x128 tiles",
        "seconds": round(t2 - t0, 3),
        "quantize_gbps": round(qbytes / (t1 - t0) / 1e9, 3),
        "gemm_gflops": round(flops / (t2 - t1) / 1e9, 3),
        "one_core": {"sample": f"quantize X[:{r1}], W[:{r1}], GEMM {r1}x{r1}x{K}",
                     "quantize_gbps": round((quant_bytes(r1, K, False) + quant_bytes(r1, K, True)) / (s1 - s0) / 1e9, 3),
                     "gemm_gflops": round(2.0 * r1 * r1 * K / (s2 - s1) / 1e9, 3)},
        "tiny_round_trip_ms": round((u1 - u0) * 1e3, 3),
        "k16384_tiles": {"sample": "64 tiles of 128x128, K = 16384 (binary64)",
                         "seconds": round(v1 - v0, 3),
                         "gemm_gflops": round(64 * 2.0 * 128 * 128 * 16384 / (v1 - v0) / 1e9, 3)},
        "nproc": os.cpu_count(),
        "cpu_model": cpu_model,
    }


if __name__ == "__main__":
    main()
