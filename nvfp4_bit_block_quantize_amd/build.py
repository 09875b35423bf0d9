"""Build libnvfp4.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m nvfp4_bit_block_quantize_amd.build            (or python nvfp4_bit_block_quantize_amd/build.py)
    python -m nvfp4_bit_block_quantize_amd.build --changed  (recompile only objects older than their
                                                             source or any header)

Every source is compiled with hipcc for gfx950 with -ffp-contract=off (no silent fused multiply-add:
the quantizer is bit-exact), packed-FP32 instructions disabled and hidden symbol visibility (only
the C ABI of include/nvfp4.h is exported).  The NVFP4 x NVFP4 GEMM kernels are instantiated one
(output type, A scale layout, B scale layout) combination per object (gemm_variant.hip compiled
twelve times), so that they compile in parallel.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libnvfp4.so")
# the GEMM design probe (measurement only, not part of the library): bench.py --workload gemm_designs
PROBE_OUT = os.path.join(HERE, "libnvfp4_probe.so")
BUILD = os.path.join(HERE, "_build")
ARCH = os.environ.get("NVFP4_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fvisibility=hidden", "-Wall",
          "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def units():
    """(source, object name, extra flags) of every translation unit."""
    u = [(s, s + ".o", []) for s in ["nvfp4_api.cpp", "quantize.hip", "dequant.hip", "gemm.hip",
                                      "gemm_w4a16.hip", "transpose.hip"]]
    for out in (0, 1, 2):
        for a2d in (0, 1):
            for b2d in (0, 1):
                u.append(("gemm_variant.hip", f"gemm_variant_{out}{a2d}{b2d}.o",
                          [f"-DNVFP4_OUT={out}", f"-DNVFP4_A2D={a2d}", f"-DNVFP4_B2D={b2d}"]))
    return u


def _stale(obj, src):
    if not os.path.exists(obj):
        return True
    deps = [src] + glob.glob(os.path.join(CSRC, "*.h*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    deps = [d for d in deps if not d.endswith(".hip") or d == src]
    return any(os.path.getmtime(d) > os.path.getmtime(obj) for d in deps)


def _compile(unit, verbose, changed_only):
    src, name, extra = unit
    obj = os.path.join(BUILD, name)
    srcp = os.path.join(CSRC, src)
    if changed_only and not _stale(obj, srcp):
        return obj
    cmd = ["hipcc", *DEVICE, *COMMON, *extra, "-c", srcp, "-o", obj + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src} {' '.join(extra)}:\n{r.stderr}")
    os.replace(obj + ".tmp", obj)
    return obj


def build(verbose=False, changed_only=False):
    os.makedirs(BUILD, exist_ok=True)
    us = units() + [("probe_designs.hip", "probe_designs.hip.o", [])]
    # the largest units first, so that they do not start last
    us.sort(key=lambda u: 0 if u[0] in ("gemm_variant.hip", "quantize.hip", "gemm_w4a16.hip") else 1)
    with cf.ThreadPoolExecutor(max_workers=max(1, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose, changed_only), us))
    probe = [o for o in objs if o.endswith("probe_designs.hip.o")]
    lib_objs = [o for o in objs if o not in probe]
    for out, parts in ((OUT, lib_objs), (PROBE_OUT, probe)):
        cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-fvisibility=hidden", *parts, "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, changed_only="--changed" in sys.argv))
