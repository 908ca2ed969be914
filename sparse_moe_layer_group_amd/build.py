"""Build the gfx950 HIP library ``libmoe_mi355x.so`` in-tree with hipcc.

Usage: ``python -m sparse_moe_layer_group_amd.build`` (or ``build()``).
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
SOURCES = ["moe_api.cpp", "route_kernels.hip", "gemm_kernels.hip", "stream_gemm.hip", "tile_gemm.hip",
           "fp8_kernels.hip", "balance_kernels.hip", "bwd_kernels.hip", "bwd_fp8_kernels.hip"]
ARCH = "gfx950"

# Packed fp32 instructions are disabled for all device code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the library."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    jobs = []
    for s in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(s)[0] + ".o")
        jobs.append((obj, [hipcc()] + compile_flags + ["-x", "hip", "-c", os.path.join(CSRC, s),
                                                      "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(_run, cmd, verbose) for _, cmd in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc()] + HIP_FLAGS + [o for o, _ in jobs] + ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
