"""Build libbaim.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m bias_addmm_im2col_amd.build

Uses hipcc directly; the library is written next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libbaim.so")
SOURCES = ["api.cpp", "tile_select.cpp", "conv_window_plan.cpp", "sdpa_plan.cpp", "addmm.hip", "conv2d_gemm.hip", "conv_window.hip", "conv_stem.hip",
           "conv_direct.hip", "sdpa.hip", "conv_transpose.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    # never emit packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _scratch_kernels(remarks: str):
    """Kernels whose resource-usage remark reports private (scratch) memory:
    a spill or an address-taken argument, both costly in these kernels."""
    bad, name = [], None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split("[")[0].strip()
        elif "ScratchSize [bytes/lane]:" in line and name:
            n = int(line.split("ScratchSize [bytes/lane]:")[1].split("[")[0].strip())
            if n > 0:
                bad.append((name, n))
    return bad


def build(verbose: bool = False) -> str:
    """Compile every source into libbaim.so (always rebuilds).  Fails if a
    kernel uses scratch memory."""
    objs = []
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(HERE, "_build", os.path.splitext(src)[0] + ".o")
        cmd = [hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c"]
        if src.endswith(".cpp"):
            cmd += ["-x", "hip"]
        else:
            cmd += ["-Rpass-analysis=kernel-resource-usage"]
        cmd += [os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), src))
        objs.append(obj)
    failed = []
    scratch = []
    for p, src in procs:
        _, err = p.communicate()
        scratch += _scratch_kernels(err)
        # hipcc's host pass does not know the packed-fp32 feature: harmless;
        # resource-usage remarks are parsed above
        err = "\n".join(l for l in err.splitlines()
                        if "packed-fp32-ops" not in l and "remark:" not in l)
        if p.returncode != 0:
            failed.append((src, err))
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"--- {s}\n{e}" for s, e in failed))
    if scratch:
        raise RuntimeError("kernels use scratch memory:\n" +
                           "\n".join(f"  {n}: {b} bytes/lane" for n, b in scratch))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
