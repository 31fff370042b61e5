"""Build tests/_build/capi_check: the C program in tests/capi_check.c that
drives libbaim.so from plain C and checks it against the oracle's C
library.  Test infrastructure (used by the test-suite and by the build
entry point, which compiles it next to the libraries)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "capi_check.c")
EXE = os.path.join(ROOT, "tests", "_build", "capi_check")


def build() -> str:
    """Compile capi_check (gcc, C11) against include/baim.h, libbaim.so,
    liboracle.so and the HIP runtime.  Returns the executable's path."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    tmp = EXE + ".tmp%d" % os.getpid()
    subprocess.check_call([
        "gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
        "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), SRC,
        "-o", tmp,
        "-L", os.path.join(ROOT, "bias_addmm_im2col_amd"), "-lbaim",
        "-L", os.path.join(ROOT, "oracle"), "-loracle",
        "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
        "-Wl,-rpath,$ORIGIN/../../bias_addmm_im2col_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
        "-Wl,-rpath," + os.path.join(rocm, "lib")])
    os.replace(tmp, EXE)
    return EXE
