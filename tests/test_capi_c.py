"""The C ABI from a plain C program (tests/capi_check.c): include/baim.h
compiles as C11, the program links against libbaim.so alone (no Python,
no torch), and on a GPU every entry point matches the oracle and reports
invalid calls through its status codes."""
import os
import subprocess

import pytest

from tests import capi_build


def _libs():
    from bias_addmm_im2col_amd import _capi
    if not os.path.exists(_capi.LIB_PATH):
        from bias_addmm_im2col_amd import build as b
        b.build()
    import oracle
    oracle.build(force=False)


def test_capi_check_compiles_as_c():
    _libs()
    assert os.path.exists(capi_build.build())


@pytest.mark.gpu
def test_capi_check_runs_on_the_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    exe = capi_build.EXE
    if not os.path.exists(exe):
        _libs()
        capi_build.build()
    print(f"[capi] running {exe}", flush=True)
    proc = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(proc.stdout)
    assert proc.returncode == 0 and "capi_check OK" in proc.stdout, proc.stdout + proc.stderr
