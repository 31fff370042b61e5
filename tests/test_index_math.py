"""Host build and run of tests/index_math_check.cpp: the kernels'
multiply-high division and block -> tile map (no GPU)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_index_math(tmp_path):
    exe = tmp_path / "index_math_check"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-Wall",
                           "-I", os.path.join(ROOT, "bias_addmm_im2col_amd", "csrc"),
                           os.path.join(ROOT, "tests", "index_math_check.cpp"), "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.strip() == "OK", out.stdout


def test_tile_select(tmp_path):
    exe = tmp_path / "tile_select_check"
    csrc = os.path.join(ROOT, "bias_addmm_im2col_amd", "csrc")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-Wall", "-I", csrc,
                           os.path.join(ROOT, "tests", "tile_select_check.cpp"),
                           os.path.join(csrc, "tile_select.cpp"), "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.strip() == "OK", out.stdout


def test_sdpa_plan(tmp_path):
    exe = tmp_path / "sdpa_plan_check"
    csrc = os.path.join(ROOT, "bias_addmm_im2col_amd", "csrc")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-Wall", "-I", csrc,
                           os.path.join(ROOT, "tests", "sdpa_plan_check.cpp"),
                           os.path.join(csrc, "sdpa_plan.cpp"), "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.strip() == "OK", out.stdout
