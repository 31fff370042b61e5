"""bench.py host logic, without a GPU: the one-GPU refusal and the hash gate
on the committed counter figures."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""


def test_counter_figures_only_for_the_hashed_kernel_sources(tmp_path, monkeypatch):
    kern = "baim::conv2d_gemm_kernel<Tile 128x64x64, 16 waves, 2 k-groups> stream 256"
    doc = {"kernel_source_sha": bench.kernel_source_hash(),
           "kernels": {kern: {"bytes_per_launch": 1234, "mfma_busy": 0.5}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(doc))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_counters(kern) == (1234, 0.5)
    assert bench.load_counters("some other kernel") == (None, None)
    # a kernel source that differs from the one the counters were taken on
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_counters(kern) == (None, None)
    # no file at all
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.load_counters(kern) == (None, None)


def test_source_hash_covers_every_library_source():
    # every kernel, header and host source of the library, and, transitively,
    # every local header they include
    import re
    csrc = os.path.join(ROOT, "bias_addmm_im2col_amd", "csrc")
    todo = [f for f in os.listdir(csrc) if f.endswith((".hip", ".cpp"))]
    seen = set()
    while todo:
        f = todo.pop()
        if f in seen:
            continue
        seen.add(f)
        if f == "baim.h":  # the public header, hashed from include/
            continue
        todo += re.findall(r'^#include "([^"]+)"', open(os.path.join(csrc, f)).read(), flags=re.M)
    seen.discard("baim.h")
    assert "conv_stem.hip" in seen and "sdpa.hip" in seen
    assert seen <= set(bench.KERNEL_SOURCES), seen - set(bench.KERNEL_SOURCES)
    assert len(bench.kernel_source_hash()) == 16


def test_source_hash_covers_the_compiler_flags(monkeypatch):
    from bias_addmm_im2col_amd import build
    h0 = bench.kernel_source_hash()
    monkeypatch.setattr(build, "HIPCC_FLAGS", build.HIPCC_FLAGS + ["-DX"])
    assert bench.kernel_source_hash() != h0
