"""Host-only code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

csrc/plan.cpp (compiled with g++) and the host side of csrc/map_cache.hip
(hipcc, sanitizers on the host pass only) are linked with
tests/host_sanitize/driver.cpp, which runs random and malformed batches
through mf_plan and inserts, lookups, pins, releases and evictions through
the prefix cache's index (entries without kept blocks, which copy nothing)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "cross_model_attention_mf_amd", "csrc")
INC = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer"]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not (shutil.which("g++") and os.path.exists(HIPCC)), reason="needs g++ and hipcc")
def test_plan_and_cache_index_under_asan_ubsan(tmp_path):
    d = str(tmp_path)
    _run(["g++", "-std=c++17", "-O1", "-g", *SAN, "-I", INC, "-I", CSRC, "-c",
          os.path.join(CSRC, "plan.cpp"), "-o", "plan.o"], d)
    _run(["g++", "-std=c++17", "-O1", "-g", *SAN, "-I", INC, "-c",
          os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp"), "-o", "driver.o"], d)
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", *host_san, "-I", INC, "-I", CSRC, "-c", os.path.join(CSRC, "map_cache.hip"),
          "-o", "map_cache.o"], d)
    _run([HIPCC, "--offload-arch=gfx950", *host_san, "plan.o", "driver.o", "map_cache.o", "-o", "driver"], d)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([os.path.join(d, "driver")], cwd=d, capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr
