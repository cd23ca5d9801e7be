"""The C ABI's host code (parameter validation, pointer and workspace checks,
workspace-size arithmetic) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven by tests/host_sanitize/abi_driver.cpp.
The sanitizers instrument host code only (each flag is passed for the host
side), and the driver makes no call that reaches a kernel launch, so no GPU
is needed."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "content_routed_block_stats_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "abi_driver.cpp")

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]
FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC,
         *SAN]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.timeout(600)
def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    from content_routed_block_stats_amd.build import SOURCES

    def compile_one(src: str) -> str:
        obj = str(tmp_path / (os.path.splitext(os.path.basename(src))[0] + ".o"))
        r = subprocess.run([hipcc, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr[-4000:]}"
        return obj

    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [DRIVER]
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([hipcc, *SAN, "--offload-arch=gfx950", *objs, "-o", exe], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"rc {r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
    assert "all expectations hold" in r.stdout
