"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds the library sources with both sanitizers on their host code, links
them with tests/host_sanitize/abi_host_check.cpp, and runs that program: it
drives every entry point's validation with counts and strides at the ends of
their ranges (see its header).  Any sanitizer report or wrong status fails.
Runs only on a machine without a GPU; the build takes a minute or two.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_quantization_02_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "abi_host_check.cpp")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = ["tq_api.hip", "tq_codec.hip", "tq_attn.hip", "tq_dense.hip", "tq_cache.hip"]
# the sanitizers apply to host code only (device code cannot carry them)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present: the checker's fake addresses would launch")
@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found")
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    objs = []
    cmds = []
    for s in SOURCES:
        o = str(tmp_path / (s + ".o"))
        objs.append(o)
        cmds.append([HIPCC, *FLAGS, *SAN, "-c", os.path.join(CSRC, s), "-o", o])
    drv = str(tmp_path / "driver.o")
    cmds.append([HIPCC, "-O1", "-g", "-std=c++17", *SAN, "-c", DRIVER, "-o", drv])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        res = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds))
    for c, r in zip(cmds, res):
        assert r.returncode == 0, f"{' '.join(c)}\n{r.stderr[-3000:]}"
    exe = str(tmp_path / "abi_host_check")
    link = [CLANG, "-fsanitize=address,undefined", drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
            "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    if r.returncode == 77:
        pytest.skip("a GPU is present")
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-5000:]
    assert r.returncode == 0, out[-5000:]
    assert "0 failures" in out, out[-2000:]
