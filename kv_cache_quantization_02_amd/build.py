"""Build libtq.so (the HIP codec library) in-tree for gfx950.

    python -m kv_cache_quantization_02_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtq.so")
SOURCES = ["tq_api.hip", "tq_codec.hip", "tq_attn.hip", "tq_dense.hip", "tq_cache.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # one IEEE operation per source operation: no contraction into fma,
    # correctly rounded fp32 division and sqrt, subnormals kept
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-source flags: the paper-variant kernels read their MFMA results with
# VALU code right away, so their accumulators are kept in VGPRs.
SOURCE_FLAGS = {"tq_dense.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libtq.so."""
    from concurrent.futures import ThreadPoolExecutor

    objs = [LIB + "." + os.path.splitext(s)[0] + ".o" for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, *SOURCE_FLAGS.get(s, []), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        results = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    if all(r.returncode == 0 for r in results):
        results.append(_run([HIPCC, *FLAGS, "-shared", *objs, "-o", tmp]))
    for o in objs:
        if os.path.exists(o):
            os.remove(o)
    failed = [r for r in results if r.returncode != 0]
    noise = "is not a recognized feature for this target"
    for r in (failed if failed else (results if verbose else [])):
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if msg.strip():
            sys.stderr.write(msg + "\n")
    if failed:
        raise RuntimeError("hipcc failed building libtq.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
