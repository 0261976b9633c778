"""Build libtq.so (the HIP codec library) and libtq_check.so (the same
sources with every kernel's bounds tests compiled in, TQ_CHECK) in-tree for
gfx950.

    python -m kv_cache_quantization_02_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtq.so")
LIB_CHECK = os.path.join(PKG, "libtq_check.so")
# library -> extra flags
VARIANTS = {LIB: [], LIB_CHECK: ["-DTQ_CHECK"]}
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
    """Compile every source of both libraries to objects (in parallel), then
    link each; returns the path of libtq.so."""
    from concurrent.futures import ThreadPoolExecutor

    jobs = []  # (library, object, command)
    for lib, extra in VARIANTS.items():
        for src in SOURCES:
            obj = lib + "." + os.path.splitext(src)[0] + ".o"
            jobs.append((lib, obj, [HIPCC, *FLAGS, *extra, *SOURCE_FLAGS.get(src, []), "-c",
                                    os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        results = list(ex.map(_run, [cmd for _, _, cmd in jobs]))
    links = []
    if all(r.returncode == 0 for r in results):
        for lib in VARIANTS:
            objs = [obj for l, obj, _ in jobs if l == lib]
            links.append((lib, _run([HIPCC, *FLAGS, "-shared", *objs, "-o", lib + ".tmp"])))
    for _, obj, _ in jobs:
        if os.path.exists(obj):
            os.remove(obj)
    results += [r for _, r in links]
    failed = [r for r in results if r.returncode != 0]
    noise = "is not a recognized feature for this target"
    for r in (failed if failed else (results if verbose else [])):
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if msg.strip():
            sys.stderr.write(msg + "\n")
    if failed:
        raise RuntimeError("hipcc failed building libtq.so / libtq_check.so")
    for lib, _ in links:
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
