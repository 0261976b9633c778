"""MI355X (gfx950) TurboQuant-style KV-cache codec.

The codec lives in libtq.so (HIP kernels behind the C ABI of include/tq.h);
``binding`` is a thin ctypes layer over it and ``synth`` draws the seeded
synthetic inputs used by the tests and the benchmark.
"""
from . import binding  # noqa: F401
