import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_addoption(parser):
    parser.addoption("--checked-build", action="store_true", default=False,
                     help="run every GPU test's calls through libtq_check.so (the bounds-checked build) "
                          "and require a clean bounds-test flag word after each test")


@pytest.fixture(autouse=True)
def _checked_build(request):
    """With --checked-build, each GPU test runs against the bounds-checked
    library and fails if any kernel derived a row, record or byte outside the
    extents of its buffers."""
    if not request.config.getoption("--checked-build") or request.node.get_closest_marker("gpu") is None:
        yield
        return
    import torch
    from kv_cache_quantization_02_amd import binding as tq
    with tq.checked_library():
        tq.tq_check_set_margin(0)
        tq.tq_check_flags()
        yield
        torch.cuda.synchronize()
        flags = tq.tq_check_flags()
    assert flags == 0, f"bounds-test flags {flags:#x} after {request.node.nodeid}"


def pytest_collection_modifyitems(config, items):
    # GPU tests run on the GPU machine only; elsewhere they are skipped, not failed.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


# The five named workloads print last, so that they sit at the end of the log.
_NAMED_LAST = ("roundtrip k8v3 d128", "decode append k8v3 d128", "prefill k8v3 d128", "wide k4v4 d256",
               "wide k5v2 d512", "decode attention k8v3 d128")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Boundary ties and inexact dequant elements per configuration (parity.record)."""
    mod = sys.modules.get("parity")
    rec = getattr(mod, "RECORD", None)
    if not rec:
        return
    terminalreporter.section("parity record: index ties counted, dequant elements not bit-exact")

    def fmt(name, r):
        parts = [f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}" for k, v in r.items()]
        return f"{name}: " + ", ".join(parts)
    named = [n for n in rec if any(n.startswith(p) for p in _NAMED_LAST)]
    other = [n for n in rec if n not in named]
    if other:
        agg = {}
        for n in other:
            for k, v in rec[n].items():
                agg[k] = max(agg.get(k, 0.0), v) if isinstance(v, float) else agg.get(k, 0) + v
        terminalreporter.write_line(fmt(f"other cases ({len(other)})", agg))
    for p in _NAMED_LAST:
        for n in named:
            if n.startswith(p):
                terminalreporter.write_line(fmt(n, rec[n]))
