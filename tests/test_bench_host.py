"""Host-side checks of bench.py (no GPU): the multi-GPU refusal and the
committed traffic-counter summary it reads its roofline 'traffic' from."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_source_hash_covers_the_kernel_file_and_shared_headers():
    for k in bench.KERNEL_SOURCES:
        h = bench.source_hash(k)
        assert len(h) == 16 and int(h, 16) >= 0
    # kernels in one source file share the hash; different files differ
    assert bench.source_hash("quantize_kernel") == bench.source_hash("dequantize_kernel")
    assert bench.source_hash("quantize_kernel") != bench.source_hash("decode_attn_mfma_kernel")


def test_traffic_summary_lines_are_well_formed_and_near_the_algorithmic_bytes():
    # algorithmic bytes per launch of each recorded workload
    want = {"quantize_kernel": 4194304 * 712, "dequantize_kernel": 4194304 * 712,
            "decode_attn_mfma_kernel": 16 * 8 * 32768 * 200 + 2 * (2 * 16 * 32 * 128),
            "dense_quantize_kernel": 8388608 * (256 + 52), "dense_dequantize_kernel": 8388608 * (256 + 52)}
    seen = set()
    for line in open(os.path.join(ROOT, "profiles", "traffic_counters.txt")):
        if line.startswith("#") or not line.strip():
            continue
        f = dict(kv.split("=", 1) for kv in line.split())
        assert set(f) == {"kernel", "src", "bytes_per_launch", "workload"}, line
        assert f["kernel"] in bench.KERNEL_SOURCES, line
        b = float(f["bytes_per_launch"])
        assert abs(b - want[f["kernel"]]) <= 0.01 * want[f["kernel"]], (f["kernel"], b)
        seen.add(f["kernel"])
    assert seen == set(bench.KERNEL_SOURCES)
