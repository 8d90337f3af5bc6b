"""Host logic of bench.py (no GPU): the multi-GPU refusal, the code digest
that keys the stored counter readings, and the stored readings themselves."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_code_digest_ignores_comments_only():
    a = "int f(int x) {\n  return x + 1;  // add one\n}\n"
    b = "/* increment */\nint f(int x) {\n\n  return x + 1;\n}  \n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_stored_readings_apply_only_to_the_code_they_were_taken_on():
    for kernel in bench.KERNEL_SOURCES:
        assert len(bench.source_digest(kernel)) == 16
    for (workload, kernel), (digest, fetch, write) in bench.MEASURED_KIB.items():
        t = bench.measured_traffic(workload, kernel)
        if digest == bench.source_digest(kernel):
            assert t == pytest.approx((fetch * bench.FETCH_SCALE + write * bench.WRITE_SCALE) * 1024)
        else:
            assert t is None  # the kernel changed since the counters were taken
    assert bench.measured_traffic("no_such_workload", "k_topk_stream") is None
