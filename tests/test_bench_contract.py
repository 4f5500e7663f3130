"""CPU checks of the benchmark's command-line contract and of its HBM-traffic lookup."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("args, words", [
    (["--chunks", "4"], "--chunks"),                    # chunks serve the one-shot prefill (c3) only
    (["--config", "c3", "--chunks", "0"], "--chunks"),
    (["--config", "c3", "--verify", "4"], "--verify"),  # verification serves the decode workloads
    (["--window", "-1"], "--window"),
])
def test_workload_options_are_checked_before_any_gpu_work(args, words):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert words in r.stderr


def _summary_lines():
    for line in open(os.path.join(ROOT, "profiles", "hbm_traffic.txt")):
        if not line.startswith("#") and line.strip():
            yield line.split()


def test_traffic_lookup_follows_the_source_hash():
    lines = list(_summary_lines())
    assert lines and all(len(f) == 8 for f in lines)
    for kernel, workload, fetch_kib, write_kib, fscale, wscale, total, src in lines:
        # the stored total is the two counters scaled as the header says (the printed counters and
        # scales are rounded, the total was not)
        expect = float(fetch_kib) * 1024 * float(fscale) + float(write_kib) * 1024 * float(wscale)
        assert abs(int(total) - expect) <= 1e-4 * expect + 4096
        m = hashlib.sha256()
        for fn in bench.KERNEL_SOURCES[kernel]:
            m.update(open(os.path.join(ROOT, fn), "rb").read())
        got = bench.measured_traffic(kernel, workload)
        # reported only while the kernel sources are the ones the counters were taken on
        assert got == (int(total) if m.hexdigest()[:16] == src else None)
    assert bench.measured_traffic("decode_split", "no_such_workload") is None
    assert bench.measured_traffic("no_such_kernel", "c2_decode_b32") is None


@pytest.mark.parametrize("stem", sorted(f[:-len("_kernel_trace.md")] for f in os.listdir(os.path.join(ROOT, "profiles"))
                                        if f.endswith("_kernel_trace.md")))
def test_each_trace_summary_states_its_command(stem):
    text = open(os.path.join(ROOT, "profiles", stem + "_kernel_trace.md")).read()
    assert "rocprofv3 --kernel-trace --stats" in text and "-- python3 bench.py" in text
    assert "roofline:" in text
