"""CPU checks of bench.py's contract: it measures one GPU and says so for more,
its algorithmic byte counts, and when it reports the counter-based traffic."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes():
    # read X and layer_out, write X' and layer_in (state dtype), W f16 and bias
    # once, coefficients [T, 24] f32
    T, n, d = 4096, 4, 4096
    m, K = 24, n * d
    want = T * K * 4 * 2 + T * d * 4 * 2 + m * K * 2 + m * 4 + T * m * 4
    assert bench.algorithmic_bytes(T, n, d, 4) == want == 672_268_384
    assert bench.algorithmic_bytes(16384, 4, 7168, 2) == 2_351_759_456
    assert bench.algorithmic_bytes(T, n, d, 4, with_coeffs=False) == want - T * m * 4


def test_traffic_reported_only_for_matching_sources():
    for workload, path in bench.COUNTERS_FILE.items():
        with open(os.path.join(ROOT, path)) as f:
            rec = json.load(f)
        assert rec["workload"] == workload
        got = bench.load_traffic(workload, rec["source_sha256"])
        assert got == rec["traffic_bytes_per_launch"]
        assert bench.load_traffic(workload, "0" * 64) is None
        # the record is plausible: within 10 % of the algorithmic bytes
        assert 0.9 < rec["traffic_over_algorithmic"] < 1.1
