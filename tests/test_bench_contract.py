"""bench.py's contract on the CPU: one GPU only (more exits with a message and
code 2, before any device work), and the committed HBM traffic records carry
the counter readings, the copy-kernel calibration and the algorithmic bytes
that the bench line's roofline.traffic is derived from."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("kind", sorted(bench.TRAFFIC))
def test_traffic_records_are_complete(kind):
    spec = bench.TRAFFIC[kind]
    rec = json.load(open(os.path.join(ROOT, "profiles", spec["record"])))
    assert rec["kernel"] == spec["kernel"] and rec["source_files"] == spec["sources"]
    assert rec["algorithmic_bytes_per_launch"] == spec["algorithmic_bytes"]
    # the copy kernel reads and writes 1 GiB: the scales map its counter readings to that
    assert rec["fetch_scale"] * rec["copy_fetch_size_kib"] * 1024 == pytest.approx(bench.COPY_BYTES)
    assert rec["write_scale"] * rec["copy_write_size_kib"] * 1024 == pytest.approx(bench.COPY_BYTES)
    traffic = (rec["fetch_size_kib"] * rec["fetch_scale"] + rec["write_size_kib"] * rec["write_scale"]) * 1024
    assert rec["traffic_bytes_per_launch"] == pytest.approx(traffic)
    assert rec["traffic_bytes_per_launch"] >= 0.99 * rec["algorithmic_bytes_per_launch"]
    assert any("--pmc FETCH_SIZE" in c for c in rec["commands"]) and any("--pmc WRITE_SIZE" in c for c in rec["commands"])


def test_attention_record_matches_the_current_source():
    # the bench line reports roofline.traffic only while this holds
    assert bench.measured_traffic("attention") is not None
