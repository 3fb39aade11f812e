"""Host-side pieces of bench.py: the traffic record and the rooflines built
from it must evaluate without a GPU (a stale record gives None, never an
error), and --gpus above 1 is refused."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_record_lookups_evaluate():
    for key in bench.CALL_GROUPS:
        t = bench.measured_traffic(key)
        assert t is None or t > 0
    assert bench.measured_traffic("no_such_call") is None
    v = bench.intra_valu(3.8)
    assert v is None or (v["bound"] == "alu" and 0 < v["frac"] < 1)


def test_traffic_record_names_every_group():
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert set(rec["sources_sha"]) == set(bench.SOURCE_GROUPS)
    assert set(rec["calls"]) == set(bench.CALL_GROUPS)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True)
    assert r.returncode == 2 and "one GPU" in r.stdout


def test_per_call_statistics_and_host_description():
    assert bench.stats([3.0, 1.0, 2.0, 10.0]) == {"median": 2.5, "min": 1.0, "max": 10.0, "mean": 4.0, "n": 4}
    assert bench.stats([5.0, 1.0, 4.0])["median"] == 4.0
    h = bench.host_cpu()
    assert h["cores_available"] >= 1
