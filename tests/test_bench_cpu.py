"""Host-side checks of bench.py (no GPU): the one-GPU contract and the traffic bookkeeping."""
import json
import os
import subprocess
import sys

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_stored_traffic_matches_the_sources_it_names():
    """profiles/hbm_traffic.json holds bytes per launch with a hash of the kernel sources they were
    taken on; bench.py reports a kernel's traffic only while the hash matches.  Every entry names
    sources that exist, and its hash has the source_hash form."""
    with open(bench.COUNTERS) as fh:
        c = json.load(fh)
    assert c["copy_bytes"] > 0 and c["scale_fetch"] > 0 and c["scale_write"] > 0
    for name, e in c["kernels"].items():
        assert name in bench.KERNEL_SOURCES
        assert sorted(e["sources"]) == sorted(bench.KERNEL_SOURCES[name])
        h = bench.source_hash(e["sources"])
        assert len(e["source_hash"]) == len(h) == 16
        assert e["bytes_per_launch"] > 0
