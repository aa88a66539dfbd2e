"""The benchmark's contract on the CPU: one GPU per process, and the HBM
traffic figure of a kernel reported only while its sources are those the
counters were taken on."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
VALUE_FILES = ["rl_experience_collection_amd/csrc/value.hip",
               "rl_experience_collection_amd/csrc/nets.hpp",
               "rl_experience_collection_amd/csrc/device.hpp"]


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _copy_tree(tmp_path):
    for f in VALUE_FILES + ["profiles/value_kernel_n8192_l500_traffic.txt"]:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), dst)


def test_traffic_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    name = "value_kernel_n8192_l500_traffic.txt"
    kv = dict(line.split(":", 1) for line in open(tmp_path / "profiles" / name)
              if ":" in line and not line.startswith("#"))
    recorded = kv["source_sha256_16"].strip()
    if recorded == bench.source_hash(VALUE_FILES):
        assert bench.load_traffic(name, VALUE_FILES) == float(kv["hbm_bytes_per_launch"])
    # one byte more in a kernel source: the figure no longer applies
    with open(tmp_path / VALUE_FILES[0], "ab") as fh:
        fh.write(b"\n")
    assert bench.load_traffic(name, VALUE_FILES) is None
    # a summary without the figure, or none at all, gives none
    assert bench.load_traffic("no_such_summary.txt", VALUE_FILES) is None
