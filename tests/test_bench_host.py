"""bench.py host logic (CPU): the HBM traffic it reports comes from the
committed counter summary only while that summary's source hash matches the
sources the decode matvec is compiled from, and is scaled by the copy
calibration factors; a run on other sources reports none."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def summary_fields():
    kv = {}
    with open(bench.TRAFFIC_FILE) as fh:
        for line in fh:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    return kv


def test_traffic_scaled_when_the_hash_matches(monkeypatch):
    kv = summary_fields()
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: kv["source_sha1"])
    t = bench.measured_traffic()
    assert t is not None
    assert t["fetch"] == float(kv["fetch_kib_per_launch"]) * float(kv["copy_fetch_factor"]) * 1024
    assert t["write"] == float(kv["write_kib_per_launch"]) * float(kv["copy_write_factor"]) * 1024
    # the committed summary is the gate/up matvec of the 8B shape: within 1%
    # of its 234,971,136 algorithmic bytes per launch
    assert abs(t["fetch"] + t["write"] - 234971136) / 234971136 < 0.01


def test_no_traffic_on_other_sources(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 40)
    assert bench.measured_traffic() is None


def test_source_hash_covers_the_matvec_sources():
    names = sorted(os.path.basename(p) for p in bench.TRAFFIC_SOURCES)
    assert names == ["decode.hip", "device_common.h", "kernels.h"]
    h = bench.kernel_source_hash()
    assert len(h) == 40 and int(h, 16) >= 0
