"""Host-side checks of the benchmark harness (no GPU needed).

* a multi-GPU request exits before touching any device, with a message;
* the kernel-source fingerprint that keys the recorded HBM traffic ignores
  comments and whitespace but not code;
* the recorded traffic, and the deleted-load gate read from the same counter
  summary, are reported only while the fingerprint matches.
"""
import json
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def _copy_sources(dst):
    for rel in bench.GEMV_SOURCES:
        os.makedirs(os.path.join(dst, os.path.dirname(rel)), exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), os.path.join(dst, rel))


def test_source_fingerprint_ignores_comments_not_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _copy_sources(str(tmp_path))
    base = bench.gemv_source_hash()
    main = os.path.join(str(tmp_path), bench.GEMV_SOURCES[0])
    text = open(main).read()
    # comments and whitespace: same fingerprint
    open(main, "w").write("// a new comment\n/* and a\n block */\n" + text.replace("\n", "\n  ", 3))
    assert bench.gemv_source_hash() == base
    # one changed constant: a different fingerprint
    assert "kOob" in text or "0x" in text
    open(main, "w").write(text + "\nstatic const int kProbe = 1;\n")
    assert bench.gemv_source_hash() != base


def test_traffic_reported_only_for_matching_sources(tmp_path, monkeypatch):
    prof = tmp_path / "traffic.md"
    prof.write_text("# traffic\n\ntraffic_bytes_per_launch: 12345\nsource_sha256: %s\n" % bench.gemv_source_hash())
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.measured_traffic() == 12345
    prof.write_text("# traffic\n\ntraffic_bytes_per_launch: 12345\nsource_sha256: %s\n" % ("0" * 64))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "absent.md"))
    assert bench.measured_traffic() is None


def test_deleted_load_check_from_the_counter_summary(tmp_path, monkeypatch):
    prof = tmp_path / "traffic.md"
    h = bench.gemv_source_hash()
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    prof.write_text("traffic_bytes_per_launch: 1010\nfloor_fetch_bytes_per_launch: 990\n"
                    "algorithmic_bytes_per_launch: 1000\nsource_sha256: %s\n" % h)
    chk = bench.deleted_load_check()
    assert chk["floor_fetch_over_algorithmic"] == 0.99 and chk["ok"]
    # a floor that reads less than 98 % of the algorithmic bytes skipped loads
    prof.write_text("traffic_bytes_per_launch: 1010\nfloor_fetch_bytes_per_launch: 970\n"
                    "algorithmic_bytes_per_launch: 1000\nsource_sha256: %s\n" % h)
    assert not bench.deleted_load_check()["ok"]
    # stale summary: no verdict
    prof.write_text("traffic_bytes_per_launch: 1010\nfloor_fetch_bytes_per_launch: 990\n"
                    "algorithmic_bytes_per_launch: 1000\nsource_sha256: %s\n" % ("0" * 64))
    assert bench.deleted_load_check() is None

