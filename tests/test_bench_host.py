"""Host-side logic of bench.py that needs no GPU: the one-GPU guard, the
counter-traffic records being tied to the kernel sources they were taken on,
and the warm-up floor."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line


@pytest.mark.parametrize("key", sorted(bench.TRAFFIC))
def test_traffic_is_null_once_a_source_changes(key, monkeypatch):
    rec = dict(bench.TRAFFIC[key])
    monkeypatch.setitem(bench.TRAFFIC, key, dict(rec, sha256="0" * 64))
    assert bench.traffic_of(key) is None
    monkeypatch.setitem(bench.TRAFFIC, key, rec)
    got = bench.traffic_of(key)
    # the committed figures either match the committed sources or are withheld
    assert got is None or got == rec["read_bytes"] + rec["write_bytes"]


def test_traffic_records_name_existing_sources():
    for rec in bench.TRAFFIC.values():
        for f in rec["sources"]:
            assert os.path.exists(os.path.join(ROOT, "int4_group_quantized_q4_amd", "csrc", f)), f
        assert rec["read_bytes"] > 0 and rec["write_bytes"] > 0


def test_warm_up_runs_at_least_the_steps_and_the_time(monkeypatch):
    monkeypatch.setattr(bench.torch.cuda, "synchronize", lambda *a, **k: None)
    monkeypatch.setattr(bench, "WARMUP_MIN_S", 0.05)
    seen = []
    n = bench.warm_up(lambda i: seen.append(i), 3)
    assert n == len(seen) and n >= 3
    assert seen == list(range(n))
    import time
    t0 = time.perf_counter()
    monkeypatch.setattr(bench, "WARMUP_MIN_S", 0.0)
    assert bench.warm_up(lambda i: None, 7) == 7
    assert time.perf_counter() - t0 < 1.0
