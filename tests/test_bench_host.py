"""bench.py host logic: the one-GPU refusal and the HBM traffic records.

The traffic figure in a bench line comes from committed rocprofv3 counter
passes; it is only reported while the kernel source it was measured on is
unchanged.  These tests pin that the committed records match the current
kernel sources (so the default bench line carries a measured figure) and
that a changed source or an unknown workload gives null.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(args, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _records():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        return json.load(f)


def _kind(key):
    """The kernel a traffic record measures, from its key."""
    if key.startswith("fixed|"):
        return "fixed"
    return {"|L=2": "decode2_kernel", "|L=3": "decode3_kernel"}.get(key[-4:], "decode_kernel")


def test_committed_traffic_records_match_the_kernel_sources():
    rec = _records()
    assert rec["workloads"], "no traffic records"
    for key, w in rec["workloads"].items():
        kind = _kind(key)
        assert w["kernel_source_sha256"] == bench.kernel_source_sha256(kind), key
        assert bench.measured_traffic(key, kind) == w["traffic_bytes"]
        # counters close to the algorithmic bytes: nothing re-read.  A
        # workload of a few MB (config 1, 3.5 MB) also fetches its record's
        # table image once into each XCD's L2 (8 x 80 KiB in layout 3), which
        # the algorithmic bytes do not count
        bound = 1.03 if w["alg_bytes"] >= 64 << 20 else 1.3
        assert 1.0 <= w["traffic_bytes"] / w["alg_bytes"] < bound, key
        assert w["traffic_bytes"] == w["fetch_bytes"] + w["write_bytes"]


def test_traffic_keys_name_the_layout():
    for key in _records()["workloads"]:
        assert key.startswith("fixed|") or key.endswith(("|L=1", "|L=2", "|L=3")), key


def test_unknown_workload_or_changed_source_gives_null(monkeypatch):
    assert bench.measured_traffic("no such workload") is None
    key = next(iter(_records()["workloads"]))
    kind = _kind(key)
    assert bench.measured_traffic(key, kind) is not None
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda kind: "0" * 64)
    assert bench.measured_traffic(key, kind) is None


def test_copy_calibration_scales():
    rec = _records()
    # a plain copy reads back half its bytes in FETCH_SIZE and all of them in WRITE_SIZE
    assert rec["fetch_scale"] == pytest.approx(2.0, abs=0.01)
    assert rec["write_scale"] == pytest.approx(1.0, abs=0.01)


def test_default_workload_has_a_traffic_record():
    """The default bench line (the 84-layer checkpoint in layout 3, chunks of
    32,768 weights over 128 lanes in one stream) reports a measured traffic
    figure."""
    from lossless_entropy_coding_amd import synth
    key = f"cfg5_checkpoint_84layers_{len(synth.cfg5_layout(layers=84))}tensors|W=32768|K=128|P=128|L=3"
    assert bench.measured_traffic(key, "decode3_kernel") is not None, key
