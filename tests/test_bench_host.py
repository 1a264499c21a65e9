"""Host logic of bench.py (no GPU): committed counter results are reported
only for the kernel they were taken on, and only while its source is the one
they were taken from; the fused kernel's name follows the library's choice."""
import hashlib
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _fake_tree(tmp_path, source_text: bytes, recorded: bytes, kernel="k_transition_ws"):
    csrc = tmp_path / "padding_free_pair_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_bytes(source_text)
    prof = tmp_path / "profiles"
    prof.mkdir()
    entry = {"kernel": kernel, "source": "k.hip",
             "source_sha256": hashlib.sha256(recorded).hexdigest(),
             "bytes_per_launch": 123.0, "mfma_busy_frac": 0.5}
    (prof / "traffic.json").write_text(json.dumps({"k_transition_ws:wl": entry}))


def test_counters_match_source(tmp_path, monkeypatch):
    _fake_tree(tmp_path, b"kernel v1", b"kernel v1")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for("k_transition_ws:wl") == 123.0
    assert bench.counters_for("k_transition_ws:wl")["mfma_busy_frac"] == 0.5


def test_counters_dropped_when_source_changed(tmp_path, monkeypatch):
    _fake_tree(tmp_path, b"kernel v2", b"kernel v1")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for("k_transition_ws:wl") is None
    assert bench.counters_for("k_transition_ws:wl") == {}


def test_counters_dropped_for_another_kernel(tmp_path, monkeypatch):
    # an entry recorded for one kernel is never reported under another's key
    _fake_tree(tmp_path, b"kernel v1", b"kernel v1", kernel="k_transition_p32")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for("k_transition_ws:wl") is None
    assert bench.traffic_for("k_transition_ws:other") is None


def test_no_counter_file(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for("k_transition_ws:wl") is None


@pytest.mark.parametrize("c_z,hidden,dtype,want", [
    (128, 512, "bf16", "k_transition_ws"),
    (64, 128, "bf16", "k_transition_p32"),
    (128, 512, "f32", "fused"),
])
def test_transition_kernel_id(c_z, hidden, dtype, want):
    assert bench.transition_kernel_id(c_z, hidden, dtype) == want


def test_committed_counters_are_current():
    """The committed counters of the roofline kernel match its source, so the
    bench line carries them. After a change to the kernel they are stale
    until retaken on a GPU: the test then skips and says so."""
    key = f"k_transition_ws:{bench.HEADLINE}"
    c = bench.counters_for(key)
    if not c:
        pytest.skip("counters in profiles/traffic.json were taken on another kernel source")
    assert c.get("bytes_per_launch", 0) > 0
    assert 0 < c.get("mfma_busy_frac", 0) <= 1
