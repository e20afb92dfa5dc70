"""CPU checks of bench.py's host logic: it refuses more than one GPU before
touching one, its algorithmic-work formulas (the numerators of the roofline
figures) agree with the oracle's own enumeration of the retained tokens and
with hand-computed closed forms, and the measured-traffic records under
profiles/ are reported only for their workload and current sources."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import retained  # noqa: E402
from rpkv_inputs import WORKLOADS  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, r
    assert "one GPU" in r.stderr and r.stdout == ""


def test_visible_tokens_match_the_oracle_retained_set():
    """bench.visible_tokens (a closed form) against the oracle's explicit
    enumeration of the visible frames, every frame of every workload."""
    for wl in WORKLOADS.values():
        for f in range(wl.frames):
            patch, special = retained.visible_for_schedule(f, wl.keyframe_interval, wl.scale_frames,
                                                           wl.sliding_window)
            want = len(patch) * wl.patches + len(special) * wl.n_special
            assert bench.visible_tokens(wl, f) == want, (wl.name, f)


def test_algorithmic_work_closed_forms():
    # 37x37 single layer at frame 63: 8 scale + 16 window pages + its own,
    # 1369 patches each, and the specials of the 63 keyframes before it and
    # its own: 25 * 1369 + 64 * 6 keys.
    wl = WORKLOADS[1]
    assert bench.visible_tokens(wl, 63) == 25 * 1369 + 64 * 6
    # FLOP per (frame, stream): QK^T and PV, 2 * 2 * H * D * N_q * keys.
    assert bench.attn_flops(wl, 63) == 4.0 * 16 * 64 * 1375 * (25 * 1369 + 64 * 6)
    # Append bytes per stream-frame: Q, K, V read and q_rot, K, V written, bf16.
    assert bench.append_bytes(wl) == 6 * 1375 * 16 * 64 * 2
    # Full depth, frame 255 (keyframe every 2nd frame: 128 stored before it):
    # 8 scale + 32 window + own pages, 129 special groups, 4 streams.
    wl = WORKLOADS[4]
    assert bench.visible_tokens(wl, 255) == 41 * 1369 + 129 * 6
    assert bench.append_bytes(wl) == 4 * 6 * 1375 * 16 * 64 * 2


def test_traffic_record_needs_its_workload_and_current_sources(tmp_path, monkeypatch):
    """A measured-traffic record is reported for its own workload only, and
    only while the sources it names hash as they did when it was taken."""
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_text("kernel, first version")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"workload": "w", "sources": ["k.hip"], "source_sha256_16": bench.source_digest(["k.hip"]),
           "bytes_per_launch": 123}
    (tmp_path / "profiles" / "r.json").write_text(json.dumps(rec))
    assert bench.read_traffic("w", "r.json") == 123
    assert bench.read_traffic("other", "r.json") is None
    assert bench.read_traffic("w", "missing.json") is None
    (tmp_path / "k.hip").write_text("kernel, second version")
    assert bench.read_traffic("w", "r.json") is None
