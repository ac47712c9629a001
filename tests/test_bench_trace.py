"""CPU checks of the benchmark's host logic: the tail measure on hand-made tile
traces, the custom-workload flags, and the one-GPU rule."""
import json
import os
import subprocess
import sys

import numpy as np

import bench


def test_drain_starts_when_the_first_slot_runs_dry():
    # 4 slots: workgroup 0 runs three back-to-back tiles of 10, the others two; starts staggered
    st, en = [], []
    for w in range(4):
        t = w
        for _ in range(3 if w == 0 else 2):
            st.append(t)
            en.append(t + 10)
            t += 10
    st, en = np.array(st), np.array(en)
    # full from t=3; workgroup 1 ends its last tile at 21 and nothing replaces it
    assert bench.drain_start(st, en, 4, np) == 21


def test_drain_with_no_events_inside_a_wave():
    # two aligned waves of 3 slots and a third partial one: full until the second wave ends
    st = np.array([0, 0, 0, 100, 100, 100, 200])
    en = np.array([100, 100, 100, 200, 200, 200, 300])
    assert bench.drain_start(st, en, 3, np) == 200
    assert bench.drain_start(st, en, 4, np) == 0  # never full: the drain is the whole run


def test_custom_workload_from_flags(monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--workload", "custom", "--prec", "bf16", "--M", "1000",
                                     "--N", "2048", "--K-range", "256", "768", "--K-step", "256",
                                     "--modes", "0,1", "--grid-multiples", "1,2"])
    args = bench.parse()
    bench.add_custom_workload(args)
    desc, dtype, kind, wid, probs = bench.problems("custom")
    assert dtype == "bf16" and kind == "uniform"
    # the non-persistent mode ignores grid multiples; the persistent ones run each
    assert probs == [(1000, 2048, K, m, g) for K in (256, 512, 768) for m, g in ((0, 0), (1, 1), (1, 2))]


def test_more_than_one_gpu_is_refused_with_a_message():
    """The benchmark runs on one GPU; --gpus above 1 exits (status 2) with a JSON message,
    before anything touches a device."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=root, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] and msg["n_gpus_requested"] == 2


def test_vendor_flag_parses(monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--workload", "fp8", "--b-layout", "nk", "--vendor"])
    args = bench.parse()
    assert args.vendor and args.b_layout == "nk"
    monkeypatch.setattr("sys.argv", ["bench.py"])
    assert not bench.parse().vendor
