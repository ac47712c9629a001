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


def test_crossover_summary_on_hand_made_timings():
    """Persistent leads at K = 256 (ranges separated), non-persistent from K = 512 on: the
    crossover is 512; medians, not means, decide (one slow outlier per variant)."""
    us = 1e-6
    times = {
        (8192, 8192, 256, 0, 0): [64 * us] * 99 + [500 * us],
        (8192, 8192, 256, 1, 1): [54 * us] * 99 + [500 * us],
        (8192, 8192, 256, 2, 1): [55 * us] * 100,
        (8192, 8192, 512, 0, 0): [80 * us] * 100,
        (8192, 8192, 512, 1, 1): [81 * us] * 100,
        (8192, 8192, 768, 0, 0): [100 * us] * 100,
        (8192, 8192, 768, 1, 1): [100 * us] * 100,
    }
    out = bench.crossover_summary(times, np)
    p256 = out["points"]["K=256"]
    assert p256["fastest"] == "static@g1" and p256["best_persistent"] == "static@g1"
    assert p256["variants"]["nonpersistent"]["median_us"] == 64.0
    assert p256["variants"]["nonpersistent"]["max_us"] == 500.0
    assert p256["nonpersistent_over_best_persistent"] == round(64 / 54, 4)
    assert p256["separated"] is False  # the 500 us outliers overlap the other range
    assert out["persistent_ahead_at_K"] == [256]
    assert out["nonpersistent_ahead_at_K"] == [512, 768]  # a tie counts for non-persistent
    assert out["crossover_K"] == 512
    # persistent ahead at the largest K: no crossover
    times[(8192, 8192, 768, 1, 1)] = [90 * us] * 100
    assert bench.crossover_summary(times, np)["crossover_K"] is None


def test_workloads_match_the_configured_problems():
    """The workload table holds the configured problems: the 256^3 case, the two fp16 K sweeps,
    fp8 8192^3 and the bf16 tail set, with their modes and grid multiples."""
    def probs(wl):
        return bench.problems(wl)[4]
    assert {(m, n, k) for m, n, k, _, _ in probs("small256")} == {(256, 256, 256)}
    p4 = probs("sweep4k")
    assert sorted({k for _, _, k, _, _ in p4}) == list(range(128, 4097, 128))
    assert {(m, n) for m, n, _, _, _ in p4} == {(4096, 4096)} and {md for _, _, _, md, _ in p4} == {0, 1, 2}
    p8 = probs("sweep8k")
    assert sorted({k for _, _, k, _, _ in p8}) == list(range(256, 8193, 256))
    assert {(md, gm) for _, _, _, md, gm in p8} == {(0, 0), (1, 1), (1, 2), (1, 3), (2, 1), (2, 2), (2, 3)}
    assert bench.WORKLOADS["fp8"][1] == "e4m3fn" and {(m, n, k) for m, n, k, _, _ in probs("fp8")} == {(8192,) * 3}
    assert bench.WORKLOADS["tail"][1] == "bf16" and bench.WORKLOADS["tail"][7] == "normal"
    assert {m for m, _, _, _, _ in probs("tail")} == {4000, 6144, 8200}
    assert all(m == n == k for m, n, k, _, _ in probs("tail"))
