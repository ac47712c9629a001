"""CPU race test of the claim protocol of the claiming schedulers (no GPU).

tests/sched_sim.cpp calls the kernels' own claim_tile() from host threads
standing in for the workgroups: G persistent workgroups that start on tile
w (dynamic), or one per tile, started at staggered times, that claim their
first tile too (cancel-and-reuse). What it must show, whatever the
interleaving:

* every tile is processed exactly once per launch;
* a launch makes exactly T (dynamic) or T + G (cancel-and-reuse) claims, of
  which exactly G fail (each worker's last; KernelWiki "Persistent Kernels
  with Cluster Launch Control", intro: a failed request means that worker
  never requests again);
* the counter reads 0 after every launch (the last claim resets it), so
  launches on one stream need no reset in between;
* a worker that stalls on its first tile does not hold back the rest: the
  others take every remaining tile (the case where the CUs actually
  available differ from the static assumption, same page, "Choosing between
  static and CLC scheduling");
* a counter that does not read 0 at launch (a cut-short launch) is caught:
  a value >= the claim total makes every claim fail, which the tile-visit
  counter exposes as unvisited tiles; a negative one only fails the first
  claims, and the counter is then left non-zero after the launch.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "sched_sim.cpp")
EXE = os.path.join(ROOT, "_build", "sched_sim")


@pytest.fixture(scope="module")
def sim():
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    hdr = os.path.join(ROOT, "persistent_tile_scheduling_macro_amd", "csrc", "device_common.h")
    if not os.path.exists(EXE) or os.path.getmtime(EXE) < max(os.path.getmtime(SRC), os.path.getmtime(hdr)):
        subprocess.check_call(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", "-pthread", "--offload-arch=gfx950",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "-Wall", "-Werror", "-Wno-unused-command-line-argument",
                               SRC, "-o", EXE + ".tmp"])
        os.replace(EXE + ".tmp", EXE)

    def run(scenario, T, G, launches, seed, arg=None, mode="dynamic"):
        cmd = [EXE, scenario, mode, str(T), str(G), str(launches), str(seed)] + ([str(arg)] if arg is not None else [])
        out = subprocess.run(cmd, capture_output=True, text=True, timeout=120, check=True).stdout
        kv = dict(item.split("=") for item in out.split())
        res = {k: int(v) for k, v in kv.items() if k != "counter_after"}
        res["counter_after"] = [int(x) for x in kv["counter_after"].split(",")]
        return res

    return run


@pytest.mark.parametrize("T,G", [(1, 1), (7, 3), (64, 64), (1089, 256), (576, 256), (1024, 97), (300, 1)])
@pytest.mark.parametrize("seed", [1, 2])
def test_exactly_once_and_counter_reset(sim, T, G, seed):
    launches = 3
    r = sim("race", T, G, launches, seed)
    assert r["visits_min"] == launches and r["visits_max"] == launches
    assert r["claims"] == T * launches
    assert r["failed"] == G * launches
    assert r["counter_after"] == [0] * launches


@pytest.mark.parametrize("T", [1, 5, 64, 300, 1089])
@pytest.mark.parametrize("seed", [1, 2])
def test_cancel_and_reuse_exactly_once(sim, T, seed):
    """One worker per tile, claiming its first tile too: T successful claims, one
    failing claim per worker, the counter back at 0 after every launch."""
    launches = 2
    r = sim("race", T, T, launches, seed, mode="cancel")
    assert r["visits_min"] == launches and r["visits_max"] == launches
    assert r["claims"] == 2 * T * launches
    assert r["failed"] == T * launches
    assert r["counter_after"] == [0] * launches


def test_cancel_and_reuse_late_workers_take_nothing(sim):
    """Worker 0 stalls on its first tile; the rest finish every other tile, and
    workers that start late fail their first claim (they never get a tile)."""
    T = 256
    r = sim("stall", T, T, 1, 4, 300, mode="cancel")
    assert r["visits_min"] == 1 and r["visits_max"] == 1
    assert r["worker_tiles_min"] == 0  # some workers found no tile left at their start
    assert r["worker0_tiles"] == 1
    assert r["counter_after"] == [0]


def test_stalled_worker_does_not_hold_back_the_rest(sim):
    T, G = 1024, 64
    r = sim("stall", T, G, 1, 5, 300)
    assert r["visits_min"] == 1 and r["visits_max"] == 1
    # static would leave worker 0 with T/G = 16 tiles behind its stall
    assert r["worker0_tiles"] == 1
    assert r["counter_after"] == [0]


def test_stale_counter_fails_every_claim(sim):
    T, G = 512, 64
    r = sim("corrupt", T, G, 1, 3, 5000)
    # only the first tiles (no claim needed) are done; the visit counter shows the rest missing,
    # and the counter is left non-zero, which the host can read back
    assert r["unvisited"] == T - G
    assert r["failed"] == G and r["claims"] == G
    assert r["counter_after"] == [5000 + G]


def test_negative_counter_only_delays_the_first_claims(sim):
    T, G = 512, 64
    r = sim("corrupt", T, G, 1, 3, -7)
    # 7 claims fail (7 workers stop after their first tile), the other 57 finish every tile
    # exactly once; the counter is left at T - 7 instead of 0 (readable on the host)
    assert r["visits_min"] == 1 and r["visits_max"] == 1
    assert r["failed"] == G
    assert r["counter_after"] == [T - 7]
