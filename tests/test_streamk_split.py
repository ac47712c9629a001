"""CPU check of the stream-K split arithmetic (no GPU).

tests/sk_split_check.cpp calls the kernels' own sk_unit() and sk_owner()
(device_common.h) for every workgroup of a sweep of launch shapes -- tile
counts that the grid divides and does not, fewer tiles than workgroups,
one to 128 k-step pairs per tile, every tail-group count the planner can
choose -- and checks that each k-step pair of each tile is computed exactly
once, that the whole-tile waves follow the static order, that tail work is
balanced to within one pair, that the fix-up's piece ranges agree with the
units the workgroups actually ran, and that partial-tile workspace slots
never collide.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "sk_split_check.cpp")
EXE = os.path.join(ROOT, "_build", "sk_split_check")


def test_streamk_split_covers_every_pair_once():
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    hdr = os.path.join(ROOT, "persistent_tile_scheduling_macro_amd", "csrc", "device_common.h")
    if not os.path.exists(EXE) or os.path.getmtime(EXE) < max(os.path.getmtime(SRC), os.path.getmtime(hdr)):
        subprocess.check_call(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", "--offload-arch=gfx950",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "-Wall", "-Werror", "-Wno-unused-command-line-argument",
                               SRC, "-o", EXE + ".tmp"])
        os.replace(EXE + ".tmp", EXE)
    out = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr
    assert int(out.stdout.split()[1]) > 1000
