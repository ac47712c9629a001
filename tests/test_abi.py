"""CPU-side checks of the C-ABI library: it loads, exports every entry point
that include/pgemm.h declares, and its host logic (status strings, argument
checks that need no device, the tile order) behaves as documented."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pgemm.h")


@pytest.fixture(scope="module")
def pg():
    import persistent_tile_scheduling_macro_amd as pg
    return pg


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pgemm_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol(pg):
    names = declared_functions()
    assert len(names) >= 12, names
    lib = ctypes.CDLL(pg.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(pg):
    assert pg.pgemm_status_string(0) == "PGEMM_OK"
    assert pg.pgemm_status_string(1) == "PGEMM_ERR_INVALID_ARG"
    assert pg.pgemm_status_string(99) == "PGEMM_ERR_UNKNOWN"


def test_null_handle_is_rejected(pg):
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_run(None, 0, 0, 0, 1, 1, 1, 0, 0, 0)
    assert e.value.status == pg.PGEMM_ERR_INVALID_ARG
    assert pg.pgemm_last_error(None) == "invalid handle"
    pg.pgemm_destroy(None)  # documented no-op


def test_tile_order_row_major_when_group_is_one(pg):
    for n_m, n_n in [(1, 1), (3, 5), (7, 2)]:
        for t in range(n_m * n_n):
            assert pg.pgemm_tile_coords(t, n_m, n_n, 1, 0) == (t // n_n, t % n_n)


@pytest.mark.parametrize("n_m,n_n,g,chunk", [(32, 32, 8, 256), (33, 33, 8, 256), (24, 24, 8, 256),
                                              (16, 64, 4, 256), (5, 7, 3, 0), (16, 16, 8, 256), (1, 9, 8, 8)])
def test_tile_order_is_a_bijection(pg, n_m, n_n, g, chunk):
    seen = set()
    for t in range(n_m * n_n):
        pm, pn = pg.pgemm_tile_coords(t, n_m, n_n, g, chunk)
        assert 0 <= pm < n_m and 0 <= pn < n_n
        seen.add((pm, pn))
    assert len(seen) == n_m * n_n


def test_grouped_order_walks_columns_inside_a_group(pg):
    # group_m = 8 over a 16 x 4 grid, no XCD remap: tiles 0..7 are rows 0..7 of column 0,
    # 8..15 rows 0..7 of column 1, ...; the second group starts at row 8.
    assert [pg.pgemm_tile_coords(t, 16, 4, 8, 0) for t in range(9)] == \
        [(r, 0) for r in range(8)] + [(0, 1)]
    assert pg.pgemm_tile_coords(32, 16, 4, 8, 0) == (8, 0)


def test_xcd_remap_gives_each_xcd_a_compact_block(pg):
    # 32 x 32 tiles, chunks of 256 (the CU count): tile ids t = x (mod 8) run on XCD x;
    # after the remap each XCD's 32 tiles in a chunk form an 8-row x 4-column block.
    for chunk_start in (0, 256):
        for x in range(8):
            coords = [pg.pgemm_tile_coords(chunk_start + x + 8 * j, 32, 32, 8, 256) for j in range(32)]
            rows = {pm for pm, _ in coords}
            cols = {pn for _, pn in coords}
            assert len(rows) == 8 and len(cols) == 4, (x, rows, cols)


def test_tile_coords_rejects_bad_arguments(pg):
    with pytest.raises(pg.PgemmError):
        pg.pgemm_tile_coords(6, 2, 3, 1, 0)
    with pytest.raises(pg.PgemmError):
        pg.pgemm_tile_coords(0, 2, 3, 0, 0)


def test_hold_cus_argument_checks(pg):
    """The benchmark aid rejects out-of-range arguments before touching a
    device, and launches nothing for zero CUs or zero time."""
    for n, us in [(-1, 10), (70000, 10), (4, -1), (4, 2_000_000)]:
        with pytest.raises(pg.PgemmError) as e:
            pg.pgemm_hold_cus(None, 0, n, us)
        assert e.value.status == pg.PGEMM_ERR_INVALID_ARG
    pg.pgemm_hold_cus(None, 0, 0, 100)
    pg.pgemm_hold_cus(None, 0, 8, 0)


def test_cancel_mode_is_accepted_and_unknown_modes_are_not(pg):
    assert pg.PGEMM_SCHED_CANCEL == 3
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_run(None, 0, 0, 0, 1, 1, 1, 0, 3, 0)
    assert e.value.status == pg.PGEMM_ERR_INVALID_ARG  # null handle, not an unknown mode


def test_query_entry_points_reject_a_null_handle(pg):
    """The planning queries need a handle (its CU count); without one they fail cleanly."""
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_query_launch(None, 256, 256, 256, 0, 1, 0)
    assert e.value.status == pg.PGEMM_ERR_INVALID_ARG
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_query_streamk(None, 256, 256, 256, 0, 0)
    assert e.value.status == pg.PGEMM_ERR_INVALID_ARG


def test_streamk_mode_constant_matches_the_header(pg):
    text = open(HEADER).read()
    m = re.search(r"PGEMM_SCHED_STREAMK\s*=\s*(\d+)", text)
    assert m and int(m.group(1)) == pg.PGEMM_SCHED_STREAMK == 4
    assert pg.SCHED_NAMES["streamk"] == 4


def test_tile_trace_argument_checks(pg):
    """The trace entry points reject a null handle or output pointer without a device."""
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_set_tile_trace(None, None)
    assert e.value.status == pg.PGEMM_ERR_INVALID_ARG
    lib = ctypes.CDLL(pg.LIB_PATH)
    lib.pgemm_clock_khz.argtypes = [ctypes.c_int, ctypes.c_void_p]
    assert lib.pgemm_clock_khz(0, None) == pg.PGEMM_ERR_INVALID_ARG


def test_wait_argument_checks(pg):
    """The watchdog wait needs a handle and a non-negative deadline; its status has a name."""
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_wait(None, 10)
    assert e.value.status == pg.PGEMM_ERR_INVALID_ARG
    assert pg.pgemm_status_string(pg.PGEMM_ERR_TIMEOUT) == "PGEMM_ERR_TIMEOUT"
    text = open(HEADER).read()
    m = re.search(r"PGEMM_ERR_TIMEOUT\s*=\s*(\d+)", text)
    assert m and int(m.group(1)) == pg.PGEMM_ERR_TIMEOUT


def test_b_layout_argument_checks(pg):
    """The B-layout setter needs a handle; the layout constants match the header."""
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_set_b_layout(None, pg.PGEMM_B_NK)
    assert e.value.status == pg.PGEMM_ERR_INVALID_ARG
    text = open(HEADER).read()
    for name in ("PGEMM_B_KN", "PGEMM_B_NK"):
        m = re.search(name + r"\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == getattr(pg, name)


def test_mainloop_argument_checks(pg):
    """The wave-schedule setter needs a handle; the schedule constants match the header, and the
    library was built with the producer-wave kernels (the body only the setter selects)."""
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_set_mainloop(None, pg.PGEMM_MAINLOOP_PRODUCER)
    assert e.value.status == pg.PGEMM_ERR_INVALID_ARG
    text = open(HEADER).read()
    for name, val in (("PGEMM_MAINLOOP_AUTO", 0), ("PGEMM_MAINLOOP_LOCKSTEP", 1), ("PGEMM_MAINLOOP_PINGPONG", 2),
                      ("PGEMM_MAINLOOP_PRODUCER", 3)):
        m = re.search(name + r"\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == getattr(pg, name) == val
    path = os.path.join(ROOT, "persistent_tile_scheduling_macro_amd", "_build", "kernel_resources.txt")
    if os.path.exists(path):
        names = {l.split()[0] for l in open(path) if not l.startswith("#")}
        for body in ("gemm_pp_kernel", "gemm_pw_kernel"):
            assert sum(body in n for n in names) == 48, body  # 3 dtypes x 4 modes x traced x B layout


def test_fp8_scales_argument_checks(pg):
    """The fp8 scale setter needs a handle (no device is touched on the failure path)."""
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_set_fp8_scales(None, 1.0, 1.0)
    assert e.value.status == pg.PGEMM_ERR_INVALID_ARG


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_pgemm_build", os.path.join(ROOT, "persistent_tile_scheduling_macro_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


def test_resource_remark_parser_and_trace_flag():
    """The build collects hipcc's per-kernel resource remarks; the parser reads every field and
    tells the tile-trace instantiations (first bool template argument true) from the timed ones."""
    b = _build_module()
    text = "\n".join([
        "./x.h:1:1: remark: Function Name: _ZN5pgemm2pp14gemm_pp_kernelILi0ELi1ELb0ELb1EEEvNS_6ParamsE [-Rpass]",
        "./x.h:1:1: remark:     TotalSGPRs: 101 [-Rpass]", "./x.h:1:1: remark:     VGPRs: 126 [-Rpass]",
        "./x.h:1:1: remark:     AGPRs: 128 [-Rpass]", "./x.h:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass]",
        "./x.h:1:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass]",
        "./x.h:1:1: remark:     LDS Size [bytes/block]: 131072 [-Rpass]",
        "./x.h:1:1: remark: Function Name: _ZN5pgemm4fast16gemm_fast_kernelILi0ELi3ELi0ELb1ELb0EEEvNS_6ParamsE",
        "./x.h:1:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass]"])
    ks = b.parse_resource_remarks(text)
    assert ks[0] == {"name": "_ZN5pgemm2pp14gemm_pp_kernelILi0ELi1ELb0ELb1EEEvNS_6ParamsE", "sgpr": 101, "vgpr": 126,
                     "agpr": 128, "scratch": 0, "occupancy": 2, "lds": 131072}
    assert ks[1]["scratch"] == 12
    assert not b.is_traced(ks[0]["name"]) and b.is_traced(ks[1]["name"])
    assert not b.is_traced("_ZN5pgemm7generic19gemm_generic_kernelILi0ELi1EEEvNS_6ParamsE")
    # the ping-pong and producer-wave bodies' traced instantiations (TRACE is their first bool)
    assert b.is_traced("_ZN5pgemm2pp14gemm_pp_kernelILi0ELi1ELb1ELb0EEEvNS_6ParamsE")
    assert b.is_traced("_ZN5pgemm2pw14gemm_pw_kernelILi2ELi3ELb1ELb1EEEvNS_6ParamsE")
    assert not b.is_traced("_ZN5pgemm2pw14gemm_pw_kernelILi2ELi3ELb0ELb1EEEvNS_6ParamsE")


def test_built_kernels_do_not_spill():
    """Report written by the last build: no kernel that timed runs launch uses scratch memory,
    and every fast kernel fits two waves per SIMD."""
    path = os.path.join(ROOT, "persistent_tile_scheduling_macro_amd", "_build", "kernel_resources.txt")
    if not os.path.exists(path):
        pytest.skip("no build report (run the build first)")
    rows = [l.split() for l in open(path) if not l.startswith("#")]
    assert len(rows) > 100
    for name, vgpr, agpr, sgpr, scratch, occ, lds, traced in rows:
        if traced == "0":
            assert int(scratch) == 0, name
        if "gemm_fast_kernel" in name or "gemm_pp_kernel" in name or "gemm_pw_kernel" in name:
            assert int(occ) >= 2 and int(vgpr) >= 0, name
