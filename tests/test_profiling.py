"""Host logic of the rocprofv3 summaries (moe_grouped_gemm_scaled_amd.profiling),
on a small SQLite database with the tables and columns rocprofv3 writes.
"""
import json
import sqlite3

import pytest

from moe_grouped_gemm_scaled_amd import profiling

SUFFIX = "_0123abcd"
KERNEL = ("void dg::pipe_kernel<256, 256, 2, 4, 2, 1, true, (dg::Mode)0, false, false, false, false>"
          "(dg::PipeParams)")
CONFIG = ("family=pipe mode=0 tile=256x256x128 waves=2x4 stages=2 kblocks_per_stage=1 deep=1 splits=1 "
          "grid=448")


def make_db(path, dispatches, counters):
    """dispatches: [(event_id, start_ns, end_ns)] of KERNEL on 448 workgroups of 512;
    counters: {name: {event_id: [row values]}}."""
    con = sqlite3.connect(path)
    con.execute(f"create table rocpd_info_kernel_symbol{SUFFIX} (id integer, display_name text)")
    con.execute(f"create table rocpd_kernel_dispatch{SUFFIX} (id integer, event_id integer, kernel_id integer, "
                f"grid_size_x integer, workgroup_size_x integer, start integer, end integer)")
    con.execute(f"create table rocpd_info_pmc{SUFFIX} (id integer, name text)")
    con.execute(f"create table rocpd_pmc_event{SUFFIX} (id integer, event_id integer, pmc_id integer, value real)")
    con.execute(f"insert into rocpd_info_kernel_symbol{SUFFIX} values (1, ?)", (KERNEL,))
    for i, (ev, t0, t1) in enumerate(dispatches):
        con.execute(f"insert into rocpd_kernel_dispatch{SUFFIX} values (?, ?, 1, ?, 512, ?, ?)",
                    (i, ev, 448 * 512, t0, t1))
    rid = 0
    for k, (name, per_event) in enumerate(counters.items()):
        con.execute(f"insert into rocpd_info_pmc{SUFFIX} values (?, ?)", (k, name))
        for ev, vals in per_event.items():
            for v in vals:
                con.execute(f"insert into rocpd_pmc_event{SUFFIX} values (?, ?, ?, ?)", (rid, ev, k, v))
                rid += 1
    con.commit()
    con.close()


def test_per_dispatch_sums_the_rows_of_each_dispatch(tmp_path):
    db = str(tmp_path / "ops.db")
    make_db(db, [(10, 0, 1000), (11, 5000, 7000)],
            {"SQ_INSTS_VALU_MFMA_MOPS_F8": {10: [1.0] * 32, 11: [2.0] * 32}})
    got = profiling.per_dispatch(db, "SQ_INSTS_VALU_MFMA_MOPS_F8")
    assert list(got) == [(KERNEL, 448)]
    assert sorted(got[(KERNEL, 448)]) == [(32.0, 32, 1000.0), (64.0, 32, 2000.0)]


def test_mfma_summary(tmp_path):
    util_db, ops_db = str(tmp_path / "util.db"), str(tmp_path / "ops.db")
    make_db(util_db, [(1, 0, 100_000), (2, 200_000, 300_000)],
            {"MfmaUtil": {1: [40.0], 2: [50.0]}, "LdsUtil": {1: [60.0], 2: [70.0]},
             "LDSBankConflict": {1: [1.0], 2: [3.0]}, "VALUBusy": {1: [20.0], 2: [20.0]}})
    # 100 us dispatches; 240 000 active cycles on each of the 8 XCDs -> 2.4 GHz;
    # FP8 MOPS: 1e6 per row x 32 rows x 512 = 16.384e9 operations
    make_db(ops_db, [(7, 0, 100_000), (8, 500_000, 600_000)],
            {"SQ_INSTS_VALU_MFMA_MOPS_F8": {7: [1e6] * 32, 8: [1e6] * 32},
             "SQ_INSTS_VALU_MFMA_MOPS_F6F4": {7: [0.0] * 32, 8: [0.0] * 32},
             "GRBM_GUI_ACTIVE": {7: [240_000.0] * 8, 8: [240_000.0] * 8}})
    bench = tmp_path / "bench.json"
    flops = 16.384e9
    bench.write_text("noise line\n" + json.dumps({
        "config": {"workload": "w"},
        "per_gemm": [{"name": "job", "config": CONFIG, "gemm_us": 100.0, "gemm_TFLOPs": flops / 100e-6 / 1e12}]}))
    out = profiling.mfma(str(bench), util_db, ops_db)
    rec = out["jobs"]["job"]
    assert rec["MfmaUtil_pct"] == pytest.approx(45.0)
    assert rec["LdsUtil_pct"] == pytest.approx(65.0)
    assert rec["LDSBankConflict_pct"] == pytest.approx(2.0)
    assert rec["VALUBusy_pct"] == pytest.approx(20.0)
    assert rec["mfma_ops_counted_per_launch"] == pytest.approx(16.384e9)
    assert rec["counted_over_algorithmic"] == pytest.approx(1.0)
    assert rec["rows_per_dispatch"] == 8
    assert rec["gui_active_cycles_per_xcd"] == pytest.approx(240_000.0)
    assert rec["clock_ghz"] == pytest.approx(2.4)
    assert out["source_hash"] == profiling.kernel_source_hash()


def test_kernel_fragment_matches_pipe_symbol():
    frag, grid = profiling._kernel_fragment(CONFIG)
    assert frag in KERNEL and grid == 448


def test_kernel_fragment_matches_stream_and_skinny_symbols():
    frag, grid = profiling._kernel_fragment("family=stream rows=64 cols=32 waves=4x1 stages=8 splits=3+ grid=256")
    assert grid == 256 and "void dg::stream_kernel<4, 2, 4, 1, 8>(dg::StreamParams)".find(frag) > 0
    frag, grid = profiling._kernel_fragment("family=stream rows=128 cols=128 waves=2x4 stages=4 splits=4+ grid=256")
    assert "void dg::stream_kernel<8, 8, 2, 4, 4>(dg::StreamParams)".find(frag) > 0
    assert "void dg::stream_kernel<8, 8, 2, 4, 5>(dg::StreamParams)".find(frag) < 0
    frag, grid = profiling._kernel_fragment(
        "family=skinny mode=0 rows=64 cols=96 waves=4x3 ks=1 pd=2 splits=1 grid=256")
    assert "void dg::skinny_kernel<4, 6, 4, 3, 1, 2, (dg::Mode)0>(dg::SkinnyParams)".find(frag) > 0
