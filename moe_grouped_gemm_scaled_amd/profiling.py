"""Summaries of rocprofv3 result databases for this library's kernels.

    python -m moe_grouped_gemm_scaled_amd.profiling stats RESULTS_DB
        Markdown table: per (kernel, workgroups) launch count, mean and median
        duration, from a `rocprofv3 --kernel-trace` run.

    python -m moe_grouped_gemm_scaled_amd.profiling traffic --bench-json B.json \\
            --fetch F.db --write W.db --copy-fetch CF.db --copy-write CW.db --copy-bytes N
        JSON: HBM bytes per GEMM launch of each benchmark job, from one
        `rocprofv3 --pmc FETCH_SIZE` and one `--pmc WRITE_SIZE` run of the
        benchmark, each counter scaled by what it reads for a device copy of
        N bytes (`bench.py --copy-calibration`), plus the hash of the kernel
        sources the counters were taken on.

    python -m moe_grouped_gemm_scaled_amd.profiling mfma --bench-json B.json \\
            --util U.db --ops O.db
        JSON: per GEMM launch of each benchmark job, the matrix-core and LDS
        counters of one `rocprofv3 --pmc MfmaUtil LdsUtil LDSBankConflict
        VALUBusy` run and one `--pmc SQ_INSTS_VALU_MFMA_MOPS_F8
        SQ_INSTS_VALU_MFMA_MOPS_F6F4 GRBM_GUI_ACTIVE` run of the benchmark:
        MFMA-busy, LDS-busy, bank-conflict and VALU-busy percentages, the FP8
        matrix operations counted (MOPS x 512) against the job's algorithmic
        flops, and the GPU clock implied by the active-cycle count over the
        dispatch duration.

The databases are the `*_results.db` files rocprofv3 writes (SQLite); only
the standard library is used to read them.
"""
import argparse
import hashlib
import json
import os
import sqlite3
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["dg_device.h", "dg_internal.h", "dg_pipeline.h", "gemm.hip", "decode.hip", "pipelined.hip", "mqa.hip",
                  "persistent.hip", "quant.hip", "stream.hip", "noalloc.hip"]


def kernel_source_hash():
    """sha256 over the HIP sources of the kernels (counters go stale when it changes)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(HERE, "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def _tables(con):
    names = [r[0] for r in con.execute("select name from sqlite_master where type='table'")]

    def pick(prefix):
        for n in names:
            if n.startswith(prefix):
                return n
        raise KeyError(f"no table {prefix}* in database")
    return pick


def dispatches(db):
    """[(kernel display name, workgroups, duration ns)] in start order."""
    con = sqlite3.connect(db)
    t = _tables(con)
    kd, ks = t("rocpd_kernel_dispatch_"), t("rocpd_info_kernel_symbol_")
    rows = con.execute(f"select s.display_name, d.grid_size_x / d.workgroup_size_x, d.end - d.start "
                       f"from {kd} d join {ks} s on d.kernel_id = s.id order by d.start").fetchall()
    con.close()
    return rows


def counter_values(db, counter):
    """{(kernel display name, workgroups): [counter value per dispatch]}."""
    con = sqlite3.connect(db)
    t = _tables(con)
    kd, ks, pe, ip = (t("rocpd_kernel_dispatch_"), t("rocpd_info_kernel_symbol_"), t("rocpd_pmc_event_"),
                      t("rocpd_info_pmc_"))
    rows = con.execute(f"select s.display_name, d.grid_size_x / d.workgroup_size_x, p.value "
                       f"from {pe} p join {kd} d on p.event_id = d.event_id join {ks} s on d.kernel_id = s.id "
                       f"join {ip} i on p.pmc_id = i.id where i.name = ?", (counter,)).fetchall()
    con.close()
    out = {}
    for name, wg, v in rows:
        out.setdefault((name, int(wg)), []).append(float(v))
    return out


def per_dispatch(db, counter):
    """{(kernel display name, workgroups): [(counter value, rows, duration ns) per dispatch]}: the rows
    of one dispatch (one per hardware instance, for counters reported per shader engine or XCD)
    are summed."""
    con = sqlite3.connect(db)
    t = _tables(con)
    kd, ks, pe, ip = (t("rocpd_kernel_dispatch_"), t("rocpd_info_kernel_symbol_"), t("rocpd_pmc_event_"),
                      t("rocpd_info_pmc_"))
    rows = con.execute(f"select s.display_name, d.grid_size_x / d.workgroup_size_x, d.end - d.start, "
                       f"sum(p.value), count(*) "
                       f"from {pe} p join {kd} d on p.event_id = d.event_id join {ks} s on d.kernel_id = s.id "
                       f"join {ip} i on p.pmc_id = i.id where i.name = ? group by p.event_id", (counter,)).fetchall()
    con.close()
    out = {}
    for name, wg, dur, v, n in rows:
        out.setdefault((name, int(wg)), []).append((float(v), int(n), float(dur)))
    return out


def _job_values(table, frag, grid):
    hits = [v for (n, g), v in table.items() if frag in n and g == grid]
    return hits[0] if len(hits) == 1 else None


def mfma(bench_json, util_db, ops_db):
    with open(bench_json) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    util = {c: per_dispatch(util_db, c) for c in ("MfmaUtil", "LdsUtil", "LDSBankConflict", "VALUBusy")}
    ops = {c: per_dispatch(ops_db, c) for c in ("SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F6F4",
                                                 "GRBM_GUI_ACTIVE")}
    jobs = {}
    for job in bench["per_gemm"]:
        frag, grid = _kernel_fragment(job["config"])
        rec = {}
        for c, table in util.items():
            v = _job_values(table, frag, grid)
            rec[c + "_pct"] = None if v is None else statistics.mean(x for x, _n, _d in v)
        f8 = _job_values(ops["SQ_INSTS_VALU_MFMA_MOPS_F8"], frag, grid)
        f64 = _job_values(ops["SQ_INSTS_VALU_MFMA_MOPS_F6F4"], frag, grid)
        gui = _job_values(ops["GRBM_GUI_ACTIVE"], frag, grid)
        flops = job["gemm_TFLOPs"] * 1e12 * job["gemm_us"] * 1e-6
        rec["algorithmic_flop_per_launch"] = flops
        if f8 is not None and f64 is not None:
            counted = 512.0 * (statistics.mean(x for x, _n, _d in f8) + statistics.mean(x for x, _n, _d in f64))
            rec["mfma_ops_counted_per_launch"] = counted
            rec["counted_over_algorithmic"] = counted / flops if flops else None
        if gui is not None:
            # GRBM_GUI_ACTIVE is reported per XCD (8 rows per dispatch when not aggregated); the clock is
            # the cycles of one XCD over the dispatch duration
            cyc = statistics.mean(x / max(n, 1) for x, n, _d in gui)
            dur = statistics.mean(d for _x, _n, d in gui)
            rec["gui_active_cycles_per_xcd"] = cyc
            rec["rows_per_dispatch"] = gui[0][1]
            rec["dispatch_us_under_counters"] = dur / 1e3
            rec["clock_ghz"] = cyc / dur if dur > 0 else None
        jobs[job["name"]] = rec
    return {"workload": bench["config"]["workload"], "source_hash": kernel_source_hash(), "jobs": jobs}


def stats_table(db, min_calls=1):
    groups = {}
    for name, wg, dur in dispatches(db):
        groups.setdefault((name, int(wg)), []).append(dur)
    lines = ["| kernel | workgroups | launches | mean us | median us | total ms |", "|---|---|---|---|---|---|"]
    for (name, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        if len(v) < min_calls:
            continue
        lines.append(f"| `{name}` | {wg} | {len(v)} | {statistics.mean(v) / 1e3:.2f} | "
                     f"{statistics.median(v) / 1e3:.2f} | {sum(v) / 1e6:.3f} |")
    return "\n".join(lines)


def _kernel_fragment(config):
    """Kernel symbol prefix (template arguments included) and workgroup count
    of a bench job's config string, as printed by the library."""
    kv = dict(tok.split("=", 1) for tok in config.split() if "=" in tok)
    fam, grid = kv["family"], int(kv["grid"])
    if fam in ("pipe", "persist"):
        bm, bn = kv["tile"].split("x")[:2]
        wm, wn = kv["waves"].split("x")
        frag = f"{fam}_kernel<{bm}, {bn}, {wm}, {wn}, {kv['stages']}, {kv['kblocks_per_stage']}, "
    elif fam == "stream":
        wm, wn = kv["waves"].split("x")
        frag = f"stream_kernel<{int(kv['rows']) // 16}, {int(kv['cols']) // 16}, {wm}, {wn}, {kv['stages']}>"
    elif fam == "mqa":
        frag = f"mqa_kernel<{int(kv['heads']) // 16}, "
    elif fam == "skinny":
        wm, wn = kv["waves"].split("x")
        frag = (f"skinny_kernel<{int(kv['rows']) // 16}, {int(kv['cols']) // 16}, {wm}, {wn}, {kv['ks']}, "
                f"{kv['pd']}, ")
    else:
        bm, bn = kv["tile"].split("x")[:2]
        wm, wn = kv["waves"].split("x")
        frag = f"gemm_tiled_kernel<{bm}, {bn}, {wm}, {wn}, "
    return frag, grid


def copy_factor(db, counter, nbytes):
    """Bytes per counter KiB for the largest copy kernel in a calibration run."""
    vals = counter_values(db, counter)
    best = None
    for (name, _wg), v in vals.items():
        if "copy" in name.lower():
            m = statistics.mean(v)
            best = m if best is None else max(best, m)
    if not best:
        raise RuntimeError(f"no copy kernel with {counter} in {db}")
    return nbytes / best


def traffic(bench_json, fetch_db, write_db, copy_fetch_db, copy_write_db, copy_bytes):
    with open(bench_json) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    ff = copy_factor(copy_fetch_db, "FETCH_SIZE", copy_bytes)
    fw = copy_factor(copy_write_db, "WRITE_SIZE", copy_bytes)
    fetch = counter_values(fetch_db, "FETCH_SIZE")
    write = counter_values(write_db, "WRITE_SIZE")
    jobs = {}
    for job in bench["per_gemm"]:
        frag, grid = _kernel_fragment(job["config"])
        fk = [v for (n, g), v in fetch.items() if frag in n and g == grid]
        wk = [v for (n, g), v in write.items() if frag in n and g == grid]
        if len(fk) != 1 or len(wk) != 1:
            jobs[job["name"]] = None          # no or ambiguous match
            continue
        jobs[job["name"]] = {"fetch_bytes": statistics.mean(fk[0]) * ff, "write_bytes": statistics.mean(wk[0]) * fw,
                             "launches_fetch": len(fk[0]), "launches_write": len(wk[0])}
    return {"workload": bench["config"]["workload"], "source_hash": kernel_source_hash(),
            "calibration": {"copy_bytes": copy_bytes, "fetch_bytes_per_counter_unit": ff,
                            "write_bytes_per_counter_unit": fw},
            "jobs": jobs}


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m moe_grouped_gemm_scaled_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("db")
    s.add_argument("--min-calls", type=int, default=1)
    t = sub.add_parser("traffic")
    t.add_argument("--bench-json", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--bench-json", required=True)
    m.add_argument("--util", required=True)
    m.add_argument("--ops", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.db, a.min_calls))
    elif a.cmd == "mfma":
        print(json.dumps(mfma(a.bench_json, a.util, a.ops), indent=1))
    else:
        print(json.dumps(traffic(a.bench_json, a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes),
                         indent=1))


if __name__ == "__main__":
    sys.exit(main())
