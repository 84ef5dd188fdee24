"""Summarise a rocprofv3 results database (rocpd SQLite) as a short Markdown table.

    python -m state_space_model_ssm_amd.rocpd_summary RESULTS.db [--cmd "..."] [--title "..."]

Kernel durations come from the `kernels` view (end - start, ns). When the run
collected counters (`rocprofv3 --pmc ...`), the per-dispatch values of each
counter are averaged per kernel as well.
"""
from __future__ import annotations

import argparse
import sqlite3
import statistics


def _short(name: str, n: int = 96) -> str:
    name = name.replace("\n", " ")
    return name if len(name) <= n else name[: n - 3] + "..."


def kernel_stats(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, end - start from kernels").fetchall()
    agg = {}
    for name, dur in rows:
        agg.setdefault(name, []).append(dur)
    out = []
    for name, d in agg.items():
        d = sorted(d)
        out.append({"name": name, "calls": len(d), "avg_us": statistics.mean(d) / 1e3,
                    "p50_us": d[len(d) // 2] / 1e3, "p99_us": d[min(len(d) - 1, int(0.99 * len(d)))] / 1e3,
                    "min_us": d[0] / 1e3, "max_us": d[-1] / 1e3, "total_us": sum(d) / 1e3})
    return sorted(out, key=lambda r: -r["total_us"])


def counter_stats(db: str):
    con = sqlite3.connect(db)
    try:
        rows = con.execute("select kernel_name, counter_name, value from counters_collection").fetchall()
    except sqlite3.OperationalError:
        return []
    agg = {}
    for k, c, v in rows:
        agg.setdefault((k, c), []).append(v)
    return sorted(({"name": k, "counter": c, "n": len(v), "avg": statistics.mean(v)} for (k, c), v in agg.items()),
                  key=lambda r: -r["avg"])


def traffic(fetch_db: str, write_db: str, calib_kernel: str = "__amd_rocclr_copyBuffer",
            calib_bytes: int = 1 << 30):
    """Calibrated HBM bytes per dispatch from a FETCH_SIZE run and a WRITE_SIZE run.

    Both counters are in KiB per dispatch. Each is scaled by (known bytes / counted
    bytes) of the largest dispatch of a plain copy kernel in the same run, which
    read and wrote `calib_bytes`. Returns ({kernel: {"fetch": B, "write": B}},
    {"fetch_factor": f, "write_factor": w})."""
    out, factors = {}, {}
    for db, ctr, key in ((fetch_db, "FETCH_SIZE", "fetch"), (write_db, "WRITE_SIZE", "write")):
        rows = [r for r in counter_stats(db) if r["counter"] == ctr]
        con = sqlite3.connect(db)
        calib = con.execute("select max(value) from counters_collection where kernel_name = ? and counter_name = ?",
                            (calib_kernel, ctr)).fetchone()[0]
        factor = calib_bytes / (calib * 1024.0) if calib else None
        factors[key + "_factor"] = factor
        for r in rows:
            if factor:
                out.setdefault(r["name"], {})[key] = r["avg"] * 1024.0 * factor
    return out, factors


def render(db: str, title: str = "", cmd: str = "") -> str:
    lines = [f"# {title or 'rocprofv3 summary'}", ""]
    if cmd:
        lines += ["Command:", "", "```", cmd, "```", ""]
    ks = kernel_stats(db)
    if ks:
        lines += ["| kernel | calls | avg us | p50 us | p99 us | min us | max us |", "|---|---|---|---|---|---|---|"]
        for r in ks:
            lines.append(f"| {_short(r['name'])} | {r['calls']} | {r['avg_us']:.1f} | {r['p50_us']:.1f} | "
                         f"{r['p99_us']:.1f} | {r['min_us']:.1f} | {r['max_us']:.1f} |")
        lines.append("")
    cs = counter_stats(db)
    if cs:
        lines += ["| kernel | counter | dispatches | avg per dispatch |", "|---|---|---|---|"]
        for r in cs:
            lines.append(f"| {_short(r['name'])} | {r['counter']} | {r['n']} | {r['avg']:.0f} |")
        lines.append("")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--title", default="")
    ap.add_argument("--cmd", default="")
    ap.add_argument("--write-db", default="", help="with a FETCH_SIZE db as DB: print calibrated traffic")
    a = ap.parse_args()
    if a.write_db:
        t, f = traffic(a.db, a.write_db)
        print(f"calibration: {f}")
        for k, v in sorted(t.items(), key=lambda kv: -sum(kv[1].values())):
            print(f"{_short(k)}: fetch {v.get('fetch', 0) / 1e6:.1f} MB, write {v.get('write', 0) / 1e6:.1f} MB")
        return
    print(render(a.db, a.title, a.cmd))


if __name__ == "__main__":
    main()
