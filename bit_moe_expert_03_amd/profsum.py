"""Summaries of rocprofv3 output for the profiles/ folder.

* ``trace``: per-kernel duration statistics from the SQLite database that
  ``rocprofv3 --kernel-trace`` writes (its ``kernels`` view), as a markdown
  table under the command that produced it.
* ``traffic``: HBM bytes per dispatch of chosen kernels from two counter
  passes (``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``, CSV output), each
  scaled by what the same counter reads for a plain copy kernel of known
  size in the same run.  Written as JSON together with a hash of the source
  files each kernel is built from, so that bench.py can report the traffic
  only while those sources are unchanged.

Usage (from the repository root):
    python -m bit_moe_expert_03_amd.profsum trace DB --cmd "..." --title "..."
    python -m bit_moe_expert_03_amd.profsum traffic --fetch DIR --write DIR \\
        --copy-kernel SUBSTRING --copy-bytes N --kernel NAME=SRC[,SRC...] ... --out FILE.json [--merge]
  NAME: KEY or KEY@MATCH; MATCH (default KEY) is a substring of exactly one
  "kernel [grid N]" name (N workgroups), so a kernel launched with several
  grids needs its grid in MATCH; KEY names the entry in the JSON.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def source_hash(paths) -> str:
    """sha256 over the given files (paths relative to the repository root)."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(p.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def trace_rows(db_path):
    """(name, calls, avg_us, min_us, max_us, total_us) per kernel and launch
    shape, by total time.  A kernel launched with several grid shapes (the
    decode kernels at T = 1 and at few-token batches) gets one row per shape,
    its name suffixed with the grid in workgroups."""
    con = sqlite3.connect(db_path)
    rows = con.execute("select name, grid_x, grid_y, grid_z, workgroup_x, workgroup_y, workgroup_z, count(*), "
                       "avg(duration), min(duration), max(duration), sum(duration) "
                       "from kernels group by name, grid_x, grid_y, grid_z, workgroup_x, workgroup_y, workgroup_z "
                       "order by sum(duration) desc").fetchall()
    con.close()
    shapes = collections.Counter(r[0] for r in rows)
    out = []
    for r in rows:
        name = r[0]
        if shapes[name] > 1:
            g = [max(1, r[i] // max(1, r[i + 3])) for i in (1, 2, 3)]
            name = f"{short_name(name)} [grid {g[0]}x{g[1]}x{g[2]}]"
        out.append((name, r[7], r[8] / 1e3, r[9] / 1e3, r[10] / 1e3, r[11] / 1e3))
    return out


def short_name(name: str) -> str:
    n = name.split("(")[0]
    return n.replace("void ", "")


def counter_means(csv_dir, counter):
    """Mean value of one counter per dispatch, per kernel and launch shape
    (short name + " [grid N]", N workgroups).  A counter reported per hardware
    instance is summed over instances first."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {csv_dir}")
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                wg = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
                key = f"{short_name(r['Kernel_Name'])} [grid {wg}]"
                per[key][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def cmd_trace(a):
    rows = trace_rows(a.db)
    print(f"# {a.title}\n")
    print("Command (repository root, one MI355X):\n")
    print(f"    {a.cmd}\n")
    print("Per-kernel dispatch durations from the `kernels` view of the database that command writes.\n")
    print("| kernel | calls | avg us | min us | max us | total us |")
    print("|---|---|---|---|---|---|")
    for name, n, avg, mn, mx, tot in rows:
        label = name if "[grid" in name else short_name(name)
        print(f"| `{label[:110]}` | {n} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {tot:.1f} |")


def cmd_traffic(a):
    fetch = counter_means(a.fetch, "FETCH_SIZE")
    write = counter_means(a.write, "WRITE_SIZE")

    def pick(table, sub):
        hits = [k for k in table if sub in k]
        if len(hits) != 1:
            raise SystemExit(f"{len(hits)} kernels match {sub!r} (name [grid N] must be unique); have {sorted(table)}")
        return table[hits[0]], hits[0]

    cf, cname = pick(fetch, a.copy_kernel)
    cw, _ = pick(write, a.copy_kernel)
    fscale = a.copy_bytes / (cf * 1024.0)
    wscale = a.copy_bytes / (cw * 1024.0)
    out = {"copy_kernel": cname, "copy_bytes": a.copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": fscale, "write_scale": wscale, "kernels": {}}
    if a.merge and os.path.exists(a.out):
        # keep the rows of an earlier run (each carries its own scales); rows
        # named again here are replaced
        with open(a.out) as fh:
            old = json.load(fh)
        for key, row in old.get("kernels", {}).items():
            row.setdefault("fetch_scale", old.get("fetch_scale"))
            row.setdefault("write_scale", old.get("write_scale"))
            out["kernels"][key] = row
    for spec in a.kernel:
        name, srcs = spec.split("=", 1)
        srcs = srcs.split(",")
        key, _, match = name.partition("@")
        f, full = pick(fetch, match or key)
        w, _ = pick(write, match or key)
        out["kernels"][key] = {"matched": full, "fetch_kib": f, "write_kib": w,
                                "fetch_scale": fscale, "write_scale": wscale,
                                "fetch_bytes": f * 1024.0 * fscale, "write_bytes": w * 1024.0 * wscale,
                                "traffic_bytes": f * 1024.0 * fscale + w * 1024.0 * wscale,
                                "sources": srcs, "source_sha256": source_hash(srcs)}
    with open(a.out, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--cmd", required=True)
    t.add_argument("--title", required=True)
    f = sub.add_parser("traffic")
    f.add_argument("--fetch", required=True)
    f.add_argument("--write", required=True)
    f.add_argument("--copy-kernel", required=True)
    f.add_argument("--copy-bytes", type=int, required=True)
    f.add_argument("--kernel", action="append", required=True)
    f.add_argument("--out", required=True)
    f.add_argument("--merge", action="store_true", help="keep the rows already in --out that are not named here")
    a = ap.parse_args(argv)
    {"trace": cmd_trace, "traffic": cmd_traffic}[a.what](a)


if __name__ == "__main__":
    sys.exit(main())
