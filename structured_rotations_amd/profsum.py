"""Summaries of rocprofv3 output (SQLite result databases) for the kernels here.

    python -m structured_rotations_amd.profsum stats DB [--match SUBSTR]
    python -m structured_rotations_amd.profsum by-kernel DB [--match SUBSTR]
    python -m structured_rotations_amd.profsum traffic --kernel SUBSTR \\
        --fetch DB --write DB --copy-fetch DB --copy-write DB --copy-bytes N \\
        --workload NAME --blk f32 --command "..." --out profiles/traffic_NAME_f32.json

`stats` prints per-kernel launch counts and durations (and the per-dispatch
average of every counter the database holds, over all matching kernels);
`by-kernel` prints those averages per kernel, one column each.  `traffic` turns two counter
runs of a kernel (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) into HBM
bytes per launch, each scaled by what the same counter reads for a plain
device copy of known size, and records it with the hash of that kernel's sources
(build.KERNEL_SOURCES) it was measured on.
"""
from __future__ import annotations

import argparse
import collections
import json
import sqlite3
import sys

from .build import source_hash


def kernel_rows(db: str):
    con = sqlite3.connect(db)
    cols = [r[1] for r in con.execute("pragma table_info(kernels)")]
    return [dict(zip(cols, r)) for r in con.execute("select * from kernels")]


def kernel_stats(db: str, match: str = ""):
    """{(kernel name, grid, LDS bytes): dict(n, mean_us, min_us, max_us, grid, block, lds, vgpr)}; launches
    of one kernel with different launch shapes (e.g. the passes of a rotation) are kept apart."""
    agg = collections.OrderedDict()
    for r in kernel_rows(db):
        name = r["name"]
        if match and match not in name:
            continue
        dur = (r["end"] - r["start"]) / 1e3
        key = (name, r.get("grid_x"), r.get("lds_size"))
        a = agg.setdefault(key, {"durs": [], "grid": r.get("grid_x"), "block": r.get("workgroup_x"),
                                 "lds": r.get("lds_size"), "vgpr": r.get("vgpr_count")})
        a["durs"].append(dur)
    out = {}
    for name, a in agg.items():
        d = a.pop("durs")
        out[name] = dict(n=len(d), mean_us=sum(d) / len(d), min_us=min(d), max_us=max(d), **a)
    return out


def counters(db: str, match: str):
    """Per-dispatch average of every counter recorded for kernels containing `match`."""
    con = sqlite3.connect(db)
    tot = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    for name, d, cn, cv in con.execute("select name, dispatch_id, counter_name, counter_value from pmc_events"):
        if match in name:
            tot[cn] += cv
            disp[cn].add(d)
    return {k: tot[k] / len(disp[k]) for k in tot}


def counters_by_kernel(db: str, match: str):
    """{kernel name: {counter: per-dispatch average}} for kernels containing `match`."""
    con = sqlite3.connect(db)
    tot = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(lambda: collections.defaultdict(set))
    for name, d, cn, cv in con.execute("select name, dispatch_id, counter_name, counter_value from pmc_events"):
        if match in name:
            tot[name][cn] += cv
            disp[name][cn].add(d)
    return {n: {k: tot[n][k] / len(disp[n][k]) for k in tot[n]} for n in tot}


def cmd_by_kernel(args) -> int:
    per = counters_by_kernel(args.db, args.match)
    names = sorted(per)
    cnames = sorted({c for n in names for c in per[n]})
    for i, n in enumerate(names):
        print(f"- k{i}: `{n}`")
    print()
    print("| counter | " + " | ".join(f"k{i}" for i in range(len(names))) + " |")
    print("|---|" + "---|" * len(names))
    for c in cnames:
        print(f"| {c} | " + " | ".join(f"{per[n].get(c, float('nan')):,.0f}" for n in names) + " |")
    return 0


def cmd_stats(args) -> int:
    st = kernel_stats(args.db, args.match)
    print("| kernel | launches | mean us | min us | max us | grid (threads) | block | LDS B |")
    print("|---|---|---|---|---|---|---|---|")
    for (name, _, _), s in sorted(st.items(), key=lambda kv: -kv[1]["mean_us"] * kv[1]["n"]):
        print(f"| `{name[:110]}` | {s['n']} | {s['mean_us']:.2f} | {s['min_us']:.2f} | {s['max_us']:.2f} | "
              f"{s['grid']} | {s['block']} | {s['lds']} |")
    try:
        c = counters(args.db, args.match or "")
    except sqlite3.OperationalError:
        c = {}
    for k, v in sorted(c.items()):
        print(f"counter {k}: {v:.1f} per dispatch")
    return 0


def cmd_traffic(args) -> int:
    fetch = counters(args.fetch, args.kernel)["FETCH_SIZE"]
    write = counters(args.write, args.kernel)["WRITE_SIZE"]
    cf = counters(args.copy_fetch, args.copy_kernel)["FETCH_SIZE"]
    cw = counters(args.copy_write, args.copy_kernel)["WRITE_SIZE"]
    kib = args.copy_bytes / 1024.0
    f_read, f_write = cf / kib, cw / kib
    traffic = fetch * 1024.0 / f_read + write * 1024.0 / f_write
    rec = {
        "workload": args.workload, "blk": args.blk, "kernel": args.kernel, "kernel_hash": source_hash(args.kernel),
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
        "copy_bytes_each_way": args.copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
        "scale_read": f_read, "scale_write": f_write,
        "bytes_per_launch": round(traffic), "command": args.command,
    }
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m structured_rotations_amd.profsum")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("db")
    s.add_argument("--match", default="")
    k = sub.add_parser("by-kernel")
    k.add_argument("db")
    k.add_argument("--match", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-kernel", default="copyBuffer")
    for k in ("fetch", "write", "copy-fetch", "copy-write"):
        t.add_argument("--" + k, required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--blk", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    return {"stats": cmd_stats, "by-kernel": cmd_by_kernel, "traffic": cmd_traffic}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
