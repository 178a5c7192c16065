"""Summaries of rocprofv3 output databases (SQLite, rocpd schema) as short text.

    python -m exact_attention_99_amd.rocprof_summary stats DB --cmd "..." --out FILE.md
    python -m exact_attention_99_amd.rocprof_summary traffic --fetch DB --write DB \
        --copy-fetch DB --copy-write DB --copy-bytes N --cmd "..." --out traffic.json
    python -m exact_attention_99_amd.rocprof_summary counters --run LABEL=DB[,DB...] ... \
        --kernel PATTERN --cmd "..." --out FILE.md

`stats` tabulates per-kernel launch counts and durations (from a
`--kernel-trace --stats` run).  `counters` tabulates, for the dispatches of
one kernel family, every counter found in one or more `--pmc` databases per
labelled run (one row per run, values averaged over dispatches).  `traffic` turns FETCH_SIZE and WRITE_SIZE
readings (KiB per dispatch, from two `--pmc` runs) into HBM bytes per launch,
scaled by what the same counters read for a plain copy of known size.
Measurement tooling only; nothing on the library's compute path uses it.
"""
from __future__ import annotations

import argparse
import json
import re
import sqlite3
import sys
from collections import defaultdict


def short_name(name: str) -> str:
    n = re.sub(r"fa355::\(anonymous namespace\)::", "", name)
    n = n.replace("fa355::", "")
    n = re.sub(r"^void ", "", n)
    depth, out = 0, []
    for ch in n:  # drop the argument list
        if ch == "(" and depth == 0 and out and out[-1] not in " <,":
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    n = "".join(out)
    return n if len(n) <= 70 else n[:67] + "..."


def kernel_stats(db: str):
    c = sqlite3.connect(db)
    rows = c.execute("select name, total_calls, total_duration, average, percentage "
                     "from top_kernels order by total_duration desc").fetchall()
    return [(short_name(r[0]), int(r[1]), float(r[2]), float(r[3]), float(r[4])) for r in rows]


def counter_per_kernel(db: str, counter: str):
    c = sqlite3.connect(db)
    acc = defaultdict(list)
    for name, val in c.execute("select kernel_name, value from counters_collection where counter_name = ?",
                               (counter,)):
        acc[short_name(name)].append(float(val))
    return acc


def cmd_stats(a):
    rows = kernel_stats(a.db)
    lines = [f"# rocprofv3 kernel trace: {a.title}", "", "Command:", "", "```", a.cmd, "```", "",
             "| kernel | calls | avg (ms) | total (ms) | % of GPU time |", "|---|---|---|---|---|"]
    for n, calls, tot, avg, pct in rows[: a.top]:
        # the rocpd views report microseconds
        lines.append(f"| `{n}` | {calls} | {avg / 1e3:.3f} | {tot / 1e3:.3f} | {pct:.1f} |")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(a):
    fetch = counter_per_kernel(a.fetch, "FETCH_SIZE")
    write = counter_per_kernel(a.write, "WRITE_SIZE")
    cf = counter_per_kernel(a.copy_fetch, "FETCH_SIZE")
    cw = counter_per_kernel(a.copy_write, "WRITE_SIZE")
    # the calibration copy is the largest-reading elementwise copy dispatch
    copy_f = max(v for vals in cf.values() for v in vals)
    copy_w = max(v for vals in cw.values() for v in vals)
    f_factor = a.copy_bytes / (copy_f * 1024.0)
    w_factor = a.copy_bytes / (copy_w * 1024.0)
    out = {"command": a.cmd, "source_sha": a.sha, "copy_bytes": a.copy_bytes,
           "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
           "fetch_factor": f_factor, "write_factor": w_factor, "kernels": {}}
    # every kernel generation of a pass matches its prefix
    for pat, key in (("fwd16", "fwd"), ("delta16", "bwd_prepare"),
                     ("dkdv16", "bwd_dkdv"), ("dq16", "bwd_dq"),
                     ("fwd8_", "fwd_fp8"), ("quant8_", "fp8_quantize")):
        fk = [v for n, vals in fetch.items() if pat in n for v in vals]
        wk = [v for n, vals in write.items() if pat in n for v in vals]
        if not fk or not wk:
            continue
        f_kib = sum(fk) / len(fk)
        w_kib = sum(wk) / len(wk)
        out["kernels"][key] = {"fetch_kib_per_launch": f_kib, "write_kib_per_launch": w_kib,
                               "hbm_bytes_per_launch": f_kib * 1024 * f_factor + w_kib * 1024 * w_factor}
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def cmd_counters(a):
    rows, names = [], []
    for spec in a.run:
        label, dbs = spec.split("=", 1)
        vals = {}
        kern = None
        for db in dbs.split(","):
            c = sqlite3.connect(db)
            acc = defaultdict(list)
            for name, cn, val in c.execute(
                    "select kernel_name, counter_name, value from counters_collection"):
                n = short_name(name)
                if a.kernel not in n:
                    continue
                kern = n
                acc[cn].append(float(val))
            for cn, v in acc.items():
                vals[cn] = sum(v) / len(v)
                if cn not in names:
                    names.append(cn)
        rows.append((label, kern, vals))
    lines = [f"# rocprofv3 counters: {a.title}", "", "Commands:", "", "```", a.cmd, "```", "",
             "| run | kernel | " + " | ".join(names) + " |", "|---|---|" + "---|" * len(names)]
    for label, kern, vals in rows:
        cells = [f"{vals[n]:.4g}" if n in vals else "" for n in names]
        lines.append(f"| {label} | `{kern}` | " + " | ".join(cells) + " |")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("db")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="")
    s.add_argument("--top", type=int, default=8)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for k in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--cmd", "--out", "--sha"):
        t.add_argument(k, required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    c = sub.add_parser("counters")
    c.add_argument("--run", action="append", required=True)
    c.add_argument("--kernel", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--title", default="")
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[a.what](a)


if __name__ == "__main__":
    sys.exit(main())
