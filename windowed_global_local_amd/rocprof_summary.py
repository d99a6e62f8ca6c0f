"""Summaries of rocprofv3 result databases (rocpd SQLite) for this library.

    python -m windowed_global_local_amd.rocprof_summary trace RESULTS_DB
        per-kernel dispatch count and duration statistics (the figures
        rocprofv3 --kernel-trace --stats reports), as a text table.

    python -m windowed_global_local_amd.rocprof_summary traffic \
        --fetch FETCH_DB --write WRITE_DB --copy-bytes B --algo-bytes A \
        --source PATH --out JSON
        HBM traffic of the attention kernel from one --pmc FETCH_SIZE run and
        one --pmc WRITE_SIZE run.  Each counter is scaled by what it reads for
        a reference copy kernel of the same run whose traffic is known exactly
        (B bytes read and B bytes written per dispatch): by default the plain
        elementwise copy that bench.py --calib-bytes B runs (ordinary cached
        loads and stores, like the attention's), or --copy-kernel NAME.  The
        JSON records the sha256 of the kernel source it was measured on, so a
        later edit of the kernel invalidates it.

    python -m windowed_global_local_amd.rocprof_summary counters RESULTS_DB
        per-kernel sums of the SQ / GRBM counters of one --pmc run, with the
        matrix-core busy fraction SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x
        SQ_BUSY_CU_CYCLES), the fraction of those cycles with a VALU
        instruction co-issued, and the shader clock GRBM_GUI_ACTIVE / 8 XCDs
        over the summed dispatch time.
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import sqlite3
import statistics
import sys

ATTN = "hier_attn_kernel"
COPY = "neg_kernel"


def kernel_durations(db: str) -> dict:
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels").fetchall()
    con.close()
    out = collections.defaultdict(list)
    for name, dur in rows:
        out[name].append(dur)
    return out


def trace(db: str) -> str:
    durs = kernel_durations(db)
    total = sum(sum(v) for v in durs.values())
    lines = [f"{'calls':>6} {'total_ms':>10} {'avg_ms':>10} {'min_ms':>10} {'max_ms':>10} {'pct':>6}  kernel"]
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{len(v):6d} {sum(v) / 1e6:10.3f} {statistics.mean(v) / 1e6:10.3f} "
                     f"{min(v) / 1e6:10.3f} {max(v) / 1e6:10.3f} {100 * sum(v) / total:6.2f}  {name[:110]}")
    return "\n".join(lines)


def counter_per_dispatch(db: str, counter: str, kernel_substr: str) -> list:
    con = sqlite3.connect(db)
    rows = con.execute("select dispatch_id, kernel_name, counter_name, value from counters_collection").fetchall()
    con.close()
    per = collections.defaultdict(float)
    for did, kname, cname, val in rows:
        if cname == counter and kernel_substr in kname:
            per[did] += val
    return [per[k] for k in sorted(per)]


def counters(db: str) -> str:
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, counter_name, value, dispatch_id, duration "
                       "from counters_collection").fetchall()
    con.close()
    sums = collections.defaultdict(lambda: collections.defaultdict(float))
    durs = collections.defaultdict(dict)
    for kname, cname, val, did, dur in rows:
        sums[kname][cname] += val
        durs[kname][did] = dur
    lines = []
    for kname in sorted(sums, key=lambda k: -sum(durs[k].values())):
        c = sums[kname]
        d = durs[kname]
        lines.append(f"{kname[:110]}")
        lines.append(f"  dispatches {len(d)}, mean duration {statistics.mean(d.values()) / 1e6:.3f} ms")
        for cname in sorted(c):
            lines.append(f"  {cname:30s} {c[cname]:.4e}")
        busy = c.get("SQ_BUSY_CU_CYCLES")
        mfma = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        if busy and mfma is not None:
            lines.append(f"  MFMA busy fraction             {mfma / (4.0 * busy):.3f}")
            co = c.get("SQ_VALU_MFMA_COEXEC_CYCLES")
            if co is not None and mfma:
                lines.append(f"  VALU co-issued in MFMA cycles  {co / mfma:.3f}")
        gui = c.get("GRBM_GUI_ACTIVE")
        if gui:
            lines.append(f"  shader clock (GHz)             {gui / 8.0 / (sum(d.values()) * 1e-9) / 1e9:.3f}")
    return "\n".join(lines)


def traffic(fetch_db, write_db, copy_bytes, algo_bytes, source, copy_kernel=COPY):
    af = counter_per_dispatch(fetch_db, "FETCH_SIZE", ATTN)
    aw = counter_per_dispatch(write_db, "WRITE_SIZE", ATTN)
    cf = counter_per_dispatch(fetch_db, "FETCH_SIZE", copy_kernel)
    cw = counter_per_dispatch(write_db, "WRITE_SIZE", copy_kernel)
    if not (af and aw and cf and cw):
        raise SystemExit("missing dispatches in the counter databases")
    fetch_kib, write_kib = statistics.mean(af), statistics.mean(aw)
    copy_fetch_kib, copy_write_kib = statistics.mean(cf), statistics.mean(cw)
    fetch_scale = copy_bytes / (copy_fetch_kib * 1024.0)
    write_scale = copy_bytes / (copy_write_kib * 1024.0)
    hbm = fetch_kib * 1024.0 * fetch_scale + write_kib * 1024.0 * write_scale
    with open(source, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    return {
        "kernel": ATTN, "kernel_source": source, "kernel_source_sha256": sha,
        "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
        "copy_kernel_fetch_kib": copy_fetch_kib, "copy_kernel_write_kib": copy_write_kib,
        "copy_kernel": copy_kernel,
        "copy_kernel_known_bytes_each_way": copy_bytes,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "hbm_bytes_per_launch": hbm,
        "algorithmic_bytes_per_launch": algo_bytes,
        "traffic_over_algorithmic": hbm / algo_bytes if algo_bytes else None,
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    k = sub.add_parser("counters")
    k.add_argument("db")
    c = sub.add_parser("traffic")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--copy-bytes", type=float, required=True)
    c.add_argument("--algo-bytes", type=float, required=True)
    c.add_argument("--source", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--copy-kernel", default=COPY)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        print(trace(a.db))
        return 0
    if a.cmd == "counters":
        print(counters(a.db))
        return 0
    res = traffic(a.fetch, a.write, a.copy_bytes, a.algo_bytes, a.source, a.copy_kernel)
    with open(a.out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
