"""Summaries of rocprofv3 output for the roofline report (measurement harness).

Two subcommands, both reading CSV files that rocprofv3 wrote
(``--output-format csv``); neither touches the GPU.

  trace  --csv <..._kernel_trace.csv> --command "<profiled command>"
         [--ladder <ladder.jsonl>]
         Per (kernel, grid, workgroup) launch counts and durations; with
         --ladder, per ladder record (dispatches between its marker and the
         next), so that workloads sharing a grid stay apart.  The
         trace is used instead of rocprofv3's own stats file because one
         template instance can serve several workloads with different grids.

  pmc    --run <ladder.jsonl>:<..._counter_collection.csv> [--run ...]
         --command "<command of run 1>" [--command ...]
         [--traffic-out profiles/traffic.json]
         Joins each counter run's dispatches of this library's kernels with
         the ladder tool's records: the ladder launches a marker (a 3-float
         fill, kernel stream_tail<1>) before each record, and every dispatch
         up to the next marker belongs to that record (one rep, no warm-up;
         a product may take several launches).  Counters are summed per
         record.  The streaming copy
         probe that the ladder runs first (``--copy-mib``) moves a known
         number of bytes each way; FETCH_SIZE and WRITE_SIZE (L2 to fabric
         traffic, which includes Infinity-Cache hits) and the DRAM-bound
         request counts TCC_EA0_RDREQ_DRAM and TCC_EA0_WRREQ_DRAM are each
         scaled by known / counted on that probe to give bytes per launch.
         With ``--traffic-out`` the production kernels' calibrated bytes are
         written for the benchmark, stamped with a digest of the kernel
         source so that a changed kernel reports no stale traffic.

  clock  --counters <..._counter_collection.csv> --trace <..._kernel_trace.csv>
         --command "<profiled command>"
         The engine clock under each kernel's own load: GRBM_GUI_ACTIVE
         (busy cycles, summed over the XCDs) divided by the number of XCDs
         and by the dispatch's duration from the kernel trace of the same
         run (joined on the dispatch id), per kernel and grid.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
import sys
from collections import OrderedDict, defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
# Sources that define the production kernel's code.
PROD_SOURCES = [os.path.join(HERE, "csrc", n)
                for n in ("prod.hip", "w16_tiles.hpp", "w16_vgpr.hip", "addr_math.hpp", "host_plan.cpp", "host_plan.hpp")]
# Kernels of this library: everything in its namespace, plus the probes
# (file-local kernels of probes.hip), matched on the raw kernel name.
OUR_NAMESPACE = "gemm_f32_impl"
OUR_PROBES = re.compile(r"\b(stream_kernel|stream_tail|mfma_probe_kernel|valu_probe_kernel|"
                        r"lds_probe_kernel|fused_probe_kernel)\b")


def is_ours(raw_name: str) -> bool:
    return OUR_NAMESPACE in raw_name or OUR_PROBES.search(raw_name) is not None


def code_only(text: str) -> str:
    """Source text without comments, trailing blanks or empty lines: what
    the compiler sees.  (These sources hold no comment markers inside string
    literals.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def prod_source_digest() -> str:
    """Digest of the production kernel's code (comments excluded, so a
    changed comment keeps the measured traffic), stamped on measured traffic."""
    h = hashlib.sha256()
    for path in PROD_SOURCES:
        with open(path, encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    s = name.replace("gemm_f32_impl::", "").replace("(anonymous namespace)::", "")
    s = re.sub(r"\(.*\)$", "", s).replace("void ", "")
    return s.strip()


def _workgroups(row) -> int:
    n = 1
    for d in ("X", "Y", "Z"):
        n *= max(1, int(row[f"Grid_Size_{d}"]) // max(1, int(row[f"Workgroup_Size_{d}"])))
    return n


def _threads(row) -> int:
    return int(row["Workgroup_Size_X"]) * int(row["Workgroup_Size_Y"]) * int(row["Workgroup_Size_Z"])


def _trace_rows(paths):
    rows = []
    for path in paths:
        with open(path, newline="") as f:
            rows += list(csv.DictReader(f))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return rows


def cmd_trace(args) -> int:
    rows = _trace_rows(args.csv)
    lines = [f"# {args.title}", "", "Command:", "", "```", *args.command, "```", ""]
    if args.ladder:
        # One block per ladder record: the dispatches between its marker and
        # the next (warm-up and timed calls), per kernel and grid.
        recs = _read_ladder(args.ladder)
        segs, cur = [], None
        for r in rows:
            name = short_name(r["Kernel_Name"])
            if name == MARKER:
                cur = OrderedDict()
                segs.append(cur)
                continue
            if cur is None or (args.only_ours and not is_ours(r["Kernel_Name"])):
                continue
            key = (name, _workgroups(r), _threads(r))
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            cur.setdefault(key, []).append(dur)
        if len(segs) != len(recs):
            raise SystemExit(f"{len(recs)} ladder records but {len(segs)} marked segments")
        lines += ["| workload | record | kernel | workgroups | threads/WG | calls | avg us | median us "
                  "| min us | max us |",
                  "|---|---|---|---|---|---|---|---|---|---|"]
        for rec, seg in zip(recs, segs):
            for (name, wgs, wg), durs in seg.items():
                lines.append(f"| {rec.get('workload', '-')} | {rec.get('kernel', '-')} | `{name}` | {wgs} "
                             f"| {wg} | {len(durs)} | {statistics.mean(durs):.1f} "
                             f"| {statistics.median(durs):.1f} | {min(durs):.1f} | {max(durs):.1f} |")
    else:
        groups: dict = OrderedDict()
        for r in rows:
            if args.only_ours and not is_ours(r["Kernel_Name"]):
                continue
            key = (short_name(r["Kernel_Name"]), _workgroups(r), _threads(r))
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            groups.setdefault(key, []).append(dur)
        lines += ["| kernel | workgroups | threads/WG | calls | avg us | median us | min us | max us |",
                  "|---|---|---|---|---|---|---|---|"]
        for (name, wgs, wg), durs in groups.items():
            lines.append(f"| `{name}` | {wgs} | {wg} | {len(durs)} | {statistics.mean(durs):.1f} "
                         f"| {statistics.median(durs):.1f} | {min(durs):.1f} | {max(durs):.1f} |")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)
    return 0


MARKER = "stream_tail<1>"
DRAM_RD = "TCC_EA0_RDREQ_DRAM_sum"
DRAM_WR = "TCC_EA0_WRREQ_DRAM_sum"


def _compulsory(rec) -> int:
    """4 (MK + KN + MN) bytes (2-byte inputs for the 16-bit rungs), from the
    record's workload; 0 when it names none."""
    try:
        from gemm_inputs import WORKLOADS
    except ImportError:
        sys.path.insert(0, os.path.dirname(HERE))
        from gemm_inputs import WORKLOADS
    w = WORKLOADS.get(rec.get("workload", ""))
    if w is None:
        return 0
    elem = 2 if rec.get("variant") in ("bf16", "f16") else 4
    return elem * (w.M * w.K + w.K * w.N) + 4 * w.M * w.N


def cmd_clock(args) -> int:
    """Engine clock per kernel under its own load: GRBM_GUI_ACTIVE per XCD
    over the dispatch's duration."""
    active = defaultdict(float)
    meta = {}
    with open(args.counters, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != "GRBM_GUI_ACTIVE" or not is_ours(row["Kernel_Name"]):
                continue
            did = int(row["Dispatch_Id"])
            active[did] += float(row["Counter_Value"])
            meta[did] = short_name(row["Kernel_Name"])
    dur = {}
    for r in _trace_rows([args.trace]):
        did = int(r["Dispatch_Id"])
        if did in active:
            dur[did] = ((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0,
                        _workgroups(r))
    groups: dict = OrderedDict()
    for did in sorted(active):
        if did not in dur:
            continue
        us, wgs = dur[did]
        if us <= 0:
            continue
        mhz = active[did] / args.xcds / us
        groups.setdefault((meta[did], wgs), []).append((us, mhz))
    lines = [f"# {args.title}", "", "Command:", "", "```", *args.command, "```", "",
             f"Clock = GRBM_GUI_ACTIVE / {args.xcds} XCDs / dispatch duration (same run, joined on "
             "the dispatch id). Medians over the dispatches of each kernel and grid.", "",
             "| kernel | workgroups | dispatches | median us | median MHz | min MHz | max MHz |",
             "|---|---|---|---|---|---|---|"]
    for (name, wgs), vals in groups.items():
        if len(vals) < args.min_dispatches:
            continue
        us = statistics.median(v[0] for v in vals)
        mhz = [v[1] for v in vals]
        lines.append(f"| `{name}` | {wgs} | {len(vals)} | {us:.1f} | {statistics.median(mhz):.0f} "
                     f"| {min(mhz):.0f} | {max(mhz):.0f} |")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)
    return 0


def _segments(dispatches):
    """Split dispatches at marker launches; each segment sums its counters."""
    segs = []
    for d in dispatches:
        if d["name"] == MARKER:
            segs.append({"name": None, "grid": 0, "counters": defaultdict(float), "kernels": []})
            continue
        if not segs:
            raise SystemExit("counter run starts without a marker dispatch")
        seg = segs[-1]
        seg["kernels"].append(d["name"])
        seg["name"] = seg["name"] or d["name"]
        seg["grid"] += d["grid"]
        for k, v in d["counters"].items():
            seg["counters"][k] += v
    return segs


def _read_counter_csv(path: str):
    """Dispatches of this library's kernels, in dispatch order: list of
    (kernel short name, grid threads, {counter: value})."""
    by_dispatch: dict = OrderedDict()
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            if not is_ours(name):
                continue
            did = int(row["Dispatch_Id"])
            ent = by_dispatch.setdefault(did, {"name": short_name(name), "grid": int(row["Grid_Size"]),
                                               "counters": defaultdict(float)})
            ent["counters"][row["Counter_Name"]] += float(row["Counter_Value"])
    return [by_dispatch[k] for k in sorted(by_dispatch)]


def _read_ladder(path: str):
    recs = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                recs.append(json.loads(line))
    return recs


def cmd_pmc(args) -> int:
    joined = []  # per record: merged counters over runs
    for run in args.run:
        jl, cs = run.split(":", 1)
        recs = _read_ladder(jl)
        disp = _segments(_read_counter_csv(cs))
        if len(recs) != len(disp):
            raise SystemExit(f"{run}: {len(recs)} ladder records but {len(disp)} marked segments")
        for i, (r, d) in enumerate(zip(recs, disp)):
            if i >= len(joined):
                joined.append({"rec": r, "name": d["name"], "grid": d["grid"], "counters": {},
                               "kernels": d["kernels"]})
            elif joined[i]["rec"].get("kernel") != r.get("kernel"):
                raise SystemExit(f"{run}: record {i} is {r.get('kernel')} in one run and "
                                 f"{joined[i]['rec'].get('kernel')} in another")
            joined[i]["counters"].update(d["counters"])

    # known / counted on the copy probe: KiB per KiB for FETCH_SIZE and
    # WRITE_SIZE, bytes per request for the DRAM request counts
    cal = {}
    for j in joined:
        if j["rec"].get("kernel") == "probe_copy":
            kib = j["rec"]["bytes_read"] / 1024.0
            for cname in ("FETCH_SIZE", "WRITE_SIZE"):
                if cname in j["counters"] and j["counters"][cname] > 0:
                    cal[cname] = kib / j["counters"][cname]
            for cname in (DRAM_RD, DRAM_WR):
                if cname in j["counters"] and j["counters"][cname] > 0:
                    cal[cname] = j["rec"]["bytes_read"] / j["counters"][cname]

    counters = sorted({c for j in joined for c in j["counters"]})
    lines = [f"# {args.title}", "", "Commands:", "", "```", *args.command, "```", ""]
    if cal:
        lines += ["Calibration on the streaming copy probe (known bytes / counted bytes): " +
                  ", ".join(f"{k} x{v:.4f}" for k, v in cal.items()), ""]
    hdr = ["workload", "kernel", "launches", *counters]
    if "FETCH_SIZE" in counters:
        hdr.append("HBM read MB (cal.)")
    if "WRITE_SIZE" in counters:
        hdr.append("HBM write MB (cal.)")
    if DRAM_RD in counters:
        hdr.append("DRAM read MB (cal.)")
    if DRAM_WR in counters:
        hdr.append("DRAM write MB (cal.)")
    hdr.append("compulsory MB")
    hdr.append("model issued-load MB")
    lines += ["| " + " | ".join(hdr) + " |", "|" + "---|" * len(hdr)]
    traffic = {}
    for j in joined:
        r, c = j["rec"], j["counters"]
        row = [r.get("workload", "-"), r.get("kernel", j["name"]), str(len(j["kernels"]))]
        row += [f"{c[k]:.6g}" if k in c else "-" for k in counters]
        rd = c.get("FETCH_SIZE", 0.0) * 1024 * cal.get("FETCH_SIZE", 1.0)
        wr = c.get("WRITE_SIZE", 0.0) * 1024 * cal.get("WRITE_SIZE", 1.0)
        if "FETCH_SIZE" in counters:
            row.append(f"{rd / 1e6:.1f}")
        if "WRITE_SIZE" in counters:
            row.append(f"{wr / 1e6:.1f}")
        drd = c.get(DRAM_RD, 0.0) * cal.get(DRAM_RD, 64.0)
        dwr = c.get(DRAM_WR, 0.0) * cal.get(DRAM_WR, 64.0)
        if DRAM_RD in counters:
            row.append(f"{drd / 1e6:.1f}" if DRAM_RD in c else "-")
        if DRAM_WR in counters:
            row.append(f"{dwr / 1e6:.1f}" if DRAM_WR in c else "-")
        comp = _compulsory(r)
        row.append(f"{comp / 1e6:.1f}" if comp else "-")
        row.append(f"{r['model_issued_load_bytes'] / 1e6:.1f}" if r.get("model_issued_load_bytes") else "-")
        lines.append("| " + " | ".join(row) + " |")
        if (r.get("variant") == "prod" and "FETCH_SIZE" in c and "WRITE_SIZE" in c
                and "FETCH_SIZE" in cal and "WRITE_SIZE" in cal):
            rec = {
                "config": r["kernel"], "prod_source_sha256_16": prod_source_digest(),
                "fetch_kib_counted": c["FETCH_SIZE"], "write_kib_counted": c["WRITE_SIZE"],
                "fetch_scale": cal["FETCH_SIZE"], "write_scale": cal["WRITE_SIZE"],
                "l2_fabric_read_bytes": round(rd), "l2_fabric_write_bytes": round(wr),
                "hbm_bytes_per_launch": round(rd + wr),
                "compulsory_bytes": comp}
            if DRAM_RD in c and DRAM_WR in c and DRAM_RD in cal and DRAM_WR in cal:
                rec.update({"dram_rdreq_counted": c[DRAM_RD], "dram_wrreq_counted": c[DRAM_WR],
                            "dram_read_bytes_per_request": cal[DRAM_RD],
                            "dram_write_bytes_per_request": cal[DRAM_WR],
                            "dram_read_bytes": round(drd), "dram_write_bytes": round(dwr),
                            "dram_bytes_per_launch": round(drd + dwr)})
            traffic[r["workload"]] = rec
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)
    if args.traffic_out and traffic:
        old = {}
        if os.path.exists(args.traffic_out):
            with open(args.traffic_out) as f:
                old = json.load(f)
        old.update(traffic)
        old["_about"] = ("Bytes per product of the production kernel's automatic entry. "
                         "hbm_bytes_per_launch = l2_fabric_read_bytes + l2_fabric_write_bytes: "
                         "rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by "
                         "the streaming copy probe's known/counted ratio; this is traffic from "
                         "L2 to the fabric and includes Infinity-Cache hits. dram_* = "
                         "TCC_EA0_RDREQ_DRAM and TCC_EA0_WRREQ_DRAM request counts scaled by the "
                         "copy probe's known bytes per counted request. Commands in the matching "
                         "profiles/*.md summary.")
        with open(args.traffic_out, "w") as f:
            json.dump(old, f, indent=1, sort_keys=True)
            f.write("\n")
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--csv", action="append", required=True)
    t.add_argument("--command", action="append", default=[])
    t.add_argument("--title", default="rocprofv3 kernel trace")
    t.add_argument("--out")
    t.add_argument("--only-ours", action="store_true")
    t.add_argument("--ladder", help="ladder JSONL of the traced run: group dispatches per record")
    p = sub.add_parser("pmc")
    p.add_argument("--run", action="append", required=True, help="LADDER_JSONL:COUNTER_CSV")
    p.add_argument("--command", action="append", default=[])
    p.add_argument("--title", default="rocprofv3 counters")
    p.add_argument("--out")
    p.add_argument("--traffic-out")
    c = sub.add_parser("clock")
    c.add_argument("--counters", required=True)
    c.add_argument("--trace", required=True)
    c.add_argument("--command", action="append", default=[])
    c.add_argument("--title", default="Engine clock under load")
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--min-dispatches", type=int, default=5)
    c.add_argument("--out")
    args = ap.parse_args(argv)
    return {"trace": cmd_trace, "pmc": cmd_pmc, "clock": cmd_clock}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
