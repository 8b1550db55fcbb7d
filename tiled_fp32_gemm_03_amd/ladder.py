"""Time the kernel ladder on the named workloads (measurement harness).

    python -m tiled_fp32_gemm_03_amd.ladder --workloads square_4096 \
        --variants naive,tiled,tiled32,prod --reps 10

``--variants`` takes rung names (naive, tiled, tiled32, tiled32_pad, tiled4,
valu, prod, and the 16-bit-input rungs bf16 and f16) and, for rungs with a
launch table, ``<rung>:<i>`` for entry i or ``<rung>:all`` for every entry.
The 16-bit rungs take each workload rounded to their format (the seeded
generator's rounding) and report against the dense bf16/fp16 matrix peak.
``splitk`` runs the split-K form of the production kernel with its automatic
plan; ``splitk:<s>`` asks for s chunks (workspace allocated once per record,
outside the timed region).  ``--alu-probes`` first measures the fp32
vector-FMA probe at 1, 2, 4, 8 and 16 waves per SIMD, the LDS read-bandwidth
probe and the fp32 MFMA probe (the compute and on-chip roofs of the rungs).  ``--copy-mib N`` first runs the streaming copy
probe once over N MiB (a kernel of known traffic: N MiB read, N MiB written)
so that memory counters collected over the same run can be calibrated.
Before each record the tool launches a marker (a 3-float fill, which runs
only the scalar tail kernel), so that a
counter run can attribute every dispatch between two markers -- a product
may take more than one launch -- to the record that follows the marker.

Each measurement prints one JSON line (kernel; ms per launch from HIP events
on the launch stream -- the mean over back-to-back calls, plus the median and
minimum of the per-call times read from events between the calls; TFLOP/s,
compulsory-byte GB/s, the tiled load model; with ``--cold`` the same timings
for calls that each follow a 1 GiB fill, i.e. inputs out of the caches);
a markdown table goes to stderr at the end.  Inputs come from the seeded
generator and are resident on the GPU before timing.  After the timed calls
each record checks a sample of its result (2048 random elements and the four
corners) against dot products formed in float64 on the host with numpy:
equal for integer-valued workloads, within 1e-4 sqrt(K) otherwise.  That
reference is written here, not taken from the CPU oracle, which the package
never loads; the GPU test suite compares every element of every rung's
result on these workloads with the oracle, and the benchmark reports that
comparison for the production kernel's automatic entry on each workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


MIXED = ("bf16", "f16")


def _num_configs(g, name: str) -> int:
    if name == "splitk":
        raise ValueError("splitk takes a chunk count (splitk:<s>), not 'all'")
    return g.gemm_mixed_num_configs() if name in MIXED else g.gemm_f32_num_configs(name)


def _expand_variants(spec: str, g) -> list[tuple[str, int]]:
    out = []
    for item in spec.split(","):
        item = item.strip()
        if not item:
            continue
        if ":" in item:
            name, cfg = item.split(":", 1)
            if cfg == "all":
                out += [(name, i) for i in range(_num_configs(g, name))]
            else:
                out.append((name, int(cfg)))
        else:
            out.append((item, -1))
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workloads", default="square_256,square_1024_int,square_4096,ragged,skinny_k64")
    ap.add_argument("--variants", default="naive,tiled,tiled32,prod")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--copy-mib", type=int, default=0)
    ap.add_argument("--alu-probes", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="also time each call after a 1 GiB fill (inputs out of the caches)")
    ap.add_argument("--max-naive-gflop", type=float, default=200.0,
                    help="skip the naive rung on workloads above this many GFLOP")
    args = ap.parse_args(argv)

    import numpy as np
    import torch

    import tiled_fp32_gemm_03_amd as g
    from gemm_inputs import make_mixed_workload, make_workload
    from tiled_fp32_gemm_03_amd import roofline as rf

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream

    flush = None
    if args.cold:
        flush_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB

        def flush():
            g.gemm_f32_probe_stream(g.PROBE_FILL, flush_buf.numel(), 0, 0, flush_buf.data_ptr(), s)

    def timed_stats(fn, reps, warmup, cold=False):
        """(mean, median, min) ms per call.  Warm: the calls run back to back
        with an event between consecutive calls (no extra work on the
        stream); mean = whole span / reps.  Cold: a 1 GiB fill runs before
        each call, outside its events."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        if cold:
            spans = []
            for _ in range(reps):
                flush()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                spans.append((e0, e1))
            torch.cuda.synchronize()
            per = [a.elapsed_time(b) for a, b in spans]
            return sum(per) / len(per), statistics.median(per), min(per)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
        return ev[0].elapsed_time(ev[reps]) / max(reps, 1), statistics.median(per), min(per)

    def timed(fn, reps, warmup):
        return timed_stats(fn, reps, warmup)[0]

    marker = torch.empty(4, device=dev)

    def mark():
        g.gemm_f32_probe_stream(g.PROBE_FILL, 3, 0, 0, marker.data_ptr(), s)

    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        x = torch.ones(n, device=dev)
        z = torch.empty(n, device=dev)
        torch.cuda.synchronize()
        print(f"[ladder] copy probe over {args.copy_mib} MiB", file=sys.stderr, flush=True)
        mark()
        ms = timed(lambda: g.gemm_f32_probe_stream(g.PROBE_COPY, n, x.data_ptr(), 0, z.data_ptr(), s), 1, 0)
        print(json.dumps({"kernel": "probe_copy", "bytes_read": n * 4, "bytes_written": n * 4,
                          "ms": round(ms, 5)}), flush=True)
        del x, z
        torch.cuda.empty_cache()

    if args.alu_probes:
        simds = 4 * torch.cuda.get_device_properties(dev).multi_processor_count
        for waves in (1, 2, 4, 8, 16):
            wgs = waves * simds // 4  # 4 waves per 256-thread workgroup
            iters = 1000
            buf = torch.zeros(wgs * 4, device=dev)
            ms = timed(lambda: g.gemm_f32_probe_valu(wgs, iters, buf.data_ptr(), s), 5, 2)
            tf = g.gemm_f32_probe_valu_flops(wgs, iters) / (ms * 1e-3) / 1e12
            print(json.dumps({"kernel": "probe_valu", "waves_per_simd": waves, "workgroups": wgs,
                              "ms": round(ms, 5), "tflops": round(tf, 2)}), flush=True)
        for wg_per_cu in (1, 2, 8):
            wgs, iters = wg_per_cu * simds // 4, 2000
            buf = torch.zeros(wgs * 4, device=dev)
            ms = timed(lambda: g.gemm_f32_probe_lds(wgs, iters, buf.data_ptr(), s), 5, 2)
            nbytes = g.gemm_f32_probe_lds_bytes(wgs, iters)
            print(json.dumps({"kernel": "probe_lds", "workgroups": wgs, "ms": round(ms, 5),
                              "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                              "bytes_per_cu_clock_at_2p4ghz": round(
                                  nbytes / (ms * 1e-3) / (simds // 4) / 2.4e9, 1)}), flush=True)
        wgs, iters = simds, 2000
        buf = torch.zeros(wgs * 4, device=dev)
        ms = timed(lambda: g.gemm_f32_probe_mfma(wgs, iters, buf.data_ptr(), s), 5, 2)
        tf = g.gemm_f32_probe_mfma_flops(wgs, iters) / (ms * 1e-3) / 1e12
        print(json.dumps({"kernel": "probe_mfma", "workgroups": wgs, "ms": round(ms, 5),
                          "tflops": round(tf, 2)}), flush=True)
        del buf

    def decode16(bits, fmt):
        """float64 values of bf16 or fp16 codes (uint16 bit patterns)."""
        bits = np.asarray(bits).view(np.uint16)
        if fmt == "f16":
            return bits.view(np.float16).astype(np.float64)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    def sampled_check(host, wl, fmt, n=2048):
        """Sampled elements of tc against float64 dot products on the host."""
        rng = np.random.default_rng(12345)
        ii = np.concatenate([rng.integers(0, wl.M, n), [0, wl.M - 1, 0, wl.M - 1]])
        jj = np.concatenate([rng.integers(0, wl.N, n), [0, 0, wl.N - 1, wl.N - 1]])
        ha, hb = host[fmt]
        if fmt == "f32":
            ra, rb = ha[ii].astype(np.float64), hb[:, jj].astype(np.float64)
        else:
            ra, rb = decode16(ha[ii], fmt), decode16(hb[:, jj], fmt)
        ref = np.einsum("ik,ki->i", ra, rb)
        got = tc[torch.from_numpy(ii).to(dev), torch.from_numpy(jj).to(dev)].double().cpu().numpy()
        err = float(np.max(np.abs(got - ref))) if len(ref) else 0.0
        exact = wl.dist == "int4"
        bar = 0.0 if exact else 1e-4 * float(np.sqrt(max(wl.K, 1)))
        return {"samples": int(len(ref)), "max_abs_err": err,
                "bar": "equal" if exact else f"max|d| <= 1e-4 sqrt(K) = {bar:.3g}",
                "pass": bool(np.isfinite(got).all() and err <= bar)}

    rows = []
    specs = _expand_variants(args.variants, g)
    for wname in [w for w in args.workloads.split(",") if w]:
        fmts = sorted({v for v, _ in specs if v in MIXED})
        w, a, b = make_workload(wname)
        ops = {"f32": (torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev))}
        host = {"f32": (a, b)}
        for fmt in fmts:
            _, a16, b16 = make_mixed_workload(wname, fmt)
            ops[fmt] = (torch.from_numpy(a16.view(np.int16)).to(dev),
                        torch.from_numpy(b16.view(np.int16)).to(dev))
            host[fmt] = (a16, b16)
        del a, b
        tc = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        for vname, cfg in specs:
            gflop = rf.flops(w.M, w.N, w.K) / 1e9
            if vname == "naive" and gflop > args.max_naive_gflop:
                continue
            mixed = vname in MIXED
            split = vname == "splitk"
            try:
                if mixed:
                    tile = g.gemm_mixed_tile(cfg, w.M, w.N, w.K)
                elif split:
                    plan = g.gemm_f32_splitk_plan(w.M, w.N, w.K, -1, max(cfg, 0))
                    tile = g.gemm_f32_tile("prod", plan["config"], w.M, w.N, w.K)
                else:
                    tile = g.gemm_f32_tile(vname, cfg, w.M, w.N, w.K)
            except g.GemmError:  # entry does not accept this shape (small-K entries)
                continue
            if mixed:
                label = g.mixed_config_name(vname, cfg, w.M, w.N, w.K)
            elif split:
                label = (g.config_name("prod", plan["config"], w.M, w.N, w.K).replace("prod", "splitk")
                         + f"/{plan['splits']}x{plan['kc']}")
                ws = torch.empty(max(plan["workspace_bytes"] // 4, 1), dtype=torch.float32, device=dev)
            else:
                label = g.config_name(vname, cfg, w.M, w.N, w.K)
            reps = args.reps if vname != "naive" else max(1, min(args.reps, 3))
            print(f"[ladder] {wname} {label} reps={reps}", file=sys.stderr, flush=True)
            ta, tb = ops[vname if mixed else "f32"]

            if mixed:
                def call():
                    g.gemm_mixed(w.M, w.N, w.K, ta.data_ptr(), w.K, tb.data_ptr(), w.N,
                                 tc.data_ptr(), w.N, vname, cfg, s)
            elif split:
                def call():
                    g.gemm_f32_splitk(w.M, w.N, w.K, ta.data_ptr(), w.K, tb.data_ptr(), w.N,
                                      tc.data_ptr(), w.N, -1, plan["splits"], ws.data_ptr(),
                                      ws.numel() * 4, s)
            else:
                def call():
                    g.gemm_f32_ex(w.M, w.N, w.K, ta.data_ptr(), w.K, tb.data_ptr(), w.N,
                                  tc.data_ptr(), w.N, vname, cfg, s)

            mark()

            ms, ms_med, ms_min = timed_stats(call, reps,
                                             args.warmup if vname != "naive" else min(args.warmup, 1))
            tflops = rf.flops(w.M, w.N, w.K) / (ms * 1e-3) / 1e12
            half = mixed
            peak = rf.PEAK_BF16_MFMA_TFLOPS if half else rf.PEAK_FP32_MFMA_TFLOPS
            elem = 2 if half else 4
            rec = {"workload": wname, "kernel": label, "variant": vname, "config": tile["config"],
                   "ms": round(ms, 5), "ms_median": round(ms_med, 5), "ms_min": round(ms_min, 5),
                   "tflops": round(tflops, 3),
                   "frac_peak": round(tflops / peak, 4), "peak_tflops": peak,
                   "gbps_compulsory": round(rf.compulsory_bytes(w.M, w.N, w.K, elem) / (ms * 1e-3) / 1e9, 1),
                   "model_issued_load_bytes": elem * rf.issued_load_elements(
                       "prod" if (mixed or split) else vname, w.M, w.N, w.K, tile),
                   "flops": rf.flops(w.M, w.N, w.K)}
            if args.cold:
                cms, cmed, cmin = timed_stats(call, reps, 0, cold=True)
                rec.update({"cold_ms": round(cms, 5), "cold_ms_median": round(cmed, 5),
                            "cold_ms_min": round(cmin, 5)})
            torch.cuda.synchronize()
            rec["check"] = sampled_check(host, w, vname if mixed else "f32")
            rows.append(rec)
            print(json.dumps(rec), flush=True)
        del ops, tc, host
        torch.cuda.empty_cache()

    print("\n| workload | kernel | ms | TFLOP/s | % of dtype peak | GB/s (compulsory) | median ms | min ms |"
          + (" cold median ms |" if args.cold else "") + " sampled check |", file=sys.stderr)
    print("|---|---|---|---|---|---|---|---|" + ("---|" if args.cold else "") + "---|", file=sys.stderr)
    for r in rows:
        c = r["check"]
        print(f"| {r['workload']} | {r['kernel']} | {r['ms']:.4f} | {r['tflops']:.2f} | "
              f"{100 * r['frac_peak']:.1f} | {r['gbps_compulsory']:.0f} | {r['ms_median']:.4f} | "
              f"{r['ms_min']:.4f} |" + (f" {r['cold_ms_median']:.4f} |" if args.cold else "")
              + f" {'pass' if c['pass'] else 'FAIL'} ({c['max_abs_err']:.2g}) |", file=sys.stderr)
    failed = [r for r in rows if not r["check"]["pass"]]
    if failed:
        print(f"[ladder] {len(failed)} record(s) failed the sampled check", file=sys.stderr)
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
