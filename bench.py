#!/usr/bin/env python3
"""Benchmark of the fp32 matrix multiply C = A x B on one MI355X.

A step is one call of the production kernel on the square 4096^3 workload
(A, B ~ U[-1, 1], seed 2; inputs resident in HBM before timing starts).
Before the timed steps the same call runs for a fixed settle period, so the
timed region sees the engine clock the kernel sustains rather than its ramp.

Prints ONE JSON line with TFLOP/s, the roofline of the dominant kernel, and,
as extra keys:
  * measured denominators (HBM streaming probes, fp32 MFMA probe, the fused
    MFMA + store probe at the skinny product's intensity, with the engine
    clock it ran at);
  * one record per workload (square_256, square_1024_int, square_4096,
    ragged, skinny_k64): the automatic entry, its time, TFLOP/s, GB/s and the
    fraction of its binding roof, the CPU oracle's time for the same full
    product on this host, and the verdict of comparing every element of the
    GPU result with the oracle's (bit-exact on integer inputs, the fp32
    tolerance otherwise), taken outside the timed regions;
  * the skinny K = 64 block against the bandwidth measured in the same run;
  * the CPU oracle on the benchmark workload as the reported baseline.

  python bench.py [--gpus 1] [--steps 100] [--warmup 20]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fp32 GEMM TFLOPS @N=4096 (% of fp32 peak); HBM GB/s on K=64 skinny shape"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
WORKLOADS = ("square_256", "square_1024_int", "square_4096", "ragged", "skinny_k64")
# Timed calls per workload record: more for the few-microsecond products.
RECORD_REPS = {"square_256": 50, "square_1024_int": 50}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def settle(fn, settle_ms: float) -> tuple[int, float]:
    """Run fn back to back for at least settle_ms of wall time (synchronising
    every few launches), so the engine clock reaches what this load sustains."""
    import torch
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def time_launches(fn, steps: int, warmup: int, stream) -> tuple[float, float]:
    """(average ms per launch from HIP events on `stream`, wall seconds)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def time_each(fn, reps: int, warmup: int, stream) -> dict:
    """Per-call times from events recorded between back-to-back calls on
    `stream` (no work added to the stream): mean, median and min in ms."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    return {"mean_ms": ev[0].elapsed_time(ev[-1]) / reps, "median_ms": statistics.median(per),
            "min_ms": min(per), "reps": reps}


def measure_hbm(g, stream, reps: int = 8) -> dict:
    """Streaming probes over 1 GiB arrays (far above the 256 MB Infinity Cache)."""
    import torch
    n = 1 << 28  # floats per array
    dev = torch.device("cuda:0")
    x = torch.ones(n, device=dev)
    y = torch.ones(n, device=dev)
    z = torch.empty(n, device=dev)
    s = stream.cuda_stream
    out = {}
    for kind, name, bytes_per in ((g.PROBE_COPY, "copy", 8), (g.PROBE_FILL, "fill", 4),
                                  (g.PROBE_VADD, "vector_add", 12)):
        ms, _ = time_launches(lambda: g.gemm_f32_probe_stream(kind, n, x.data_ptr(), y.data_ptr(),
                                                               z.data_ptr(), s), reps, 2, stream)
        out[name] = round(n * bytes_per / (ms * 1e-3) / 1e9, 1)
    del x, y, z
    torch.cuda.empty_cache()
    out["best"] = max(out.values())
    return out


def measure_mfma(g, stream) -> float:
    """fp32 MFMA probe: 8 independent accumulator chains per wave, two waves
    per SIMD, about 1.7 ms per launch; 20 timed launches after 5 warm-up ones."""
    import torch
    wgs, iters = 256 * 2, 4000
    buf = torch.zeros(wgs * 4, device="cuda:0")
    ms, _ = time_launches(lambda: g.gemm_f32_probe_mfma(wgs, iters, buf.data_ptr(), stream.cuda_stream),
                          20, 5, stream)
    return g.gemm_f32_probe_mfma_flops(wgs, iters) / (ms * 1e-3) / 1e12


def measure_mfma16(g, stream) -> dict:
    """bf16 MFMA probe at one wave per SIMD (one 256-thread workgroup per
    CU), the 16-bit rung's occupancy: TFLOP/s of independent 16x16x32 and
    32x32x16 chains; 20 timed launches after 5 warm-up ones, about 1 ms each."""
    import torch
    wgs = 256
    buf = torch.zeros(wgs * 4, device="cuda:0")
    out = {}
    for shape, iters in ((16, 2500), (32, 7000)):
        ms, _ = time_launches(lambda: g.gemm_f32_probe_mfma16(shape, wgs, iters, buf.data_ptr(),
                                                              stream.cuda_stream), 20, 5, stream)
        name = "16x16x32" if shape == 16 else "32x32x16"
        out[name] = round(g.gemm_f32_probe_mfma16_flops(shape, wgs, iters) / (ms * 1e-3) / 1e12, 1)
    return out


def measure_valu(g, stream) -> float:
    import torch
    wgs, iters = 256 * 8, 500
    buf = torch.zeros(wgs * 4, device="cuda:0")
    ms, _ = time_launches(lambda: g.gemm_f32_probe_valu(wgs, iters, buf.data_ptr(), stream.cuda_stream),
                          5, 2, stream)
    return g.gemm_f32_probe_valu_flops(wgs, iters) / (ms * 1e-3) / 1e12


def measure_fused(g, stream, settle_ms: float) -> dict:
    """The fused probe at the skinny product's intensity (32 FLOP per stored
    byte) with the FLOPs and the 1 GiB output of 16384 x 16384 x 64: MFMAs
    and stores together, each alone, at one and two waves per SIMD.  Reports
    each mode's time, rates and the engine clock the waves saw."""
    import torch
    dev = torch.device("cuda:0")
    out = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    s = stream.cuda_stream
    res = {}
    for wgs, trips in ((256, 1024), (512, 512)):
        clocks = torch.zeros(2 * wgs * 4, dtype=torch.int64, device=dev)
        for mode, name in ((g.FUSED_BOTH, "both"), (g.FUSED_MFMA, "mfma_only"),
                           (g.FUSED_STORE, "store_only")):
            def call():
                g.gemm_f32_probe_fused(mode, wgs, trips, out.data_ptr(), out.numel() * 4,
                                       clocks.data_ptr(), s)
            settle(call, settle_ms)
            t = time_each(call, 10, 2, stream)
            ms = t["median_ms"]
            fl = g.gemm_f32_probe_fused_flops(mode, wgs, trips)
            by = g.gemm_f32_probe_fused_bytes(mode, wgs, trips) if mode != g.FUSED_MFMA else 0
            c = clocks.view(-1, 2).double()
            mhz = float((c[:, 0] / c[:, 1]).mean().item() * 100.0)
            res[f"{name}_w{wgs // 256}"] = {
                "ms": round(ms, 5), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                "gbps": round(by / (ms * 1e-3) / 1e9, 1), "clock_mhz": round(mhz, 1)}
    del out
    torch.cuda.empty_cache()
    best = max((v for k, v in res.items() if k.startswith("both")), key=lambda v: v["tflops"])
    res["best_both_tflops"] = best["tflops"]
    res["best_both_gbps"] = best["gbps"]
    return res


def load_traffic(workload: str, config_label: str) -> dict:
    """Bytes per launch from committed rocprofv3 counter runs: calibrated
    FETCH_SIZE + WRITE_SIZE (L2 to fabric), the DRAM-bound request counts
    scaled the same way, and their split; empty when absent or taken on a
    different version of the production kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return {}
    from tiled_fp32_gemm_03_amd.counters import prod_source_digest

    rec = data.get(workload)
    if not rec or rec.get("prod_source_sha256_16") != prod_source_digest():
        return {}
    if rec.get("config") != config_label:
        return {}
    keys = ("hbm_bytes_per_launch", "l2_fabric_read_bytes", "l2_fabric_write_bytes",
            "dram_bytes_per_launch", "dram_read_bytes", "dram_write_bytes")
    return {k: rec[k] for k in keys if k in rec}


def cpu_model() -> str:
    name = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return name


def oracle_product(a, b) -> tuple:
    """The CPU oracle (test infrastructure) on the whole product: (C, seconds)."""
    import oracle
    t0 = time.perf_counter()
    c = oracle.gemm(a, b)
    return c, time.perf_counter() - t0


def compare_full(got, ref, K: int, exact: bool) -> dict:
    """Every element of the GPU result against the oracle's, in fp64, a band
    of rows at a time (bit-exact bar for integer inputs, else max |diff| <=
    1e-4 sqrt(K) and relative Frobenius <= 1e-5)."""
    import numpy as np
    M, N = got.shape
    rows = max(1, (1 << 22) // max(N, 1))
    max_err, err2, ref2, mism, finite = 0.0, 0.0, 0.0, 0, True
    for r0 in range(0, M, rows):
        g64 = got[r0:r0 + rows].astype(np.float64)
        r64 = ref[r0:r0 + rows].astype(np.float64)
        finite = finite and bool(np.isfinite(g64).all())
        d = np.abs(g64 - r64)
        if d.size:
            max_err = max(max_err, float(d.max()))
        err2 += float(np.dot(d.ravel(), d.ravel()))
        ref2 += float(np.dot(r64.ravel(), r64.ravel()))
        mism += int(np.count_nonzero(got[r0:r0 + rows] != ref[r0:r0 + rows]))
    fro = (err2 ** 0.5) / (ref2 ** 0.5) if ref2 > 0 else err2 ** 0.5
    if exact:
        ok = finite and mism == 0
        bar = "bit-exact"
    else:
        ok = finite and max_err <= 1e-4 * max(K, 1) ** 0.5 and fro <= 1e-5
        bar = "max|d| <= 1e-4 sqrt(K), rel Frobenius <= 1e-5"
    return {"pass": ok, "bar": bar, "elements": int(M * N), "max_abs_err": max_err,
            "rel_fro": fro, "mismatched_bits": mism}


def workload_record(g, rf, name: str, stream, settle_ms: float, peaks: dict) -> dict:
    """One workload through the automatic production entry: timing, roofline
    fraction, the oracle's time on the same product, and the full comparison."""
    import torch

    from gemm_inputs import make_workload
    w, a, b = make_workload(name)
    dev = torch.device("cuda:0")
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    tc = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    label = g.config_name("prod", -1, w.M, w.N, w.K)
    s = stream.cuda_stream

    def call():
        g.gemm_f32_ex(w.M, w.N, w.K, ta.data_ptr(), w.K, tb.data_ptr(), w.N, tc.data_ptr(), w.N,
                      "prod", -1, s)

    settle(call, settle_ms)
    reps = RECORD_REPS.get(name, 20)
    t = time_each(call, reps, 5, stream)
    # The same calls with no event between them (as the headline is timed):
    # for the few-microsecond products the per-call events add a few us.
    b2b_ms, _ = time_launches(call, reps, 0, stream)
    got = tc.cpu().numpy()
    del ta, tb, tc
    torch.cuda.empty_cache()
    ms = t["median_ms"]
    fl = rf.flops(w.M, w.N, w.K)
    by = rf.compulsory_bytes(w.M, w.N, w.K)
    tflops = fl / (ms * 1e-3) / 1e12
    gbps = by / (ms * 1e-3) / 1e9
    rec = {"workload": name, "M": w.M, "N": w.N, "K": w.K, "dist": w.dist, "seed": w.seed,
           "kernel": label, **{k: round(v, 5) if isinstance(v, float) else v for k, v in t.items()},
           "tflops": round(tflops, 3), "gbps": round(gbps, 1),
           "back_to_back_ms": round(b2b_ms, 5),
           "tflops_back_to_back": round(fl / (b2b_ms * 1e-3) / 1e12, 3),
           "intensity_flop_per_byte": round(rf.intensity(w.M, w.N, w.K), 2)}
    ai = rf.intensity(w.M, w.N, w.K)
    if name == "square_256":
        rec["roof"] = "launch latency (a few microseconds): no roofline claim"
        rec["frac_of_binding_roof"] = None
    else:
        pmeas = peaks.get("mfma_fp32_tflops", rf.PEAK_FP32_MFMA_TFLOPS)
        bmeas = peaks.get("hbm_gbps", {}).get("best", rf.PEAK_HBM_GBPS)
        roof = rf.binding_roof_tflops(w.M, w.N, w.K, pmeas, bmeas)
        rec["roof"] = "mfma" if pmeas <= ai * bmeas / 1000 else "hbm"
        rec["binding_roof_tflops"] = round(roof, 2)
        rec["frac_of_binding_roof"] = round(tflops / roof, 4)
        rec["frac_of_peak_fp32"] = round(tflops / rf.PEAK_FP32_MFMA_TFLOPS, 4)
    log(f"{name} {label}: median {ms:.4f} ms, {tflops:.2f} TFLOP/s, {gbps:.0f} GB/s; "
        f"back to back {b2b_ms:.4f} ms")
    ref, osec = oracle_product(a, b)
    import oracle
    rec["oracle"] = {"seconds": round(osec, 3), "gflops": round(fl / osec / 1e9, 2),
                     "cores": oracle.num_threads(), "cpu_model": cpu_model(),
                     "gpu_over_oracle": round(osec / (ms * 1e-3), 1)}
    rec["verdict"] = compare_full(got, ref, w.K, exact=(w.dist == "int4"))
    log(f"{name}: oracle {osec:.2f} s on {oracle.num_threads()} threads; verdict {rec['verdict']}")
    del got, ref
    return rec


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="wall time the benchmark call runs before warm-up and timing")
    ap.add_argument("--workload", default="square_4096")
    ap.add_argument("--variant", default="prod")
    ap.add_argument("--config", type=int, default=-1, help="launch-table entry (-1 = automatic)")
    ap.add_argument("--record-settle-ms", type=float, default=200.0)
    ap.add_argument("--no-probes", action="store_true")
    ap.add_argument("--no-records", action="store_true",
                    help="skip the per-workload records (and with them the oracle runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; this library measures one GPU "
              "(the product is a single-GPU kernel; see the sharding notes in the design doc)",
              file=sys.stderr, flush=True)
        return 2

    import torch

    import tiled_fp32_gemm_03_amd as g
    from gemm_inputs import make_workload
    from tiled_fp32_gemm_03_amd import roofline as rf

    if not torch.cuda.is_available():
        print("bench.py: no visible GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    stream = torch.cuda.current_stream(dev)

    w, a, b = make_workload(args.workload)
    log(f"workload {w.name}: {w.description}; device {props.name}, {props.multi_processor_count} CUs")
    ta = torch.from_numpy(a).to(dev)
    tb = torch.from_numpy(b).to(dev)
    tc = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    tile = g.gemm_f32_tile(args.variant, args.config, w.M, w.N, w.K)
    label = g.config_name(args.variant, args.config, w.M, w.N, w.K)
    s = stream.cuda_stream

    def step():
        g.gemm_f32_ex(w.M, w.N, w.K, ta.data_ptr(), w.K, tb.data_ptr(), w.N, tc.data_ptr(), w.N,
                      args.variant, args.config, s)

    n_settle, t_settle = settle(step, args.settle_ms)
    log(f"settled {label}: {n_settle} calls in {t_settle * 1e3:.0f} ms")
    log(f"timing {label}: {args.warmup} warmup + {args.steps} steps")
    ms, wall = time_launches(step, args.steps, args.warmup, stream)
    flops = rf.flops(w.M, w.N, w.K)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{label}: {ms:.4f} ms/launch, {tflops:.2f} TFLOP/s (wall {wall:.3f} s for {args.steps})")

    traffic = load_traffic(w.name, label)
    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "dist": w.dist,
                   "seed": w.seed, "variant": args.variant, "tile": label},
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 3),
            "peak": rf.PEAK_FP32_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / rf.PEAK_FP32_MFMA_TFLOPS, 4),
            "traffic": traffic.get("hbm_bytes_per_launch"),
            "traffic_detail": traffic or None,
            "kernel": label,
            "algorithmic_flops_per_launch": flops,
            "compulsory_bytes_per_launch": rf.compulsory_bytes(w.M, w.N, w.K),
            "model_issued_load_bytes_per_launch": 4 * rf.issued_load_elements(
                args.variant, w.M, w.N, w.K, tile),
        },
        "settle": {"calls": n_settle, "ms": round(t_settle * 1e3, 1)},
        "wall_s_timed_region": round(wall, 4),
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   **g.gemm_f32_device_props(0)},
    }
    if traffic and tile["BM"] == 256 and tile["BN"] == 256:
        # The floor eight L2s set: each XCD fetches every panel its tiles
        # touch once (one persistent workgroup per CU).
        cus = props.multi_processor_count
        tiles = -(-w.M // 256) * -(-w.N // 256)
        floor = rf.xcd_panel_bytes(w.M, w.N, w.K, 256, 256, min(cus, tiles))
        result["roofline"]["traffic_floor_xcd_panels"] = {
            **floor, "measured_over_floor": round(traffic["hbm_bytes_per_launch"] / floor["bytes"], 4)}
    del tc
    torch.cuda.empty_cache()

    measured = {}
    if not args.no_probes:
        log("HBM streaming probes (1 GiB arrays)")
        hbm = measure_hbm(g, stream)
        log(f"HBM GB/s: {hbm}")
        pm = measure_mfma(g, stream)
        log(f"fp32 MFMA probe: {pm:.1f} TFLOP/s")
        pv = measure_valu(g, stream)
        log(f"fp32 vector FMA probe: {pv:.1f} TFLOP/s")
        pb = measure_mfma16(g, stream)
        log(f"bf16 MFMA probe, one wave per SIMD: {pb} TFLOP/s")
        fused = measure_fused(g, stream, args.record_settle_ms)
        log(f"fused MFMA + store probe at 32 FLOP/B: {fused}")
        # The fused probe's store-only mode is a streaming write too: the
        # measured bandwidth is the best of every streaming rate of the run.
        hbm["fused_store_only"] = max(v["gbps"] for k, v in fused.items()
                                      if k.startswith("store_only"))
        hbm["best"] = max(hbm["copy"], hbm["fill"], hbm["vector_add"], hbm["fused_store_only"])
        measured = {"hbm_gbps": hbm, "mfma_fp32_tflops": round(pm, 2),
                    "valu_fp32_tflops": round(pv, 2), "mfma_bf16_one_wave_per_simd_tflops": pb,
                    "fused_k64": fused}
        result["measured_peaks"] = measured
        result["roofline"]["frac_of_measured_mfma"] = round(tflops / pm, 4)

    if not args.no_records:
        records = {}
        for name in WORKLOADS:
            records[name] = workload_record(g, rf, name, stream, args.record_settle_ms, measured)
        result["workloads"] = records
        sk = dict(records["skinny_k64"])
        sk.pop("verdict", None)
        gbps = sk["gbps"]
        sk["frac_of_peak_hbm"] = round(gbps / rf.PEAK_HBM_GBPS, 4)
        if measured:
            bmeas = measured["hbm_gbps"]["best"]
            sk["frac_of_measured_hbm"] = round(gbps / bmeas, 4)
            sk["target_tflops_at_80pct_hbm"] = round(0.8 * bmeas * sk["intensity_flop_per_byte"] / 1000, 2)
            fz = measured["fused_k64"]["best_both_tflops"]
            sk["fused_probe_tflops"] = fz
            sk["frac_of_fused_probe"] = round(sk["tflops"] / fz, 4)
            sk["target_feasible_by_fused_probe"] = fz >= sk["target_tflops_at_80pct_hbm"]
            # The binding roof at this intensity is the lowest of the MFMA
            # probe, intensity x measured bandwidth and the fused probe's
            # rate (matrix work and output stores together, as measured).
            if fz < sk["binding_roof_tflops"]:
                for r in (sk, records["skinny_k64"]):
                    r["binding_roof_tflops"] = fz
                    r["roof"] = "fused mfma+store probe"
                    r["frac_of_binding_roof"] = round(r["tflops"] / fz, 4)
        sk["verdict_pass"] = records["skinny_k64"]["verdict"]["pass"]
        result["skinny_k64"] = sk
        c3 = records.get(w.name)
        if c3 is not None:
            o = c3["oracle"]
            result["cpu_baseline"] = {
                "value": round(flops / o["seconds"] / 1e12, 5), "unit": "TFLOP/s",
                "cores": o["cores"], "kind": "oracle",
                "sample": f"the whole {w.M}x{w.N}x{w.K} product ({w.M * w.N} outputs, full K), "
                          f"{o['seconds']:.2f} s wall",
                "seconds": o["seconds"], "cpu_model": o["cpu_model"]}
        result["all_verdicts_pass"] = all(r["verdict"]["pass"] for r in records.values())
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
