#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long]

One step = one fa_fwd call over one batch of the workload (the whole hot
path: Q.K^T, mask, online softmax, P.V, epilogue). Inputs are seeded
synthetic Gaussians already resident in HBM when timing starts. Prints one
JSON line (rank 0) with the metric, a roofline entry for the kernel, and the
CPU oracle timed on a bounded sample of the same workload.

Default workload: B=2, H=16, S=8192, D=128, bf16, causal (the long-context
configuration the metric is quoted on). FLOPs follow the metric:
4*B*H*S^2*D, halved when causal.

--workload long8 times the 8-bit entry point (fa_fwd_fp8) on the same shape
with E4M3 inputs and per-tensor descales, against the fp8 MFMA peak, and
prints its own JSON line (its CPU baseline is the same oracle on the decoded
values).

--varlen times the variable-length entry point instead, on a packed batch of
16 causal sequences with seeded lengths in [256, 8192] (H=16, D=128, bf16),
and prints its own JSON line; FLOPs then sum the metric over the sequences.

Before the W warm-up steps the same call runs back to back for --settle-s
seconds (default 0.3): the MI355X power manager needs tens of milliseconds
of a given load to settle the engine clock, and the metric is sustained
throughput. The engine clock is sampled (sysfs pp_dpm_sclk) during the timed
region and reported with the fraction of the peak re-derived at that clock
("sclk", "pct_of_peak_at_sclk"). Workloads under 64 MiB (tiny, dec) also get
a cold-cache leg ("cold"): launches timed one by one after a 512 MiB scrub
write that evicts L2 and the MALL.

Extra modes (used to take profiles): --calibrate-copy runs plain device
copies of a known size first (for scaling HBM byte counters);
--no-cpu-baseline skips the oracle leg; --write-traffic FETCH_CSV WRITE_CSV
(no GPU needed) turns two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE,
each of a --calibrate-copy bench run) into the per-launch HBM traffic file
that fills roofline.traffic.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "attention fwd TFLOPS (B·H·S²·D·4, causal halved) + % of bf16 MFMA peak"
PEAK_TFLOPS = 2516.6  # MI355X dense fp16/bf16 MFMA peak (published 2.5 PFLOP/s)
PEAK_TFLOPS_FP8 = 5033.2  # MI355X dense fp8 MFMA peak (published 5.0 PFLOP/s)
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "exact_attention_16_amd", "csrc")


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"fa_fwd_{workload}_hbm_traffic.json")


def _code_only(text: str) -> str:
    """C++ source without comments and blank lines (what changes the kernels)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def kernel_source_hash() -> str:
    """Hash of the code (comments dropped) of every attention kernel source
    file (the issue-rate probes are not one)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")) and name != "fa_probe.hip":
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch from the committed counter profile, if it was
    taken on the current kernel source; otherwise None."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


CALIBRATION_BYTES = 1 << 30  # each --calibrate-copy copy reads and writes 1 GiB
PEAK_SCLK_MHZ = 2400.0  # engine clock at which the published peaks are quoted


class ClockSampler:
    """Samples the GPU engine clock (MHz) in a background thread while a
    timed region runs: the current level of sysfs pp_dpm_sclk, else amdsmi's
    GPU metrics (the mean of the per-XCD gfx clocks, with socket power).
    The published peaks assume 2.4 GHz; under sustained MFMA load the part
    holds a lower clock, which this records beside every timing."""

    def __init__(self, period_s: float = 0.002):
        import threading
        self.period = period_s
        self.samples: list[float] = []
        self.power: list[float] = []
        self.source = None
        self._stop = threading.Event()
        self._thread = None
        self._read = self._setup()

    def _setup(self):
        # sysfs first: its current level is re-read on every access, while
        # amdsmi's metrics table refreshes too slowly for a sub-second region
        import glob
        for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            def read_sysfs(path=path):
                with open(path) as f:
                    for line in f:
                        if line.rstrip().endswith("*"):
                            return float(re.findall(r"(\d+)\s*[Mm]hz", line)[0]), None
                return None, None
            try:
                if read_sysfs()[0] is not None:
                    self.source = f"sysfs {path}"
                    return read_sysfs
            except Exception:
                continue
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            h = amdsmi.amdsmi_get_processor_handles()[0]

            def read_smi():
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                clks = m.get("current_gfxclks")
                vals = [float(c) for c in clks if isinstance(c, (int, float)) and 0 < c < 10000] \
                    if isinstance(clks, list) else []
                p = m.get("current_socket_power")
                return (sum(vals) / len(vals) if vals else None,
                        float(p) if isinstance(p, (int, float)) and 0 < p < 5000 else None)

            if read_smi()[0] is not None:
                self.source = "amdsmi gpu_metrics current_gfxclks"
                return read_smi
        except Exception:
            pass
        return None

    def _loop(self):
        while not self._stop.is_set():
            try:
                c, p = self._read()
            except Exception:
                return
            if c is not None:
                self.samples.append(c)
            if p is not None:
                self.power.append(p)
            time.sleep(self.period)

    def __enter__(self):
        import threading
        if self._read is not None:
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=5)
        return False

    def report(self) -> dict:
        """Mean / min / max engine clock over the samples, with the source."""
        if not self.samples:
            return {"sclk_mhz": None, "source": self.source, "samples": 0}
        s = self.samples
        return {"sclk_mhz": sum(s) / len(s), "sclk_min_mhz": min(s), "sclk_max_mhz": max(s),
                "samples": len(s), "source": self.source,
                "socket_power_w": sum(self.power) / len(self.power) if self.power else None}


def clock_fields(tflops: float, peak: float, clk: dict) -> dict:
    """The bench line's clock entries: the sampled clock and the fraction of
    the peak re-derived at that clock (peak x sclk / 2400 MHz)."""
    mhz = clk.get("sclk_mhz")
    return {"sclk": clk,
            "pct_of_peak_at_sclk": 100 * tflops / (peak * mhz / PEAK_SCLK_MHZ) if mhz else None}


def kernel_name(w) -> str:
    """The kernel fa_fwd launches for this workload (from the tile query)."""
    import exact_attention_16_amd as fa
    bm, bn, threads, groups = fa.fa_fwd_tile(w.D, w.B, w.H, w.S, w.causal)
    kind = {256: "fa_fwd_pp", 128: "fa_fwd_k4", 64: "fa_fwd_split"}[bm]
    if bm == 256 and bn == 64:
        kind = "fa_fwd_occ4"
    return (f"{kind}<{w.dtype},D={w.D},causal={int(w.causal)}> "
            f"({groups} work-groups x {threads} threads, {bm} query rows, {bn}-key tiles)")


def write_traffic(fetch_csv: str, write_csv: str, workload: str) -> dict:
    """Per-launch HBM bytes of the attention kernel from two rocprofv3 --pmc
    counter files. FETCH_SIZE and WRITE_SIZE are in KiB per dispatch; each is
    scaled by the ratio of the known size of the plain 1 GiB device copies
    that --calibrate-copy runs to what the same counter reads for them."""
    import csv

    def per_dispatch(path, counter):
        rows = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = r["Dispatch_Id"]
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            prev = rows.get(key, (name, 0.0))
            rows[key] = (name, prev[1] + v)
        copies = [v for n, v in rows.values() if "copyBuffer" in n and v > 1e5]
        attn = [v for n, v in rows.values() if "fa_fwd_" in n]
        names = sorted({n for n, _ in rows.values() if "fa_fwd_" in n})
        if not copies or not attn:
            raise SystemExit(f"{path}: no calibration copies or attention dispatches for {counter}")
        factor = CALIBRATION_BYTES / (sum(copies) / len(copies) * 1024.0)
        return factor, sum(attn) / len(attn), len(attn), names

    ff, fkib, fn, names = per_dispatch(fetch_csv, "FETCH_SIZE")
    wf, wkib, wn, _ = per_dispatch(write_csv, "WRITE_SIZE")
    out = {
        "source_hash": kernel_source_hash(),
        "workload": workload,
        "kernels": names,
        "fetch_kib_per_dispatch": fkib, "fetch_dispatches": fn, "fetch_scale": ff,
        "write_kib_per_dispatch": wkib, "write_dispatches": wn, "write_scale": wf,
        "bytes_per_launch": fkib * 1024.0 * ff + wkib * 1024.0 * wf,
        "note": "scale = 1 GiB / (counter KiB x 1024) of the calibration copies",
    }
    os.makedirs(os.path.dirname(traffic_file(workload)), exist_ok=True)
    with open(traffic_file(workload), "w") as f:
        json.dump(out, f, indent=1)
    return out


def blas_threads() -> int:
    try:
        import threadpoolctl
        np.ones((64, 64)) @ np.ones((64, 64))
        info = threadpoolctl.threadpool_info()
        n = [i["num_threads"] for i in info if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w: W.Workload, qb, kb, vb, budget_s: float = 15.0, descale=(1.0, 1.0, 1.0)):
    """The float64 oracle on a random sample of query rows of the workload.

    Rows are drawn uniformly over all heads and positions, processed in
    batches until the time budget is spent; the metric FLOPs of the sample are
    the workload's metric FLOPs times the fraction of rows done.
    """
    import oracle
    rng = np.random.default_rng(123)
    BH = w.B * w.H
    rows_total = BH * w.S
    done = 0
    t0 = time.perf_counter()
    heads = rng.permutation(BH)
    batch = 64
    i = 0
    while time.perf_counter() - t0 < budget_s:
        bh = int(heads[i % len(heads)])
        i += 1
        b, h = divmod(bh, w.H)
        rows = np.sort(rng.choice(w.S, size=batch, replace=False))
        q = W.decode(qb[b, h], w.dtype) * descale[0]
        k = W.decode(kb[b, h], w.dtype) * descale[1]
        v = W.decode(vb[b, h], w.dtype) * descale[2]
        oracle.attention_rows(q, k, v, rows, w.causal, w.scale)
        done += batch
    dt = time.perf_counter() - t0
    tflops = w.flops * done / rows_total / dt / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} random query rows of {rows_total} ({i} batches of {batch} rows, "
                      f"float64 numpy, full key range per row) in {dt:.1f} s; value = metric "
                      f"FLOPs x rows fraction / time",
            "seconds": dt, "cpu": cpu_model()}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="long", choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", dest="cold", action="store_true", default=None,
                    help="also time launches one by one after a cache scrub (default: only "
                         "for workloads under 64 MiB)")
    ap.add_argument("--no-cold", dest="cold", action="store_false")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of back-to-back calls before the warm-up steps, to bring the "
                         "engine clock to its steady state under this load (0: none)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run plain 1 GiB device copies first (counter scaling)")
    ap.add_argument("--varlen", action="store_true",
                    help="time fa_fwd_varlen on the packed variable-length batch")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic file from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args(argv)

    if args.write_traffic:
        print(json.dumps(write_traffic(*args.write_traffic, args.workload), indent=1))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import exact_attention_16_amd as fa

    if args.varlen:
        return bench_varlen(args, torch, fa)
    w = W.WORKLOADS[args.workload]
    if w.dtype == W.E4M3:
        return bench_fp8(args, torch, fa, w)
    dev = torch.device("cuda:0")
    fa.load()  # fails loudly if the HIP library is not built
    qb, kb, vb = W.make_inputs(w)
    tdt = torch.bfloat16 if w.dtype == W.BF16 else torch.float16
    q, k, v = (torch.from_numpy(x.view(np.int16)).view(tdt).to(dev) for x in (qb, kb, vb))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)  # default priority
    code = W.DTYPE_CODE[w.dtype]

    def step():
        fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                  w.B, w.H, w.S, w.D, int(w.causal), w.scale, stream.cuda_stream, code)

    torch.cuda.synchronize()
    if args.calibrate_copy:
        calibrate_copy(torch, dev, stream)
    settled = settle(step, torch, args.settle_s)

    ms_per_step, wall, med_ms, clk = timed(step, stream, torch, args.steps, args.warmup)
    gpu_ms = ms_per_step * args.steps
    tflops = w.flops / (ms_per_step * 1e-3) / 1e12
    assert bool(torch.isfinite(lse).all()), "non-finite output"
    cold = None
    if args.cold or (args.cold is None and w.algorithmic_bytes < COLD_MAX_BYTES):
        cold = cold_timing(step, stream, torch, dev, w.algorithmic_bytes)

    bytes_alg = w.algorithmic_bytes
    print(f"Elapsed Time (total):      {gpu_ms / 1e3:.4f} seconds\n"
          f"Average Time Per Step:     {ms_per_step:.4f} ms\n"
          f"Compute Performance:       {tflops:.2f} TFLOPS ({100 * tflops / PEAK_TFLOPS:.1f}% of "
          f"{PEAK_TFLOPS} peak)\n"
          f"Memory Throughput:         {bytes_alg / (ms_per_step * 1e-3) / 1e9:.2f} GB/s "
          f"(algorithmic bytes, decimal GB)\n"
          f"Median single launch:      {med_ms:.4f} ms\n"
          f"Engine clock (sampled):    {clk.get('sclk_mhz')} MHz", file=sys.stderr, flush=True)

    traffic = load_traffic(w.name)
    gbs = bytes_alg / (ms_per_step * 1e-3) / 1e9
    if w.flops / bytes_alg >= PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        bound = {"bound": "mfma", "achieved": tflops, "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / PEAK_TFLOPS}
    else:  # below the ridge (about 315 FLOP per byte): the algorithmic bytes bound it
        bound = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": gbs / HBM_PEAK_GBS}
    roofline = {**bound, "traffic": traffic,
                "kernel": kernel_name(w),
                "flops_per_launch": w.flops, "avg_launch_ms": ms_per_step,
                "median_launch_ms": med_ms, "algorithmic_bytes_per_launch": bytes_alg,
                "algorithmic_gbs": bytes_alg / (ms_per_step * 1e-3) / 1e9,
                "hbm_gbs": traffic / (ms_per_step * 1e-3) / 1e9 if traffic else None}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, qb, kb, vb)

    out = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to 16-bit",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} S={w.S} D={w.D} {w.dtype} "
                               f"{'causal' if w.causal else 'non-causal'}",
                   "B": w.B, "H": w.H, "S": w.S, "D": w.D, "causal": w.causal,
                   "parallelism": "single GPU"},
        "pct_of_peak": 100 * tflops / PEAK_TFLOPS,
        **clock_fields(tflops, PEAK_TFLOPS, clk),
        "settle": settled,
        "wall_s": wall,
        "roofline": roofline,
        "cold": cold,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def calibrate_copy(torch, dev, stream):
    """Three plain 1 GiB device copies (the known size HBM counters are scaled by)."""
    src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(3):
            dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    print("calibrate-copy: 3 x 1 GiB device copies done", file=sys.stderr, flush=True)


def timed(step, stream, torch, steps: int, warmup: int):
    """W untimed steps, then K timed back-to-back on `stream` (HIP events on
    that stream), with the engine clock sampled meanwhile; returns (ms per
    step, wall seconds, median single-launch ms, clock report)."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sampler = ClockSampler()
    with sampler:
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * min(steps, 20))]
    for i in range(0, len(evs), 2):
        evs[i].record(stream)
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    med = float(np.median([evs[i].elapsed_time(evs[i + 1]) for i in range(0, len(evs), 2)]))
    return ms, wall, med, sampler.report()


COLD_MAX_BYTES = 64 << 20  # workloads below this get the cold-cache leg by default
SCRUB_BYTES = 512 << 20    # larger than the 256 MB last-level cache (MALL) plus the L2s


def cold_timing(step, stream, torch, dev, alg_bytes: int, reps: int = 20) -> dict:
    """Each launch timed on its own after a 512 MiB scrub write has evicted
    the inputs from L2 and the MALL: the cold-cache rate of a small workload
    whose inputs otherwise stay cached between back-to-back launches."""
    scrub = torch.empty(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    per = []
    with torch.cuda.stream(stream):
        for i in range(reps + 2):
            scrub.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            e1.synchronize()
            if i >= 2:
                per.append(e0.elapsed_time(e1))
    del scrub
    med = float(np.median(per))
    return {"median_launch_ms": med, "min_launch_ms": float(min(per)), "launches": len(per),
            "algorithmic_gbs": alg_bytes / (med * 1e-3) / 1e9,
            "scrub_bytes": SCRUB_BYTES,
            "note": "each launch alone after a 512 MiB scrub write (L2 and MALL evicted)"}


def settle(step, torch, seconds: float) -> dict:
    """Brings the GPU to the steady state of this workload before the W
    warm-up steps: the same call, back to back, for `seconds`. From idle, or
    after lighter work, the power manager takes tens of milliseconds of this
    load to settle the engine clock (the first launches of the long workload
    after idle run up to 1.7x their steady duration, and still about 3%
    slower after other work), and the metric is sustained throughput. These
    launches are neither warm-up nor timed steps: those stay exactly W and
    K."""
    if seconds <= 0:
        return {"seconds": 0.0, "launches": 0}
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            step()
        n += 16
        torch.cuda.synchronize()
    return {"seconds": round(time.perf_counter() - t0, 3), "launches": n,
            "what": "the same call, back to back, before the warm-up steps (engine clock to "
                    "its steady state under this load)"}


def bench_fp8(args, torch, fa, w) -> int:
    """Time fa_fwd_fp8 on the 8-bit workload; one JSON line."""
    dev = torch.device("cuda:0")
    fa.load()
    (qc, kc, vc), ds = W.make_fp8_inputs(w)
    q, k, v = (torch.from_numpy(x).to(dev) for x in (qc, kc, vc))
    o = torch.empty((w.B, w.H, w.S, w.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)

    def step():
        fa.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      w.B, w.H, w.S, w.D, int(w.causal), w.scale, ds[0], ds[1], ds[2],
                      stream.cuda_stream)

    torch.cuda.synchronize()
    if args.calibrate_copy:
        calibrate_copy(torch, dev, stream)
    settled = settle(step, torch, args.settle_s)
    ms, wall, med, clk = timed(step, stream, torch, args.steps, args.warmup)
    assert bool(torch.isfinite(lse).all()), "non-finite output"
    tflops = w.flops / (ms * 1e-3) / 1e12
    print(f"Average Time Per Step:     {ms:.4f} ms\n"
          f"Compute Performance:       {tflops:.2f} TFLOPS ({100 * tflops / PEAK_TFLOPS_FP8:.1f}% "
          f"of {PEAK_TFLOPS_FP8} fp8 peak)\n"
          f"Median single launch:      {med:.4f} ms", file=sys.stderr, flush=True)
    groups = w.B * w.H * -(-w.S // 256)
    roofline = {"bound": "mfma", "achieved": tflops, "peak": PEAK_TFLOPS_FP8, "unit": "TFLOP/s",
                "frac": tflops / PEAK_TFLOPS_FP8, "traffic": load_traffic(w.name),
                "kernel": f"fa_fwd_il8<D={w.D},causal={int(w.causal)}> ({groups} work-groups x "
                          f"512 threads, 256 query rows, {64 if w.D == 128 else 128}-key tiles)",
                "flops_per_launch": w.flops, "avg_launch_ms": ms, "median_launch_ms": med,
                "algorithmic_bytes_per_launch": w.algorithmic_bytes,
                "algorithmic_gbs": w.algorithmic_bytes / (ms * 1e-3) / 1e9}
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, qc, kc, vc, descale=ds)
    out = {
        "metric": "attention fwd TFLOPS (B·H·S²·D·4, causal halved) + % of fp8 MFMA peak",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "e4m3",
        "data": "synthetic: seeded N(0,1) Q/K/V, per-tensor scaled to E4M3",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} S={w.S} D={w.D} e4m3 inputs, bf16 "
                               f"output, {'causal' if w.causal else 'non-causal'}",
                   "B": w.B, "H": w.H, "S": w.S, "D": w.D, "causal": w.causal,
                   "descales": list(ds), "parallelism": "single GPU"},
        "pct_of_peak": 100 * tflops / PEAK_TFLOPS_FP8,
        **clock_fields(tflops, PEAK_TFLOPS_FP8, clk),
        "settle": settled,
        "wall_s": wall,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_varlen(args, torch, fa) -> int:
    """Time fa_fwd_varlen on the packed variable-length batch; one JSON line."""
    w = W.VARLEN
    dev = torch.device("cuda:0")
    fa.load()
    cu, qb, kb, vb = W.make_varlen_inputs(w)
    L = w.lengths()
    total = int(cu[-1])
    q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
               for x in (qb, kb, vb))
    cu_d = torch.from_numpy(cu).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.H, total), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    st = [w.D, w.H * w.D] * 4 + [total]

    def step():
        fa.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         cu_d.data_ptr(), cu_d.data_ptr(), w.B, w.H, int(L.max()), int(L.max()),
                         total, total, w.D, int(w.causal), w.scale, stream.cuda_stream,
                         W.DTYPE_CODE[w.dtype], st)

    settled = settle(step, torch, args.settle_s)
    ms, wall, med, clk = timed(step, stream, torch, args.steps, args.warmup)
    assert bool(torch.isfinite(lse).all()), "non-finite output"
    tflops = w.flops() / (ms * 1e-3) / 1e12
    print(f"Average Time Per Step:     {ms:.4f} ms\n"
          f"Compute Performance:       {tflops:.2f} TFLOPS ({100 * tflops / PEAK_TFLOPS:.1f}% of "
          f"{PEAK_TFLOPS} peak)", file=sys.stderr, flush=True)
    out = {
        "metric": "varlen attention fwd TFLOPS (sum over sequences of H·L²·D·4, causal halved)",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic: seeded N(0,1) Q/K/V, "
        "seeded uniform lengths",
        "config": {"workload": f"varlen: {w.B} causal sequences, lengths uniform in "
                               f"[{w.lo}, {w.hi}] (seed {w.seed}; {total} tokens), H={w.H} "
                               f"D={w.D} {w.dtype}, packed [total, H, D]",
                   "lengths": [int(x) for x in L], "parallelism": "single GPU"},
        "pct_of_peak": 100 * tflops / PEAK_TFLOPS,
        **clock_fields(tflops, PEAK_TFLOPS, clk),
        "settle": settled,
        "wall_s": wall,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_TFLOPS, "traffic": None,
                     "flops_per_launch": w.flops(), "avg_launch_ms": ms,
                     "median_launch_ms": med},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
