"""Throughput of the grouped-linear hot path on one MI355X.

A step is one pass of the whole path over one batch of seeded synthetic input:
split-offset scan, grouped forward (+bias), dgrad, wgrad, bias grad, on the
8-group bf16 workload (G=8, K=4096, N=14336, 16384 rows, multinomial splits).
``value`` is the algorithmic fwd+dgrad+wgrad flops (6*T*N*K) per step divided by
the measured time of a whole step (scan and bias grad included), in TFLOP/s,
with all inputs resident in HBM before timing starts.

Also reported on the same line: per-pass kernel times from HIP events on the
launch stream, the roofline entry of the dominant kernel, the MXFP8 forward on
its own workload (G=32, K=N=4096, 32768 rows), and the CPU oracle timed on a
bounded sample of the same workload.

Also: the grouped MLP on the 8-group split, and two more workloads at full size
(64 Zipf-skewed groups with wgrad into an fp32 main_grad; 256 groups forward into a
caller buffer with per-group weights), each against its roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-mxfp8] [--no-mlp] [--no-workloads]
                    [--no-cpu-baseline] [--workloads-only]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 / MXFP8 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "grouped GEMM TFLOP/s (fwd+dgrad+wgrad) and % of MFMA peak, bf16 & MXFP8"
# every source the GEMM kernels are compiled from (the counter records are tied to them)
GEMM_SRCS = [os.path.join(ROOT, "grouped_gemm_gl_amd", "csrc", f)
             for f in ("gl_gemm_tile.hpp", "gl_gemm_bf16.hip", "gl_gemm_mxfp8.hip", "gl_common.hpp",
                       "gl_offsets.hpp")]
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
# kernel-name fragment of each pass's GEMM (template arguments <A K-major, B K-major, mode,
# fp16, schedule, bias grad>)
PASS_KERNELS = {"forward": "gemm_bf16_kernel<true, true, 0, false, 0, false>",
                "dgrad": "gemm_bf16_kernel<true, false, 0, false, 1, false>",
                "wgrad_bgrad": "gemm_bf16_kernel<false, false, 1, false, 1, true>"}
PASS_WORKLOAD = {k: "bf16_train_g8_k4096_n14336" for k in PASS_KERNELS}
# the GEMM passes of the other full-size workloads (bench.py --workloads-only NAME runs one)
WORKLOAD_KERNELS = {
    "bf16_zipf_g64_k2048_n1536": {"forward": PASS_KERNELS["forward"], "dgrad": PASS_KERNELS["dgrad"],
                                  "wgrad_main_grad": "gemm_bf16_kernel<false, false, 1, false, 1, false>"},
    # groups of 128 rows on average: the forward's schedule with the deeper weight ring
    "bf16_fwd_g256_k7168_n2048_outbuf": {"forward": "gemm_bf16_kernel<true, true, 0, false, 2, false>"},
}
GEMM_PASSES = tuple(PASS_KERNELS)
COPY_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken
    on the current kernel source; otherwise None."""
    try:
        rec = json.load(open(TRAFFIC_JSON))[f"{workload}:{kernel}"]
    except Exception:
        return None
    if rec.get("source_sha") != source_hash(GEMM_SRCS):
        return None
    return rec.get("bytes_per_launch")


def calibrate_copy():
    """A plain 1 GiB device-to-device copy, three times: the known-size workload
    that scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch

    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}))


def _pmc_rows(path, counter):
    import csv

    out = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            out.append((r["Kernel_Name"], float(r["Counter_Value"]),
                        int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return out


def _mx_traffic_kernels():
    """(table key, kernel-name fragment, algorithmic bytes) of the MXFP8 block's kernels
    that run at a single shape there (the others mix shapes in one average): codes
    1 B and one E8M0 byte per 32 codes; the columnwise layout holds every group's rows
    padded to 128."""
    import synth

    wl = synth.WORKLOADS["mxfp8_fwd_g32_k4096_n4096"]
    G, K, N, T = wl.G, wl.K, wl.N, wl.T
    ld = (T + 127 * G + 127) // 128 * 128
    codes = lambda r, c: r * c + r * c // 32
    return [(f"{wl.name}:offsets_quantize_x", "offsets_quantize_mxfp8_kernel", T * K * 2 + codes(T, K) + 8 * G),
            (f"{wl.name}:offsets_quantize_x_both", "quantize_mxfp8_colwise_tile_kernel<true>",
             T * K * 2 + codes(T, K) + codes(K, ld) + 8 * G),
            (f"{wl.name}:mx_forward_and_dgrad", "gemm_mxfp8_kernel<0,", codes(T, K) + codes(G * N, K) + T * N * 2),
            (f"{wl.name}:mx_wgrad", "gemm_mxfp8_kernel<2,", codes(N, ld) + codes(K, ld) + G * N * K * 2)]


def summarize_pmc(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, workload=None):
    """Turn two rocprofv3 --pmc runs of the benchmark (FETCH_SIZE, WRITE_SIZE, in KiB
    per dispatch) into HBM bytes per launch of each pass's GEMM kernel, each counter
    scaled by what it reads for the plain copy of known size; writes the result into
    the traffic table keyed by workload and pass, with the kernel source hash."""

    def copy_factor(path, counter):
        vals = [v for k, v, _ in _pmc_rows(path, counter) if "copy" in k.lower()]
        if not vals:
            raise SystemExit(f"no copy kernel with {counter} in {path}")
        return COPY_BYTES / (sum(vals) / len(vals) * 1024.0)

    ff = copy_factor(copy_fetch_csv, "FETCH_SIZE")
    fw = copy_factor(copy_write_csv, "WRITE_SIZE")
    # this workload's passes get new traffic fields; fields of a clock run on the same
    # source survive, anything taken on another source is dropped
    table = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    sha = source_hash(GEMM_SRCS)
    lines = [f"copy calibration ({COPY_BYTES} B): FETCH_SIZE x{ff:.3f}, WRITE_SIZE x{fw:.3f}"]
    passes = WORKLOAD_KERNELS[workload] if workload else PASS_KERNELS
    for name, args in passes.items():
        sel = lambda rows: [v for k, v, _ in rows if args in k]
        fv, wv = sel(_pmc_rows(fetch_csv, "FETCH_SIZE")), sel(_pmc_rows(write_csv, "WRITE_SIZE"))
        if not fv or not wv:
            continue
        fb = sum(fv) / len(fv) * 1024.0 * ff
        wb = sum(wv) / len(wv) * 1024.0 * fw
        wname = workload or PASS_WORKLOAD[name]
        entry = table.get(f"{wname}:{name}", {})
        if entry.get("source_sha") != sha:
            entry = {}
        entry.update({"bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                      "launches": len(fv), "source_sha": sha, "fetch_factor": round(ff, 4),
                      "write_factor": round(fw, 4)})
        table[f"{wname}:{name}"] = entry
        lines.append(f"{wname}:{name}: fetch {fb / 1e9:.3f} GB + write {wb / 1e9:.3f} GB per launch "
                     f"({len(fv)} launches)")
    # the MXFP8 block's single-shape kernels, when the runs included it: bytes per launch
    # and the rate they imply over the same run's dispatch durations
    for key, frag, alg in ([] if workload else _mx_traffic_kernels()):
        fr = [(v, d) for k, v, d in _pmc_rows(fetch_csv, "FETCH_SIZE") if frag in k]
        wr = [(v, d) for k, v, d in _pmc_rows(write_csv, "WRITE_SIZE") if frag in k]
        if not fr or not wr:
            continue
        fb = sum(v for v, _ in fr) / len(fr) * 1024.0 * ff
        wb = sum(v for v, _ in wr) / len(wr) * 1024.0 * fw
        dur = (sum(d for _, d in fr) + sum(d for _, d in wr)) / (len(fr) + len(wr)) * 1e-9
        entry = table.get(key, {})
        if entry.get("source_sha") != sha:
            entry = {}
        entry.update({"bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                      "algorithmic_bytes": alg, "launches": len(fr), "source_sha": sha,
                      "counter_gbs": round((fb + wb) / dur / 1e9, 1), "fetch_factor": round(ff, 4),
                      "write_factor": round(fw, 4)})
        table[key] = entry
        lines.append(f"{key}: fetch {fb / 1e9:.3f} GB + write {wb / 1e9:.3f} GB per launch, algorithmic "
                     f"{alg / 1e9:.3f} GB, {(fb + wb) / dur / 1e9:.0f} GB/s over the counter run's durations")
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print("\n".join(lines))


CLOCK_COUNTERS = "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE"
N_XCD, N_CU, BF16_FLOP_PER_CLK_CU, FP8_FLOP_PER_CLK_CU = 8, 256, 4096, 8192
# (table key, kernel-name fragment, workload, dense flop per clock per CU) of every GEMM
# the clock run covers; the MXFP8 forward and dgrad share one kernel and one shape
CLOCK_KERNELS = [(f"bf16_train_g8_k4096_n14336:{k}", v, "bf16_train_g8_k4096_n14336", BF16_FLOP_PER_CLK_CU)
                 for k, v in PASS_KERNELS.items()] + [
    ("mxfp8_fwd_g32_k4096_n4096:mx_forward_and_dgrad", "gemm_mxfp8_kernel<0,", "mxfp8_fwd_g32_k4096_n4096",
     FP8_FLOP_PER_CLK_CU),
    ("mxfp8_fwd_g32_k4096_n4096:mx_wgrad", "gemm_mxfp8_kernel<2,", "mxfp8_fwd_g32_k4096_n4096", FP8_FLOP_PER_CLK_CU)]


def summarize_clock(pmc_csv, workload=None):
    """Fold one rocprofv3 --pmc run of the benchmark with CLOCK_COUNTERS into the
    traffic table: the engine clock each pass's GEMM ran at (GRBM_GUI_ACTIVE is
    summed over the XCDs, so cycles = value / 8, divided by the dispatch's duration),
    the flops it reached as a fraction of the dense peak of its type at that clock, the MFMA
    busy share of SIMD-cycles, and LDS bank-conflict cycles per LDS-active cycle."""
    table = json.load(open(TRAFFIC_JSON))
    sha = source_hash(GEMM_SRCS)
    rows = {}
    for counter in CLOCK_COUNTERS.split():
        rows[counter] = _pmc_rows(pmc_csv, counter)
    import synth

    lines = [f"{'workload:pass':48s} {'sclk GHz':>9s} {'frac@sclk':>10s} {'MFMA busy':>10s} {'LDS conflicts':>14s}"]
    kernels = ([(f"{workload}:{k}", v, workload, BF16_FLOP_PER_CLK_CU) for k, v in WORKLOAD_KERNELS[workload].items()]
               if workload else CLOCK_KERNELS)
    for key, args, wname, flop_clk in kernels:
        sel = {c: [(v, d) for k, v, d in r if args in k] for c, r in rows.items()}
        if not all(sel.values()):
            continue
        mean = {c: sum(v for v, _ in x) / len(x) for c, x in sel.items()}
        dur_ns = sum(d for _, d in sel["GRBM_GUI_ACTIVE"]) / len(sel["GRBM_GUI_ACTIVE"])
        cycles = mean["GRBM_GUI_ACTIVE"] / N_XCD
        sclk = cycles / dur_ns
        wl = synth.WORKLOADS[wname]
        flops = 2.0 * wl.T * wl.N * wl.K
        frac = flops / (dur_ns * 1e-9) / (N_CU * flop_clk * sclk * 1e9)
        mfma = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * N_CU * 4)
        lds = mean["SQ_LDS_BANK_CONFLICT"] / max(mean["SQ_LDS_IDX_ACTIVE"], 1.0)
        entry = table.get(key, {})
        if entry.get("source_sha") != sha:
            entry = {"source_sha": sha}
        entry.update({"sclk_ghz": round(sclk, 3), "frac_of_peak_at_sclk": round(frac, 4),
                      "mfma_busy_frac": round(mfma, 4), "lds_bank_conflict_per_active": round(lds, 5)})
        table[key] = entry
        lines.append(f"{key:48s} {sclk:9.3f} {frac:10.3f} {mfma:10.3f} {lds:14.5f}")
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print("\n".join(lines))


def clock_for(kernel: str, workload: str):
    """Engine clock and clock-adjusted peak fraction from a committed counter run, if
    it was taken on the current kernel source; otherwise None."""
    try:
        rec = json.load(open(TRAFFIC_JSON))[f"{workload}:{kernel}"]
    except Exception:
        return None
    if rec.get("source_sha") != source_hash(GEMM_SRCS) or "sclk_ghz" not in rec:
        return None
    return rec


class EventTimer:
    """HIP events recorded on torch's current stream, which is the stream every
    library call is enqueued on."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e))

    def mean_ms(self):
        return {k: sum(s.elapsed_time(e) for s, e in v) / len(v) for k, v in self.pairs.items()}

    def spread_ms(self):
        """median, p10 and p90 of each pass's samples (nearest-rank)."""
        out = {}
        for k, v in self.pairs.items():
            xs = sorted(s.elapsed_time(e) for s, e in v)
            pick = lambda q: xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]
            out[k] = {"median": round(pick(0.5), 4), "p10": round(pick(0.1), 4), "p90": round(pick(0.9), 4)}
        return out

    def sum_spread_ms(self, names):
        """mean, median, p10 and p90 of the per-step sums of the named passes (their
        i-th samples belong to the same step)."""
        cols = [[s.elapsed_time(e) for s, e in self.pairs[k]] for k in names]
        xs = sorted(sum(v) for v in zip(*cols))
        pick = lambda q: xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]
        return {"ms": round(sum(xs) / len(xs), 4), "ms_median": round(pick(0.5), 4), "ms_p10": round(pick(0.1), 4),
                "ms_p90": round(pick(0.9), 4)}


def cpu_baseline(wl, m, x, w, b, dy, min_s=10.0):
    """The oracle, as it stands, on whole groups of the same workload, cycling
    through the groups until at least `min_s` seconds of CPU work; TFLOP/s over the
    same 6*m_g*N*K flops."""
    import numpy as np
    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    off = np.concatenate([[0], np.cumsum(m)])
    done_flops, t_total, rows = 0.0, 0.0, 0
    while t_total < min_s:
        for g in range(wl.G):
            if m[g] == 0:
                continue
            lo, hi = int(off[g]), int(off[g + 1])
            sub_m = [hi - lo]
            xs = x[lo:hi].double().numpy()
            dys = dy[lo:hi].double().numpy()
            wg = w[g:g + 1].double().numpy()
            bg = b[g:g + 1].double().numpy() if b is not None else None
            t0 = time.perf_counter()
            oracle.forward(xs, wg, bg, sub_m)
            oracle.dgrad(dys, wg, sub_m)
            oracle.wgrad(xs, dys, sub_m)
            t_total += time.perf_counter() - t0
            done_flops += 6.0 * (hi - lo) * wl.N * wl.K
            rows += hi - lo
            if t_total >= min_s:
                break
    # context only (not the oracle): the same three products per group in torch fp32 on the CPU
    import torch

    g = next(i for i in range(wl.G) if m[i])
    lo, hi = int(off[g]), int(off[g + 1])
    xs, dys, wg = x[lo:hi].float(), dy[lo:hi].float(), w[g].float()
    bg = b[g].float() if b is not None else 0.0
    f32_flops, f32_s = 0.0, 0.0
    while f32_s < 2.0:
        t0 = time.perf_counter()
        _ = xs @ wg.T + bg
        _ = dys @ wg
        _ = dys.T @ xs
        f32_s += time.perf_counter() - t0
        f32_flops += 6.0 * (hi - lo) * wl.N * wl.K
    model = ""
    try:
        model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except Exception:  # pragma: no cover
        pass
    return {"value": round(done_flops / t_total / 1e12, 4), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"oracle fp64 forward+dgrad+wgrad, group by group, over {rows} rows of the same workload "
                      f"({rows / wl.T:.2f}x its {wl.T} rows), {t_total:.1f} s",
            "cpu_model": model, "host_cpus": os.cpu_count(),
            "context_torch_f32": {"value": round(f32_flops / f32_s / 1e12, 4), "unit": "TFLOP/s",
                                  "threads": torch.get_num_threads(),
                                  "sample": f"group {g} ({hi - lo} rows), {f32_s:.1f} s"}}


def bench_bf16(torch, gl, synth, steps, warmup):
    wl = synth.WORKLOADS["bf16_train_g8_k4096_n14336"]
    dev = torch.device("cuda")
    t0 = time.time()
    m = synth.split_sizes(wl)
    x, w, b, dy = synth.x(wl), synth.weight(wl), synth.bias(wl), synth.dy(wl)
    log(f"inputs generated in {time.time() - t0:.1f}s; m_splits={m.tolist()}")
    xd, wd, bd, dyd = (t.to(dev) for t in (x, w, b, dy))
    md = torch.from_numpy(m).to(dev)
    G, K, N, T = wl.G, wl.K, wl.N, wl.T
    ws = gl.new_workspace(G, dev)
    y = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    dx = torch.empty(T, K, dtype=torch.bfloat16, device=dev)
    dw = torch.empty(G, N, K, dtype=torch.bfloat16, device=dev)
    db = torch.empty(G, N, dtype=torch.bfloat16, device=dev)
    timer = EventTimer(torch)

    def step(t=None):
        # the whole path: offsets, forward (+bias), dgrad, wgrad with the bias grad
        # summed from the same dy stages (one pass over dy)
        run = (lambda n, f: t.run(n, f)) if t else (lambda n, f: f())
        run("offsets", lambda: gl.gl_offsets(md, T, ws))
        run("forward", lambda: gl.gl_forward(xd, wd, y, ws, bias=bd))
        run("dgrad", lambda: gl.gl_dgrad(dyd, wd, dx, ws))
        run("wgrad_bgrad", lambda: gl.gl_wgrad_bgrad(xd, dyd, dw, db, ws))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if gl.gl_read_status(ws) != 0:
        raise RuntimeError("invalid split sizes")
    # whole-step wall time (no per-kernel events inside)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    # per-kernel durations on the launch stream
    queue = gl.WgradQueue()
    for _ in range(max(3, min(steps, 30))):
        step(timer)
        # for reference, outside the step: wgrad and the bias grad as separate launches,
        # and the step's wgrad put in the deferred-wgrad queue, then run from it
        timer.run("wgrad_alone", lambda: gl.gl_wgrad(xd, dyd, dw, ws))
        timer.run("bgrad_alone", lambda: gl.gl_bgrad(dyd, db, ws))
        queue.put(xd, dyd, dw, ws, db=db)
        timer.run("wgrad_bgrad_deferred", queue.flush)
    torch.cuda.synchronize()
    # host cost of recording a call: median of single puts (a mean over a loop also
    # catches the interpreter's occasional garbage-collection pass)
    put_times = []
    for _ in range(200):
        t_put = time.perf_counter()
        queue.put(xd, dyd, dw, ws, db=db)
        put_times.append(time.perf_counter() - t_put)
    put_us = sorted(put_times)[len(put_times) // 2] * 1e6
    queue.clear()
    per = timer.mean_ms()
    spread = timer.spread_ms()
    flops_pass = 2.0 * T * N * K
    ms_step = elapsed * 1e3 / steps
    value = 3 * flops_pass / (ms_step * 1e-3) / 1e12
    passes = {}
    for k, ms in per.items():
        d = {"ms": round(ms, 4), "ms_median": spread[k]["median"], "ms_p10": spread[k]["p10"],
             "ms_p90": spread[k]["p90"]}
        if k in GEMM_PASSES or k in ("wgrad_alone", "wgrad_bgrad_deferred"):
            d["tflops"] = round(flops_pass / (ms * 1e-3) / 1e12, 2)
            d["pct_bf16_peak"] = round(100 * d["tflops"] / PEAK_BF16_TFLOPS, 2)
        if k == "bgrad_alone":
            gbs = (T * N * 2 + G * N * 2) / (ms * 1e-3) / 1e9
            d["gbs"] = round(gbs, 1)
            d["pct_hbm"] = round(100 * gbs / PEAK_HBM_GBS, 2)
        if k == "offsets":
            d["us"] = round(ms * 1e3, 2)
        if k == "wgrad_bgrad_deferred":
            d["host_put_us"] = round(put_us, 2)
        passes[k] = d
    dom = max(GEMM_PASSES, key=lambda k: per[k])
    achieved = flops_pass / (per[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": f"{PASS_KERNELS[dom]} ({dom})", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(dom, wl.name),
                "algorithmic_flops_per_launch": flops_pass}
    clk = clock_for(dom, wl.name)
    if clk:
        # the same achieved rate against the peak at the clock the counter run measured
        peak_sclk = N_CU * BF16_FLOP_PER_CLK_CU * clk["sclk_ghz"] * 1e9 / 1e12
        roofline["measured_sclk_ghz"] = clk["sclk_ghz"]
        roofline["frac_at_measured_sclk"] = round(achieved / peak_sclk, 4)
        roofline["mfma_busy_frac"] = clk["mfma_busy_frac"]
    fdw = timer.sum_spread_ms(GEMM_PASSES)
    fdw["tflops"] = round(3 * flops_pass / (fdw["ms"] * 1e-3) / 1e12, 2)
    fdw["pct_bf16_peak"] = round(100 * fdw["tflops"] / PEAK_BF16_TFLOPS, 2)
    return wl, m, (x, w, b, dy), {
        "value": value, "ms_per_step": ms_step, "passes": passes, "roofline": roofline,
        "fwd_dgrad_wgrad": fdw,
    }


def bench_mxfp8(torch, gl, synth, steps, warmup):
    """MXFP8 forward and backward on the MXFP8 workload (G=32, K=N=4096, 32768 rows).
    Weights are quantized once (rowwise for the forward, columnwise for dgrad) into a
    cached workspace, whose refresh call runs in every step with its no-op flag set;
    activations and grad outputs are quantized inside each timed pass, x together
    with the split-offset scan in one launch."""
    wl = synth.WORKLOADS["mxfp8_fwd_g32_k4096_n4096"]
    dev = torch.device("cuda")
    t0 = time.time()
    m = synth.split_sizes(wl)
    x, w, dy = synth.x(wl).to(dev), synth.weight(wl).to(dev), synth.dy(wl).to(dev)
    log(f"mxfp8 inputs generated in {time.time() - t0:.1f}s")
    G, K, N, T = wl.G, wl.K, wl.N, wl.T
    ws = gl.new_workspace(G, dev)
    md = torch.from_numpy(m).to(dev)
    gl.gl_offsets(md, T, ws)
    noop_set = torch.ones(1, dtype=torch.int32, device=dev)
    noop_clear = torch.zeros(1, dtype=torch.int32, device=dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    xq, xs = torch.empty(T, K, **u8), torch.empty(T, K // 32, **u8)
    wq, wsc = torch.empty(G, N, K, **u8), torch.empty(G, N, K // 32, **u8)
    dq, ds = torch.empty(T, N, **u8), torch.empty(T, N // 32, **u8)
    wtq, wts = torch.empty(G, K, N, **u8), torch.empty(G, K, N // 32, **u8)
    ld = gl.gl_colwise_ld(G, T)
    xtq, xts = torch.empty(K, ld, **u8), torch.empty(K, ld // 32, **u8)
    dytq, dyts = torch.empty(N, ld, **u8), torch.empty(N, ld // 32, **u8)
    y = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    dx = torch.empty(T, K, dtype=torch.bfloat16, device=dev)
    dw = torch.empty(G, N, K, dtype=torch.bfloat16, device=dev)
    gl.gl_quantize_mxfp8_weights(w, wq, wsc, wtq, wts)   # cached quantized weights
    w_copy, dy_copy = torch.empty_like(w), torch.empty_like(dy)
    timer = EventTimer(torch)
    for i in range(warmup + steps):
        t = timer if i >= warmup else None
        run = (lambda n, f: t.run(n, f)) if t else (lambda n, f: f())
        # the step, in training order
        run("offsets_quantize_x_both", lambda: gl.gl_offsets_quantize_mxfp8_rowwise_colwise(md, x, ws, xq, xs,
                                                                                           xtq, xts))
        run("weights_noop", lambda: gl.gl_quantize_mxfp8_weights(w, wq, wsc, wtq, wts, noop_flag=noop_set))
        run("mx_forward", lambda: gl.gl_forward(xq, wq, y, ws, x_scale=xs, w_scale=wsc))
        run("quantize_dy_both", lambda: gl.gl_group_quantize_mxfp8_rowwise_colwise(dy, dq, ds, dytq, dyts, ws, G))
        run("mx_dgrad", lambda: gl.gl_dgrad_mxfp8(dq, ds, wtq, wts, dx, ws))
        run("mx_wgrad", lambda: gl.gl_wgrad_mxfp8(dytq, dyts, xtq, xts, dw, ws, T))
        # quantizers on their own, each on an input no pass just read (no cache warmth)
        run("quantize_w", lambda: gl.gl_group_quantize_mxfp8(w, wq, wsc))
        run("quantize_dy", lambda: gl.gl_group_quantize_mxfp8(dy, dq, ds))
        run("weights_refresh", lambda: gl.gl_quantize_mxfp8_weights(w, wq, wsc, wtq, wts, noop_flag=noop_clear))
        run("quantize_dy_colwise", lambda: gl.gl_group_quantize_mxfp8_colwise(dy, dytq, dyts, ws, G))
        run("quantize_x", lambda: gl.gl_group_quantize_mxfp8(x, xq, xs))
        run("offsets_quantize_x", lambda: gl.gl_offsets_quantize_mxfp8(md, x, ws, xq, xs))
        run("quantize_w_again", lambda: gl.gl_group_quantize_mxfp8(w, wq, wsc))  # evicts x from the caches
        run("quantize_x_colwise", lambda: gl.gl_group_quantize_mxfp8_colwise(x, xtq, xts, ws, G))
        # plain device copies of the same byte counts, the ceiling of a stream that
        # reads and writes about as much as it reads (as the quantizers do)
        run("copy_w", lambda: w_copy.copy_(w))
        run("copy_dy", lambda: dy_copy.copy_(dy))
    torch.cuda.synchronize()
    per = timer.mean_ms()
    flops = 2.0 * T * N * K
    tf = lambda k: round(flops / (per[k] * 1e-3) / 1e12, 2)
    gbs = lambda k, b: round(b / (per[k] * 1e-3) / 1e9, 1)
    row_bytes = lambda r, c: r * c * 2 + r * c + r * c // 32     # bf16 in, codes + scales out
    col_bytes = lambda r, c: r * c * 2 + (r + 127 * G) * c * (1 + 1 / 32)
    out = {"workload": wl.name}
    for k in ("mx_forward", "mx_dgrad", "mx_wgrad"):
        out[f"{k}_ms"] = round(per[k], 4)
        out[f"{k}_tflops"] = tf(k)
        out[f"{k}_pct_fp8_peak"] = round(100 * tf(k) / PEAK_FP8_TFLOPS, 2)
        # against the dense fp8 peak at the clock a committed counter run measured
        clk = clock_for("mx_wgrad" if k == "mx_wgrad" else "mx_forward_and_dgrad", wl.name)
        if clk:
            peak_sclk = N_CU * FP8_FLOP_PER_CLK_CU * clk["sclk_ghz"] * 1e9 / 1e12
            out[f"{k}_pct_fp8_peak_at_measured_sclk"] = round(100 * tf(k) / peak_sclk, 2)
    out["quantize_gbs"] = {"x": gbs("quantize_x", row_bytes(T, K)), "w": gbs("quantize_w", row_bytes(G * N, K)),
                           "dy": gbs("quantize_dy", row_bytes(T, N)),
                           "x_colwise": gbs("quantize_x_colwise", col_bytes(T, K)),
                           "dy_colwise": gbs("quantize_dy_colwise", col_bytes(T, N)),
                           "dy_rowwise_and_colwise": gbs("quantize_dy_both",
                                                         row_bytes(T, N) + col_bytes(T, N) - T * N * 2),
                           "offsets_and_x": gbs("offsets_quantize_x", row_bytes(T, K)),
                           "offsets_and_x_both": gbs("offsets_quantize_x_both",
                                                     row_bytes(T, K) + col_bytes(T, K) - T * K * 2),
                           "w_rowwise_and_colwise": gbs("weights_refresh", G * N * K * (2 + 2 * (1 + 1 / 32)))}
    out["copy_gbs"] = {"dy": gbs("copy_dy", 2 * T * N * 2), "w": gbs("copy_w", 2 * G * N * K * 2),
                       "note": "device copy of dy / w into a buffer of its size, bytes read + written"}
    out["launch_us"] = {"offsets_quantize_x": round(per["offsets_quantize_x"] * 1e3, 1),
                        "offsets_quantize_x_both_ways": round(per["offsets_quantize_x_both"] * 1e3, 1),
                        "quantize_x": round(per["quantize_x"] * 1e3, 1),
                        "weights_with_noop_flag_set": round(per["weights_noop"] * 1e3, 1)}
    # forward alone, end to end: offsets with x's rowwise quantization (one launch), the
    # cached-weight refresh skipped by its flag, the MX GEMM
    fwd_e2e = per["offsets_quantize_x"] + per["weights_noop"] + per["mx_forward"]
    out["forward_with_quantize_ms"] = round(fwd_e2e, 4)
    out["forward_with_quantize_tflops"] = round(flops / (fwd_e2e * 1e-3) / 1e12, 2)
    step = ("offsets_quantize_x_both", "weights_noop", "mx_forward", "quantize_dy_both", "mx_dgrad", "mx_wgrad")
    step_ms = sum(per[k] for k in step)
    out["mx_step_ms"] = round(step_ms, 4)
    out["mx_step_tflops"] = round(3 * flops / (step_ms * 1e-3) / 1e12, 2)
    out["mx_step"] = ("offsets + quantize x rowwise and columnwise (one launch), cached-weight refresh skipped "
                      "by its no-op flag, MX forward, quantize dy rowwise and columnwise in one pass, MX dgrad, "
                      "MX wgrad")
    return out


def bench_mlp(torch, gl, steps, warmup):
    """Grouped MLP (FC1 -> SwiGLU -> FC2) on the 8-group token split: FC1 has the
    8-group workload's shape (K=4096 -> 2F=14336), FC2 maps F=7168 -> N=4096.
    Forward and backward (with both bias grads fused into the wgrads) per step."""
    import synth
    wl = synth.WORKLOADS["bf16_train_g8_k4096_n14336"]
    dev = torch.device("cuda")
    G, T, K, F, N = wl.G, wl.T, wl.K, wl.N // 2, wl.K
    m = synth.split_sizes(wl)
    g = torch.Generator(device=dev).manual_seed(5)
    bf = torch.bfloat16
    r = lambda *s, std=1.0: (torch.randn(*s, generator=g, device=dev) * std).to(bf)
    x, dy = r(T, K), r(T, N)
    w1, b1, w2, b2 = r(G, 2 * F, K, std=0.02), r(G, 2 * F, std=0.1), r(G, N, F, std=0.02), r(G, N, std=0.1)
    h, a, y = (torch.empty(T, c, dtype=bf, device=dev) for c in (2 * F, F, N))
    da, dh, dx = (torch.empty(T, c, dtype=bf, device=dev) for c in (F, 2 * F, K))
    dw1, dw2 = torch.empty_like(w1), torch.empty_like(w2)
    db1, db2 = torch.empty_like(b1), torch.empty_like(b2)
    ws = gl.new_workspace(G, dev)
    gl.gl_offsets(torch.from_numpy(m).to(dev), T, ws)
    timer = EventTimer(torch)
    for i in range(warmup + steps):
        run = (lambda n, f: timer.run(n, f)) if i >= warmup else (lambda n, f: f())
        run("forward", lambda: gl.gl_grouped_mlp_forward(x, w1, w2, h, a, y, ws, b1=b1, b2=b2))
        run("backward", lambda: gl.gl_grouped_mlp_backward(x, w1, w2, h, a, dy, da, dh, dx, dw1, dw2, ws,
                                                           db1=db1, db2=db2))
        run("swiglu_forward", lambda: gl.gl_swiglu_forward(h, a))
        run("swiglu_backward", lambda: gl.gl_swiglu_backward(h, da, dh))
    torch.cuda.synchronize()
    per = timer.mean_ms()
    fwd_flops = 2.0 * T * (K * 2 * F + F * N)
    tf = lambda fl, ms: round(fl / (ms * 1e-3) / 1e12, 2)
    return {"config": {"num_groups": G, "total_rows": T, "in_features": K, "ffn_features": F, "out_features": N,
                       "activation": "swiglu", "bias": True},
            "forward_ms": round(per["forward"], 4), "forward_tflops": tf(fwd_flops, per["forward"]),
            "backward_ms": round(per["backward"], 4), "backward_tflops": tf(2 * fwd_flops, per["backward"]),
            "step_tflops": tf(3 * fwd_flops, per["forward"] + per["backward"]),
            "swiglu_gbs": {"forward": round(T * 3 * F * 2 / (per["swiglu_forward"] * 1e-3) / 1e9, 1),
                           "backward": round(T * 5 * F * 2 / (per["swiglu_backward"] * 1e-3) / 1e9, 1)}}


def bench_workloads(torch, gl, synth, steps, warmup, names=None):
    """The skewed 64-group workload (forward, dgrad, wgrad added into an fp32
    main_grad) and the 256-group forward into a caller buffer with per-group weight
    pointers, at full size (or only the named ones).  Split sizes come from the seeded
    recipe; the values are drawn on the device (torch.randn, bf16), since throughput
    does not depend on them and the host recipe would spend most of the run making
    7.5 GB of weights.  Each pass is reported against both rooflines, and with the
    HBM traffic and engine clock of the committed counter runs while their kernel
    source hash matches."""
    for name in names or ():
        if name not in WORKLOAD_KERNELS:
            raise SystemExit(f"unknown workload {name}; one of {sorted(WORKLOAD_KERNELS)}")
    run_wl = lambda name: names is None or name in names
    dev = torch.device("cuda")
    bf = torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(7)
    out = {}
    gbs = lambda nbytes, ms: round(nbytes / (ms * 1e-3) / 1e9, 1)
    tf = lambda fl, ms: round(fl / (ms * 1e-3) / 1e12, 2)

    def pass_entry(wname, k, fl, nb, ms):
        d = {"ms": round(ms, 4), "tflops": tf(fl, ms),
             "pct_bf16_peak": round(100 * fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
             "gbs": gbs(nb, ms), "pct_hbm": round(100 * nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
             "algorithmic_bytes": nb}
        tr = traffic_for(k, wname)
        if tr:
            d["traffic_bytes"] = tr
            d["traffic_over_algorithmic"] = round(tr / nb, 3)
        ck = clock_for(k, wname)
        if ck:
            d["measured_sclk_ghz"] = ck["sclk_ghz"]
            d["mfma_busy_frac"] = ck["mfma_busy_frac"]
        return d

    wl = synth.WORKLOADS["bf16_zipf_g64_k2048_n1536"]
    if run_wl(wl.name):
        G, K, N, T = wl.G, wl.K, wl.N, wl.T
        m = synth.split_sizes(wl)
        x = torch.randn(T, K, generator=g, device=dev, dtype=bf)
        dy = torch.randn(T, N, generator=g, device=dev, dtype=bf)
        w = torch.randn(G, N, K, generator=g, device=dev, dtype=bf) * 0.02
        mg = torch.randn(G, N, K, generator=g, device=dev)
        y = torch.empty(T, N, dtype=bf, device=dev)
        dx = torch.empty(T, K, dtype=bf, device=dev)
        ws = gl.new_workspace(G, dev)
        gl.gl_offsets(torch.from_numpy(m).to(dev), T, ws)
        timer = EventTimer(torch)
        for i in range(warmup + steps):
            run = (lambda n, f: timer.run(n, f)) if i >= warmup else (lambda n, f: f())
            run("forward", lambda: gl.gl_forward(x, w, y, ws))
            run("dgrad", lambda: gl.gl_dgrad(dy, w, dx, ws))
            run("wgrad_main_grad", lambda: gl.gl_wgrad(x, dy, mg, ws, accumulate=True))
        torch.cuda.synchronize()
        per = timer.mean_ms()
        fl = 2.0 * T * N * K
        gemm_bytes = (T * K + G * N * K + T * N) * 2
        wgrad_bytes = (T * K + T * N) * 2 + 2 * G * N * K * 4
        d = {"num_groups": G, "in_features": K, "out_features": N, "total_rows": T, "largest_group": int(m.max()),
             "empty_groups": int((m == 0).sum())}
        for k in ("forward", "dgrad", "wgrad_main_grad"):
            d[k] = pass_entry(wl.name, k, fl, wgrad_bytes if k == "wgrad_main_grad" else gemm_bytes, per[k])
        d["fwd_dgrad_wgrad_tflops"] = tf(3 * fl, sum(per[k] for k in ("forward", "dgrad", "wgrad_main_grad")))
        out[wl.name] = d
        del x, dy, w, mg, y, dx

    wl = synth.WORKLOADS["bf16_fwd_g256_k7168_n2048_outbuf"]
    if run_wl(wl.name):
        G, K, N, T = wl.G, wl.K, wl.N, wl.T
        m = synth.split_sizes(wl)
        x = torch.randn(T, K, generator=g, device=dev, dtype=bf)
        w = torch.randn(G, N, K, generator=g, device=dev, dtype=bf) * 0.02
        w_list = list(w)  # per-group weight pointers
        rows = wl.out_rows
        y = torch.full((rows, N), float("nan"), dtype=bf, device=dev)
        ws = gl.new_workspace(G, dev)
        gl.gl_offsets(torch.from_numpy(m).to(dev), T, ws)
        timer = EventTimer(torch)
        for i in range(warmup + steps):
            run = (lambda n, f: timer.run(n, f)) if i >= warmup else (lambda n, f: f())
            run("forward", lambda: gl.gl_forward(x, w_list, y, ws))
        torch.cuda.synchronize()
        if not bool(torch.isnan(y[T:]).all()):
            raise RuntimeError("the caller buffer's tail was written")
        ms = timer.mean_ms()["forward"]
        nb = (T * K + G * N * K + T * N) * 2
        fl = 2.0 * T * N * K
        out[wl.name] = {"num_groups": G, "in_features": K, "out_features": N, "total_rows": T, "output_rows": rows,
                        "weights": "per-group pointers", "forward": pass_entry(wl.name, "forward", fl, nb, ms)}
    return out


def bench_small_fp32(torch, gl, synth, reps=200, warmup=20):
    """Latency of the fp32 workload (4 groups, K=64, N=32, 32 rows, one empty group):
    a forward is a launch of a few microseconds, not a throughput figure.  Timed per
    call with HIP events on the launch stream: the forward alone (offsets already in
    the workspace) and the offsets scan + forward; median, p10 and p90 in
    microseconds."""
    wl = synth.WORKLOADS["fwd_f32_g4_k64_n32"]
    dev = torch.device("cuda")
    m = synth.split_sizes(wl)
    x, w, b = synth.x(wl).to(dev), synth.weight(wl).to(dev), synth.bias(wl).to(dev)
    md = torch.from_numpy(m).to(dev)
    y = torch.empty(wl.T, wl.N, device=dev)
    ws = gl.new_workspace(wl.G, dev)
    gl.gl_offsets(md, wl.T, ws)
    timer = EventTimer(torch)
    for i in range(warmup + reps):
        run = (lambda n, f: timer.run(n, f)) if i >= warmup else (lambda n, f: f())
        run("forward", lambda: gl.gl_forward(x, w, y, ws, bias=b))
        run("offsets_forward", lambda: (gl.gl_offsets(md, wl.T, ws), gl.gl_forward(x, w, y, ws, bias=b)))
    torch.cuda.synchronize()
    sp = timer.spread_ms()
    us = lambda d: {k: round(v * 1e3, 2) for k, v in d.items()}
    return {"workload": wl.name, "m_splits": m.tolist(), "dtype": "f32", "unit": "us", "calls": reps,
            "forward_us": us(sp["forward"]), "offsets_forward_us": us(sp["offsets_forward"])}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-mxfp8", action="store_true")
    ap.add_argument("--no-mlp", action="store_true")
    ap.add_argument("--no-workloads", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workloads-only", nargs="*", metavar="WORKLOAD", default=None,
                    help="only the 64-group and 256-group workloads, or the named ones (one JSON object; for "
                         "profiling runs)")
    ap.add_argument("--workload", default=None, help="with --summarize-pmc / --summarize-clock: the run was "
                    "--workloads-only WORKLOAD")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB copy (counter calibration)")
    ap.add_argument("--summarize-clock", metavar="PMC_CSV",
                    help=f"fold a rocprofv3 --pmc run with {CLOCK_COUNTERS} into the traffic table, then exit")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="fold rocprofv3 FETCH_SIZE/WRITE_SIZE CSVs into the traffic table, then exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, workload=args.workload)
        return
    if args.summarize_clock:
        summarize_clock(args.summarize_clock, workload=args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(groups would shard across GPUs as expert parallelism).", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return
    import torch
    import grouped_gemm_gl_amd as gl
    import synth

    gl.load()
    if args.workloads_only is not None:
        print(json.dumps({"workloads": bench_workloads(torch, gl, synth, args.steps, args.warmup,
                                                       args.workloads_only or None)}))
        return
    wl, m, host_inputs, r = bench_bf16(torch, gl, synth, args.steps, args.warmup)
    out = {
        "metric": METRIC,
        "value": round(r["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "num_groups": wl.G, "in_features": wl.K, "out_features": wl.N,
                   "total_rows": wl.T, "m_splits": m.tolist(), "bias": True,
                   "step": "offsets+forward(+bias)+dgrad+wgrad(+bias grad, one pass over dy)",
                   "parallelism": "single GPU",
                   "inputs_sha256_16": {"m_splits": synth.checksum(m), "x": synth.checksum(host_inputs[0]),
                                        "W": synth.checksum(host_inputs[1]), "b": synth.checksum(host_inputs[2]),
                                        "dy": synth.checksum(host_inputs[3])}},
        "pct_bf16_peak": round(100 * r["value"] / PEAK_BF16_TFLOPS, 2),
        "passes": r["passes"],
        "fwd_dgrad_wgrad_events": r["fwd_dgrad_wgrad"],
        "roofline": r["roofline"],
    }
    out["small_fp32_latency"] = bench_small_fp32(torch, gl, synth)
    if not args.no_mxfp8:
        out["mxfp8"] = bench_mxfp8(torch, gl, synth, max(5, args.steps // 2), 2)
    if not args.no_mlp:
        out["grouped_mlp"] = bench_mlp(torch, gl, max(5, args.steps // 2), 2)
    if not args.no_workloads:
        out["workloads"] = bench_workloads(torch, gl, synth, max(5, args.steps // 2), 2)
    if not args.no_cpu_baseline:
        x, w, b, dy = host_inputs
        out["cpu_baseline"] = cpu_baseline(wl, m.tolist(), x, w, b, dy)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
