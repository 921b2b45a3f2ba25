#!/usr/bin/env python3
"""Throughput of the packed multi-LoRA operator, forward + backward, on one MI355X.

One step = plora_forward + plora_backward_dx + plora_backward_dAdB over one
batch of synthetic inputs already resident in HBM.  Default workload: the
Llama-3-8B-shaped up projection 4096 -> 14336, bf16, 32 adapters with ranks
cycling 8/16/32/64 and alpha 8/16/32, 2048 tokens each (T = 65536).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload llama_up]
                    [--adapters 32] [--no-cpu] [--sweep]

Prints one JSON line.  ``roofline`` describes the dominant kernel (the base
GEMM with the fused LoRA expand): algorithmic FLOPs per launch over its mean
duration, measured with HIP events recorded by the library on the stream it
launches on.  ``cpu_baseline`` times the fp64 oracle on the host on a bounded
token sample of the same workload.  ``--sweep`` adds one line per adapter
count (2..32, 2048 tokens each) for the scaling curve.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def gemm_flops(wl, which):
    """Algorithmic FLOPs of one launch of the base GEMM with its fused expand."""
    nr = float(np.sum(np.diff(wl.offsets) * wl.ranks)) if wl.n_adapters else 0.0
    base = 2.0 * wl.T * wl.d_in * wl.d_out
    return base + 2.0 * nr * (wl.d_out if which == "gemm_fwd" else wl.d_in)


def step_flops(wl):
    nr = float(np.sum(np.diff(wl.offsets) * wl.ranks)) if wl.n_adapters else 0.0
    return 4.0 * wl.T * wl.d_in * wl.d_out + 6.0 * nr * (wl.d_in + wl.d_out)


def source_sha(path):
    """Hash of a kernel source without its comments and blank lines, so that
    counters stay attached to the code they were taken on."""
    import re
    txt = open(path, encoding="utf-8").read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    txt = re.sub(r"//[^\n]*", "", txt)
    code = "\n".join(ln.rstrip() for ln in txt.splitlines() if ln.strip())
    return hashlib.sha256(code.encode("utf-8")).hexdigest()[:16]


def load_traffic(kernel, wl):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current source of the kernel; else None."""
    f = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(f):
        return None
    try:
        rec = json.load(open(f)).get(kernel)
    except ValueError:
        return None
    if not rec or rec.get("workload") != wl.name or rec.get("tokens") != wl.T:
        return None
    src = os.path.join(ROOT, "packed_adapter_lora_amd", "csrc", rec.get("source", ""))
    if not os.path.exists(src) or source_sha(src) != rec.get("source_sha"):
        return None
    return rec.get("bytes_per_launch")


KERNEL_CLASSES = (("gemm_lora_bf16_pipe<true", "gemm_fwd"), ("gemm_lora_bf16_pipe<false", "gemm_bwd"),
                  ("gemm_lora_bf16<true>", "gemm_fwd"), ("gemm_lora_bf16<false>", "gemm_bwd"),
                  ("shrink_bf16", "shrink"), ("shrink_slice_sum", "shrink_sum"), ("wgrad_reduce", "reduce"),
                  ("wgrad_bf16", "wgrad"), ("wgrad_prep", "wgrad_prep"), ("adamw_panel", "adamw"))


def kernel_class(name):
    for key, cls in KERNEL_CLASSES:
        if key in name:
            return cls
    return None


def rocprof_summary(trace_dir, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes, workload, cmds,
                    mfma_dir=None):
    """Summaries of rocprofv3 csv output: per-kernel time (--kernel-trace --stats) and
    HBM bytes per launch (FETCH_SIZE / WRITE_SIZE), each counter scaled by what it
    reads for a plain device copy of known size."""
    import csv
    import glob

    def rows(d, suffix):
        f = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
        return list(csv.DictReader(open(f[0]))) if f else []

    out = {}
    stats = rows(trace_dir, "kernel_stats.csv")
    # launches of the timed steps only: the last steps / (steps + warmup) of each kernel's launches
    import re
    m = re.search(r"--steps (\d+) --warmup (\d+)", cmds["trace"])
    steps, warm = (int(m.group(1)), int(m.group(2))) if m else (1, 0)
    per_kernel = {}
    for r in rows(trace_dir, "kernel_trace.csv"):
        per_kernel.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = ["# rocprofv3 kernel statistics, workload %s" % workload, "# command: " + cmds["trace"],
             "# timed_avg_us: mean over the launches of the %d timed steps (the first %d warm-up steps' "
             "launches left out)" % (steps, warm), "",
             "%-16s %6s %12s %12s %12s  %s" % ("class", "calls", "total_ms", "avg_us", "timed_avg_us", "kernel")]
    for r in stats:
        cls = kernel_class(r["Name"]) or "-"
        d = per_kernel.get(r["Name"], [])
        keep = d[len(d) - len(d) * steps // (steps + warm):] if d else []
        tavg = "%12.1f" % (sum(keep) / len(keep) / 1e3) if keep else "%12s" % "-"
        lines.append("%-16s %6s %12.3f %12.1f %s  %s" % (cls, r["Calls"], float(r["TotalDurationNs"]) / 1e6,
                                                          float(r["AverageNs"]) / 1e3, tavg, r["Name"][:110]))
    out["stats"] = "\n".join(lines) + "\n"

    def counter(d, cname):
        acc = {}
        for r in rows(d, "counter_collection.csv"):
            if r["Counter_Name"] != cname:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc

    cf, cw = counter(copy_fetch_dir, "FETCH_SIZE"), counter(copy_write_dir, "WRITE_SIZE")
    copy_name = [k for k in cf if "copyBuffer" in k or "copy" in k.lower()]
    kib = copy_bytes / 1024.0
    f_scale = kib / max(v for k in copy_name for v in cf[k])
    w_scale = kib / max(v for k in copy_name if k in cw for v in cw[k])
    fetch, write = counter(fetch_dir, "FETCH_SIZE"), counter(write_dir, "WRITE_SIZE")
    lines = ["# HBM traffic per launch from rocprofv3 counters, workload %s" % workload,
             "# fetch: " + cmds["fetch"], "# write: " + cmds["write"],
             "# copy calibration (%d bytes): %s ; %s" % (copy_bytes, cmds["copy_fetch"], cmds["copy_write"]),
             "# scale: FETCH_SIZE x %.4f, WRITE_SIZE x %.4f (counter KiB -> bytes moved by a plain copy)" % (
                 f_scale, w_scale), "",
             "%-10s %6s %16s %16s %14s" % ("class", "disp", "fetch_MiB", "write_MiB", "total_MiB")]
    traffic = {}
    for name in sorted(set(fetch) | set(write)):
        cls = kernel_class(name)
        if not cls:
            continue
        fv = sum(fetch.get(name, [0])) / max(1, len(fetch.get(name, [0]))) * f_scale * 1024
        wv = sum(write.get(name, [0])) / max(1, len(write.get(name, [0]))) * w_scale * 1024
        lines.append("%-10s %6d %16.1f %16.1f %14.1f" % (cls, len(fetch.get(name, [])), fv / 2 ** 20, wv / 2 ** 20,
                                                          (fv + wv) / 2 ** 20))
        traffic[cls] = {"fetch_bytes": fv, "write_bytes": wv, "bytes_per_launch": fv + wv, "kernel": name}
    out["traffic_txt"] = "\n".join(lines) + "\n"
    out["traffic"] = traffic
    out["scales"] = (f_scale, w_scale)

    # matrix-core utilisation per busy cycle and the clock the kernel ran at:
    # SQ_VALU_MFMA_BUSY_CYCLES counts per SIMD (4 per CU), SQ_BUSY_CU_CYCLES per
    # CU, GRBM_GUI_ACTIVE over the 8 XCDs; the clock divides one XCD's cycles by
    # the kernel-trace duration of the same kernel
    if mfma_dir and os.path.isdir(mfma_dir):
        busy, cu, gui, n = (counter(mfma_dir, c) for c in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES",
                                                            "GRBM_GUI_ACTIVE", "SQ_INSTS_MFMA"))
        avg_ns = {r["Name"]: float(r["AverageNs"]) for r in stats}
        lines = ["# matrix-core busy fraction and effective clock, workload %s" % workload,
                 "# command: " + cmds.get("mfma", ""), "# trace durations: " + cmds["trace"],
                 "# mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES);"
                 " clock = GRBM_GUI_ACTIVE / 8 XCDs / mean kernel-trace duration", "",
                 "%-10s %12s %12s %12s %10s %10s" % ("class", "mfma_insts", "busy_cu_cyc", "cycles/xcd",
                                                     "mfma_util", "clock_GHz")]
        for name in sorted(busy):
            cls = kernel_class(name)
            if not cls:
                continue
            mean = lambda d: sum(d[name]) / len(d[name]) if name in d else float("nan")
            b, c, g = mean(busy), mean(cu), mean(gui)
            ns = avg_ns.get(name, float("nan"))
            lines.append("%-10s %12.4g %12.4g %12.4g %10.3f %10.3f" % (cls, mean(n), c, g / 8, b / (4 * c),
                                                                        g / 8 / ns))
        out["mfma_txt"] = "\n".join(lines) + "\n"

    # LDS and L2 behaviour: LDS instructions and bank-conflict cycles against the
    # cycles the LDS was busy, the share of wave cycles spent waiting to issue an
    # LDS instruction; L2 hit rate and the L2's read requests to the fabric (all,
    # and those the fabric sent to DRAM)
    lds_dir, hit_dir, ea_dir = (os.path.join(os.path.dirname(trace_dir), k) for k in ("lds", "l2hit", "l2ea"))
    if all(os.path.isdir(x) for x in (lds_dir, hit_dir, ea_dir)):
        cl = {c: counter(lds_dir, c) for c in ("SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
                                               "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES")}
        ch = {c: counter(hit_dir, c) for c in ("TCC_HIT_sum", "TCC_MISS_sum")}
        ce = {c: counter(ea_dir, c) for c in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_DRAM_sum")}
        lines = ["# LDS and L2 counters per launch, workload %s" % workload,
                 "# lds: " + cmds.get("lds", ""), "# l2 hit/miss: " + cmds.get("l2hit", ""),
                 "# l2 fabric reads: " + cmds.get("l2ea", ""),
                 "# conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles);"
                 " lds_wait = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES; l2_hit = HIT / (HIT + MISS);"
                 " ea_rd = TCC_EA0_RDREQ_sum, of which dram = TCC_EA0_RDREQ_DRAM_sum", "",
                 "%-10s %12s %9s %9s %8s %12s %12s" % ("class", "lds_insts", "conflict", "lds_wait", "l2_hit",
                                                       "ea_rd", "ea_rd_dram")]
        for name in sorted(cl["SQ_INSTS_LDS"]):
            cls = kernel_class(name)
            if not cls:
                continue
            mean = lambda d: sum(d[name]) / len(d[name]) if name in d else float("nan")
            li, bc, ia, wl_, wc = (mean(cl[c]) for c in ("SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
                                                         "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"))
            hit, miss = mean(ch["TCC_HIT_sum"]), mean(ch["TCC_MISS_sum"])
            ea, dram = mean(ce["TCC_EA0_RDREQ_sum"]), mean(ce["TCC_EA0_RDREQ_DRAM_sum"])
            lines.append("%-10s %12.4g %9.4f %9.4f %8.4f %12.4g %12.4g" % (
                cls, li, bc / ia if ia else float("nan"), wl_ / wc if wc else float("nan"),
                hit / (hit + miss) if hit + miss else float("nan"), ea, dram))
        out["lds_l2_txt"] = "\n".join(lines) + "\n"
    return out


def make_device_inputs(wl):
    import torch
    import workloads
    inp = workloads.make_inputs(wl)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = {k: torch.from_numpy(v).to("cuda").to(dt) for k, v in inp.items()}
    return inp, dev


def workload_label(wl):
    """Name of a workload by the model shape it stands for, its sizes and its
    token mix (uniform: tokens per adapter; otherwise the total)."""
    family = {"tiny": "tiny_fp32", "qwen_q": "qwen2.5_7b_q_proj", "llama_sq": "llama3_8b_square_proj",
              "llama_up": "llama3_8b_up_proj", "longtail": "llama3_8b_up_proj_longtail"}.get(wl.name, wl.name)
    if not wl.n_adapters:
        return family
    counts = wl.counts
    mix = ("x_%d_tokens" % int(counts[0])) if (counts == counts[0]).all() else ("%d_tokens_total" % int(counts.sum()))
    return "%s_%dx%d_%d_adapters_%s" % (family, wl.d_in, wl.d_out, wl.n_adapters, mix)


class Stepper:
    """Buffers and one training step (forward, backward_dx, backward_dAdB) of
    the operator on device inputs `dev` for descriptor `d` (n_adapters = 0
    runs the frozen path only)."""

    def __init__(self, P, d, dev, T, d_in, d_out, R):
        import torch
        self.P, self.d, self.dev = P, d, dev
        he = P.plora_h_elems(d) if R else 0
        dt = dev["X"].dtype
        self.Y = torch.empty((T, d_out), dtype=dt, device="cuda")
        self.dX = torch.empty((T, d_in), dtype=dt, device="cuda")
        self.H = torch.empty((max(he, 4),), dtype=torch.float32, device="cuda")[:he] if R else None
        self.G = torch.empty((max(he, 4),), dtype=torch.float32, device="cuda")[:he] if R else None
        self.dA = torch.empty((max(R, 1), d_in), dtype=torch.float32, device="cuda")[:R]
        self.dB = torch.empty((max(R, 1), d_out), dtype=torch.float32, device="cuda")[:R]
        nb = P.plora_workspace_bytes(d) if R else 0
        self.ws = torch.empty((max(nb, 16),), dtype=torch.uint8, device="cuda")
        self.R = R
        self.stream = torch.cuda.current_stream()

    def step(self):
        P, d, dev, st = self.P, self.d, self.dev, self.stream
        A, B = (dev["A"], dev["B"]) if self.R else (None, None)
        P.plora_forward(d, dev["X"], dev["W"], A, B, self.Y, self.H, st)
        P.plora_backward_dx(d, dev["dY"], dev["W"], A, B, self.dX, self.G, st)
        if self.R:
            P.plora_backward_dAdB(d, dev["X"], dev["dY"], self.H, self.G, self.dA, self.dB, self.ws, st)


def timed_steps(stepper, steps, warmup, flush=None):
    """Wall-clock seconds per step over `steps` steps (synchronised on both
    sides), plus each step's duration from a HIP event pair on the launch
    stream.  flush: a tensor rewritten before every step (evicts L2 and the
    Infinity Cache; the rewrite lies outside the events, and the wall clock
    then includes it, so only the event figures are used)."""
    import torch
    for _ in range(warmup):
        stepper.step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        if flush is not None:
            flush.fill_(float(k))
        ev[k][0].record()
        stepper.step()
        ev[k][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    return (t1 - t0) / steps, per


def summary_ms(per):
    n = len(per)
    return {"median": round(per[n // 2] if n % 2 else 0.5 * (per[n // 2 - 1] + per[n // 2]), 4),
            "mean": round(sum(per) / n, 4), "min": round(per[0], 4), "max": round(per[-1], 4)}


def run_bench(wl, steps, warmup, dev=None):
    """The timed region: `steps` steps after `warmup` with the library's
    per-kernel HIP events on (the roofline's kernel durations).  Returns
    (seconds per step, per-kernel figures, host inputs, stepper)."""
    import torch
    import packed_adapter_lora_amd as P
    inp = None
    if dev is None:
        inp, dev = make_device_inputs(wl)
    d = P.Desc.from_workload(wl)
    stp = Stepper(P, d, dev, wl.T, wl.d_in, wl.d_out, wl.R)
    for _ in range(warmup):
        stp.step()
    torch.cuda.synchronize()
    P.plora_profile_reset()
    P.plora_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        stp.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    P.plora_profile_enable(False)
    kern = {}
    for cls in ("shrink", "gemm_fwd", "gemm_bwd", "wgrad", "reduce"):
        n, ms = P.plora_profile_read(cls)
        kern[cls] = {"launches": n, "mean_ms": (ms / n) if n else 0.0, "ms_per_step": ms / steps}
    P.plora_profile_reset()
    return (t1 - t0) / steps, kern, inp, stp


def measure_ceilings():
    """Measured ceilings (include/plora_probe.h): sustained bf16 matrix-core
    throughput on random register operands, HBM copy and read bandwidth.
    Median of 5 timed launches after one warm-up."""
    import torch
    import packed_adapter_lora_amd as P
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    nb = P.plora_probe_mfma_operand_bytes()
    ops = torch.randn((nb // 2,), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    out = torch.empty((cus * 256,), dtype=torch.float32, device="cuda")

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]

    def sustained(shape, o, seconds=1.5):
        """TFLOP/s of back-to-back launches (a few ms each) over the last half
        of `seconds`, after the power controller has settled."""
        iters, fl = 12000, [0.0]
        fn = lambda: fl.__setitem__(0, P.plora_probe_mfma(o, wg, iters, out, shape=shape))
        t0, n, e0 = time.perf_counter(), 0, None
        while time.perf_counter() - t0 < seconds:
            if e0 is None and time.perf_counter() - t0 > seconds / 2:
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e0.record()
            for _ in range(4):
                fn()
                n += 1 if e0 is not None else 0
            torch.cuda.synchronize()
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record()
        torch.cuda.synchronize()
        return fl[0] * n / (e0.elapsed_time(e1) * 1e-3) / 1e12

    wg = cus  # one wave per SIMD
    t32 = sustained(0, ops)
    t16 = sustained(1, ops)
    t32l = sustained(2, ops)
    zeros = torch.zeros_like(ops)
    z32 = sustained(0, zeros)
    res = {"mfma_bf16_tflops": round(max(t32, t16), 1), "mfma_32x32x16_tflops": round(t32, 1),
           "mfma_16x16x32_tflops": round(t16, 1), "mfma_32x32x16_lds_fed_tflops": round(t32l, 1),
           "mfma_32x32x16_zero_operands_tflops": round(z32, 1),
           "mfma_probe": "%d workgroups x 4 waves (one per SIMD), each a 128x128 block of accumulators in registers "
                         "fed random bf16 operands (lds_fed: the operands read back from LDS at every step, 512 B "
                         "per instruction as in the GEMM), back-to-back launches for 1.5 s, the last 0.75 s timed"
                         % wg}
    del zeros, ops
    # L2 -> LDS: every wave streams a 2 MiB buffer (L2-resident) into LDS
    span, dwg, dit = 2 << 20, 2 * cus, 100
    dsrc = torch.ones((span // 4,), dtype=torch.float32, device="cuda")
    dout = torch.empty((dwg * 256,), dtype=torch.int32, device="cuda")
    nb_dma = [0.0]
    ms = timed(lambda: nb_dma.__setitem__(0, P.plora_probe_lds_dma(dsrc, dwg, dit, dout)))
    res["lds_dma_l2_GBps"] = round(nb_dma[0] / (ms * 1e-3) / 1e9, 1)
    res["lds_dma_probe"] = ("%d workgroups x 4 waves, each streaming a 2 MiB buffer %d times into LDS with 16-byte "
                            "buffer loads that write LDS, 6 in flight per wave" % (dwg, dit))
    del dsrc, dout
    nbytes = 2 << 30
    src = torch.ones((nbytes // 4,), dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms = timed(lambda: P.plora_probe_copy(src, dst, 8 * cus))
    res["hbm_copy_GBps"] = round(2.0 * nbytes / (ms * 1e-3) / 1e9, 1)
    red = torch.empty((8 * cus * 256,), dtype=torch.int32, device="cuda")
    ms = timed(lambda: P.plora_probe_read(src, red, 8 * cus))
    res["hbm_read_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    res["hbm_probe"] = "2 GiB, %d workgroups of 256 threads, 16-byte accesses" % (8 * cus)
    del src, dst, red, out
    torch.cuda.empty_cache()
    return res


def smi_sample():
    """One reading of the GPU's power and clocks from amd-smi (JSON), reduced
    to the fields whose names mention power or a clock; None if unavailable."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "--power", "--clock", "--json"], stdout=subprocess.PIPE,
                           stderr=subprocess.DEVNULL, text=True, timeout=20)
        data = json.loads(r.stdout)
    except Exception:
        return None
    flat = {}

    def walk(x, pre):
        if isinstance(x, dict):
            if "value" in x and not isinstance(x["value"], (dict, list)):
                flat[pre] = x["value"]
                return
            for k, v in x.items():
                walk(v, pre + "." + str(k) if pre else str(k))
        elif isinstance(x, list):
            if x and not isinstance(x[0], (dict, list)):
                return
            for k, v in enumerate(x[:1]):
                walk(v, pre)
        else:
            flat[pre] = x
    walk(data, "")
    keep = {k: v for k, v in flat.items() if ("power" in k.lower() or "clk" in k.lower() or "clock" in k.lower())
            and isinstance(v, (int, float)) and ("gfx" in k.lower() or "power" in k.lower() or "mem" in k.lower())}
    return dict(list(keep.items())[:24]) or None


def clock_record(stepper, seconds=3.0):
    """Power and clock readings (amd-smi) taken while the step runs back to
    back for about `seconds`, next to idle readings from before."""
    import threading
    import torch
    # amd-smi's socket power is a running average: let it settle after the
    # work that ran before
    torch.cuda.synchronize()
    time.sleep(3.0)
    idle = smi_sample()
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            v = smi_sample()
            if v:
                samples.append(v)
            stop.wait(0.3)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            stepper.step()
        torch.cuda.synchronize()
        n += 10
    stop.set()
    th.join(timeout=30)
    if not samples:
        return {"available": False, "note": "amd-smi gave no reading"}
    keys = sorted(set().union(*samples))
    load = {k: round(float(np.median([s[k] for s in samples if k in s])), 1) for k in keys}
    return {"available": True, "idle": idle, "under_load_median": load, "samples": len(samples),
            "steps_run": n, "source": "amd-smi metric --power --clock --json"}


def run_adamw(P, wl, d, dev, dA, dB, steps, warmup):
    """Per-adapter AdamW over the packed panels with the step's dA/dB, timed
    apart from the operator step (HIP events per launch).  Algorithmic bytes
    per element: read master, m, v, gradient (16) + write master, m, v (12) +
    the operator copy (2 for bf16, 4 for fp32)."""
    import torch
    f32 = lambda t: t.to(torch.float32).contiguous()
    PA, PB = f32(dev["A"]), f32(dev["B"])
    mA, vA, mB, vB = (torch.zeros_like(t) for t in (PA, PA, PB, PB))
    A, B = torch.empty_like(dev["A"]), torch.empty_like(dev["B"])
    lr = [1e-3 * (1 + (i % 3)) for i in range(wl.n_adapters)]
    for k in range(warmup):
        P.plora_adamw_step(d, P.AdamwConfig(lr, [k + 1] * wl.n_adapters), PA, PB, mA, vA, mB, vB, dA, dB, A, B)
    torch.cuda.synchronize()
    P.plora_profile_reset()
    P.plora_profile_enable(True)
    for k in range(steps):
        P.plora_adamw_step(d, P.AdamwConfig(lr, [warmup + k + 1] * wl.n_adapters), PA, PB, mA, vA, mB, vB, dA, dB,
                           A, B)
    torch.cuda.synchronize()
    P.plora_profile_enable(False)
    n, ms = P.plora_profile_read("adamw")
    P.plora_profile_reset()
    elems = wl.R * (wl.d_in + wl.d_out)
    nbytes = elems * (28 + (2 if wl.dtype == "bf16" else 4))
    per_call = ms / steps
    return {"launches": n, "mean_ms": ms / n if n else 0.0, "ms_per_call": per_call, "bytes_per_call": nbytes,
            "achieved_GBps": nbytes / (per_call * 1e-3) / 1e9 if per_call else 0.0}


def run_loop_bench(wl, steps, warmup, dev=None):
    """The same tokens computed adapter by adapter: one single-adapter call per
    segment for each of forward, backward_dx and backward_dAdB (the sequential
    execution that packing replaces).  Returns seconds per step."""
    import torch
    import packed_adapter_lora_amd as P
    if dev is None:
        _, dev = make_device_inputs(wl)
    dt = dev["X"].dtype
    Y = torch.empty((wl.T, wl.d_out), dtype=dt, device="cuda")
    dX = torch.empty((wl.T, wl.d_in), dtype=dt, device="cuda")
    he = int(np.sum(np.diff(wl.offsets) * wl.ranks))
    H = torch.empty((he,), dtype=torch.float32, device="cuda")
    G = torch.empty((he,), dtype=torch.float32, device="cuda")
    dA = torch.empty((wl.R, wl.d_in), dtype=torch.float32, device="cuda")
    dB = torch.empty((wl.R, wl.d_out), dtype=torch.float32, device="cuda")
    calls = []
    ro = ho = 0
    for i in range(wl.n_adapters):
        a, b = int(wl.offsets[i]), int(wl.offsets[i + 1])
        r = int(wl.ranks[i])
        d = P.Desc([0, b - a], [r], [float(wl.alphas[i])], wl.d_in, wl.d_out, wl.dtype)
        nb = P.plora_workspace_bytes(d)
        ws = torch.empty((max(nb, 16),), dtype=torch.uint8, device="cuda")
        calls.append((d, slice(a, b), slice(ro, ro + r), slice(ho, ho + (b - a) * r), ws))
        ro += r
        ho += (b - a) * r
    stream = torch.cuda.current_stream()

    def step():
        for d, rows, rr, hs, ws in calls:
            P.plora_forward(d, dev["X"][rows], dev["W"], dev["A"][rr], dev["B"][rr], Y[rows], H[hs], stream)
            P.plora_backward_dx(d, dev["dY"][rows], dev["W"], dev["A"][rr], dev["B"][rr], dX[rows], G[hs], stream)
            P.plora_backward_dAdB(d, dev["X"][rows], dev["dY"][rows], H[hs], G[hs], dA[rr], dB[rr], ws, stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del Y, dX, H, G, dA, dB, dev
    return (t1 - t0) / steps


def cpu_baseline(wl, inp, per_segment):
    """fp64 oracle on the first `per_segment` tokens of every segment: Y, H, dX,
    G and dA/dB over those tokens, as the oracle stands."""
    import oracle
    rows = []
    for i in range(wl.n_adapters):
        a, b = int(wl.offsets[i]), int(wl.offsets[i + 1])
        rows.extend(range(a, min(b, a + per_segment)))
    rows = np.array(rows, dtype=np.int64)
    seg = np.searchsorted(wl.offsets, rows, side="right") - 1
    counts = np.bincount(seg, minlength=wl.n_adapters)
    sub_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    X, dY = inp["X"][rows].astype(np.float64), inp["dY"][rows].astype(np.float64)
    W, A, B = (inp[k].astype(np.float64) for k in ("W", "A", "B"))
    t0 = time.perf_counter()
    oracle.packed_lora(sub_off, wl.ranks, wl.alphas.astype(np.float64), wl.d_in, wl.d_out, X=X, dY=dY, W=W, A=A,
                       B=B, want=("Y", "H", "dX", "G", "dA", "dB"))
    dt = time.perf_counter() - t0
    threads = oracle.threads()
    # one core: the first 4 tokens of every segment
    rows1 = np.concatenate([np.arange(int(wl.offsets[i]), min(int(wl.offsets[i + 1]), int(wl.offsets[i]) + 4))
                            for i in range(wl.n_adapters)])
    seg1 = np.searchsorted(wl.offsets, rows1, side="right") - 1
    off1 = np.concatenate([[0], np.cumsum(np.bincount(seg1, minlength=wl.n_adapters))]).astype(np.int64)
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.packed_lora(off1, wl.ranks, wl.alphas.astype(np.float64), wl.d_in, wl.d_out,
                           X=inp["X"][rows1].astype(np.float64), dY=inp["dY"][rows1].astype(np.float64), W=W, A=A,
                           B=B, want=("Y", "H", "dX", "G", "dA", "dB"))
        dt1 = time.perf_counter() - t0
    finally:
        oracle.set_threads(threads)
    model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "first %d tokens of each of the %d segments (%d tokens), full d_in x d_out, all of Y, H, dX, "
                      "G, dA, dB over them; %.1f s on %d threads" % (per_segment, wl.n_adapters, len(rows), dt,
                                                                     threads),
            "nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model,
            "single_core": {"value": len(rows1) / dt1, "unit": "tokens/s", "threads": 1,
                            "sample": "first 4 tokens of each segment (%d tokens); %.1f s" % (len(rows1), dt1)}}


BLOCK_DIMS = {"hidden": 4096, "n_q": 32, "n_kv": 8, "mlp": 14336}


def block_setup(n_adapters, tokens_each, seed=5):
    """The Llama-3-8B decoder-block workload: N adapters x tokens_each tokens
    (one sequence per adapter), ranks cycling 8/16/32/64, alphas 8/16/32, LoRA
    on all seven projections; seeded synthetic weights and activations."""
    import workloads
    ranks = [[8, 16, 32, 64][i % 4] for i in range(n_adapters)]
    alphas = [[8.0, 16.0, 32.0][i % 3] for i in range(n_adapters)]
    seg = np.arange(n_adapters + 1, dtype=np.int64) * tokens_each
    from packed_adapter_lora_amd.block import proj_dims
    dims = proj_dims(**BLOCK_DIMS)
    R = sum(ranks)
    hp = {"w1": 1.0 + workloads.draw(seed, 101, (1, BLOCK_DIMS["hidden"]), 0.1, "bf16")[0],
          "w2": 1.0 + workloads.draw(seed, 102, (1, BLOCK_DIMS["hidden"]), 0.1, "bf16")[0], "W": {}, "A": {}, "B": {},
          "ranks": np.array(ranks), "alphas": np.array(alphas), "dims": dims, "n_q": BLOCK_DIMS["n_q"],
          "n_kv": BLOCK_DIMS["n_kv"]}
    for w in ("w1", "w2"):
        hp[w] = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(hp[w]))
    for i, (n, (di, do)) in enumerate(sorted(dims.items())):
        hp["W"][n] = workloads.draw(seed, 110 + i, (do, di), 1.0 / np.sqrt(di), "bf16")
        hp["A"][n] = workloads.draw(seed, 120 + i, (R, di), 0.1, "bf16")
        hp["B"][n] = workloads.draw(seed, 130 + i, (R, do), float(np.sqrt(0.02)), "bf16")
    T = int(seg[-1])
    x = workloads.draw(seed, 140, (T, BLOCK_DIMS["hidden"]), 1.0, "bf16")
    dout = workloads.draw(seed, 141, (T, BLOCK_DIMS["hidden"]), 1.0, "bf16")
    return hp, seg, ranks, alphas, x, dout


def decode_bytes(wl):
    """Algorithmic HBM bytes of one decode-shaped forward: W, the packed A and
    B panels, X, Y and H written and read once (bf16 operands, fp32 H)."""
    nr = float(np.sum(np.diff(wl.offsets) * wl.ranks))
    return 2.0 * (wl.d_in * wl.d_out + wl.R * (wl.d_in + wl.d_out) + wl.T * (wl.d_in + wl.d_out)) + 8.0 * nr


def run_decode_bench(args):
    """Forward-only multi-LoRA at serving shapes (1 to 16 tokens per adapter):
    latency of plora_forward, bound by HBM (the frozen W and the adapters'
    panels are each read once)."""
    import torch
    import packed_adapter_lora_amd as P
    import workloads
    name = args.workload if args.workload.startswith("decode") else "decode_up"
    wl = workloads.config(name, n_adapters=args.adapters)
    log("decode workload %s: T=%d d_in=%d d_out=%d N=%d R=%d" % (wl.name, wl.T, wl.d_in, wl.d_out, wl.n_adapters,
                                                                  wl.R))
    inp = workloads.make_inputs(wl, which=("W", "A", "B", "X"))
    dev = {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in inp.items()}
    d = P.Desc.from_workload(wl)
    Y = torch.empty((wl.T, wl.d_out), dtype=torch.bfloat16, device="cuda")
    H = torch.empty((P.plora_h_elems(d),), dtype=torch.float32, device="cuda")
    calls = max(args.steps, 20) * 5
    for _ in range(args.warmup * 5):
        P.plora_forward(d, dev["X"], dev["W"], dev["A"], dev["B"], Y, H)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        P.plora_forward(d, dev["X"], dev["W"], dev["A"], dev["B"], Y, H)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    nbytes = decode_bytes(wl)
    out = {"metric": "decode-shaped packed LoRA forward latency (%d adapters, %d tokens)" % (wl.n_adapters, wl.T),
           "value": round(us, 2), "unit": "us", "n_gpus": 1, "steps": calls, "warmup": args.warmup * 5,
           "higher_is_better": False, "dtype": "bf16", "data": "synthetic (seeded normal draws)",
           "config": {"workload": wl.name, "d_in": wl.d_in, "d_out": wl.d_out, "n_adapters": wl.n_adapters,
                      "tokens": wl.T, "tokens_per_adapter": sorted(set(np.diff(wl.offsets).tolist())),
                      "sum_ranks": wl.R},
           "tokens_per_s": round(wl.T / (us * 1e-6), 1),
           "roofline": {"bound": "hbm", "achieved": round(nbytes / (us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                        "bytes_per_call": nbytes}}
    print(json.dumps(out), flush=True)


def block_flops(seg, ranks, hp):
    """Algorithmic FLOPs of one block step: per projection 4 T d_in d_out + 6 sum n_i r_i (d_in + d_out);
    attention 2 (forward) + 5 (backward) products of 2 * 128 * n_q * sum_s n_s (n_s + 1) / 2."""
    counts = np.diff(seg)
    nr = float(np.sum(counts * np.asarray(ranks)))
    T = float(seg[-1])
    f = sum(4.0 * T * di * do + 6.0 * nr * (di + do) for di, do in hp["dims"].values())
    pairs = float(np.sum(counts * (counts + 1) / 2.0))
    return f + 7 * 2.0 * 128 * hp["n_q"] * pairs


def run_block_bench(args):
    import torch
    import packed_adapter_lora_amd as P
    from packed_adapter_lora_amd.block import DecoderBlock
    n, te = args.adapters or 32, 1024
    log("decoder block: %d adapters x %d tokens, Llama-3-8B dims %s" % (n, te, BLOCK_DIMS))
    hp, seg, ranks, alphas, x, dout = block_setup(n, te)
    tb = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(torch.bfloat16)
    dp = {"w1": tb(hp["w1"]), "w2": tb(hp["w2"]), "W": {k: tb(v) for k, v in hp["W"].items()},
          "A": {k: tb(v) for k, v in hp["A"].items()}, "B": {k: tb(v) for k, v in hp["B"].items()}}
    blk = DecoderBlock(dp, seg, ranks, alphas, seg, **BLOCK_DIMS)
    xd, dd = tb(x), tb(dout)
    # per-adapter AdamW on every projection's packed A/B: fp32 masters and
    # moments; the step writes the bf16 operator copies the next forward uses
    from packed_adapter_lora_amd.block import PROJ
    opt = {}
    for pn in PROJ:
        PA, PB = dp["A"][pn].float().contiguous(), dp["B"][pn].float().contiguous()
        opt[pn] = (PA, PB, torch.zeros_like(PA), torch.zeros_like(PA), torch.zeros_like(PB), torch.zeros_like(PB))
    lr = [1e-4 * (1 + (i % 3)) for i in range(n)]
    count = [0]

    def step():
        blk.forward(xd)
        _, grads = blk.backward(dd)
        count[0] += 1
        cfg = P.AdamwConfig(lr, [count[0]] * n)
        for pn in PROJ:
            P.plora_adamw_step(blk.desc[pn], cfg, *opt[pn], *grads[pn], dp["A"][pn], dp["B"][pn])

    class _Step:
        pass
    stepper = _Step()
    stepper.step = step
    # the timed region: no per-kernel events (they cost the GPU a few
    # microseconds at every library call, and the block makes ~90 calls)
    sec, per = timed_steps(stepper, args.steps, args.warmup)
    log("per-kernel times: the same steps again with the library's per-launch events")
    P.plora_profile_reset()
    P.plora_profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    sec_prof = (time.perf_counter() - t0) / args.steps
    P.plora_profile_enable(False)
    kern = {}
    for cls in ("gemm_fwd", "gemm_bwd", "shrink", "wgrad", "reduce", "norm", "rope", "swiglu", "add", "attn_fwd",
                "attn_bwd", "adamw"):
        cnt, ms = P.plora_profile_read(cls)
        if cnt:
            kern[cls] = round(ms / args.steps, 4)
    P.plora_profile_reset()
    T = int(seg[-1])
    flops = block_flops(seg, ranks, hp)
    achieved = flops / sec / 1e12
    out = {"metric": "decoder block fwd+bwd+AdamW tokens/sec (LoRA on 7 projections, %d adapters)" % n,
           "value": round(T / sec, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(sec * 1e3, 3), "higher_is_better": True, "dtype": "bf16",
           "data": "synthetic (seeded normal draws; no dataset or checkpoint)",
           "config": {"workload": "llama3_8b_decoder_block_%d_adapters_x_%d_tokens" % (n, te), **BLOCK_DIMS,
                      "tokens": T, "ranks": sorted(set(ranks)), "sequence": te},
           "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "kernel": "whole block step",
                        "flops_per_step": flops},
           "kernels_ms_per_step": kern, "step_ms": {"timed_region_mean": round(sec * 1e3, 4),
                                                    "per_step_events": summary_ms(per),
                                                    "with_per_kernel_events": round(sec_prof * 1e3, 4)},
           "cpu_baseline": None}
    if not args.no_cpu:
        log("timing the oracle block on the host ...")
        out["cpu_baseline"] = block_cpu_baseline(hp, seg, ranks, alphas, x, dout, args.cpu_tokens)
    print(json.dumps(out), flush=True)


def time_block_step(n_adapters, tokens_each, steps=3, warmup=1):
    """Seconds per forward+backward step of one decoder block."""
    import torch
    from packed_adapter_lora_amd.block import DecoderBlock
    hp, seg, ranks, alphas, x, dout = block_setup(n_adapters, tokens_each)
    tb = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(torch.bfloat16)
    dp = {"w1": tb(hp["w1"]), "w2": tb(hp["w2"]), "W": {k: tb(v) for k, v in hp["W"].items()},
          "A": {k: tb(v) for k, v in hp["A"].items()}, "B": {k: tb(v) for k, v in hp["B"].items()}}
    blk = DecoderBlock(dp, seg, ranks, alphas, seg, **BLOCK_DIMS)
    xd, dd = tb(x), tb(dout)
    for _ in range(warmup):
        blk.forward(xd)
        blk.backward(dd)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        blk.forward(xd)
        blk.backward(dd)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def plan_jobs(n_jobs=120, layers=32, dataset=2000, epochs=3, seq=1024):
    """The fine-tuning jobs of a hyper-parameter search like the pages' 120
    configurations (rank, batch size, learning rate, scale varied): ranks
    8..64, batch sizes 1..8 sequences of 1024 tokens, `epochs` passes over
    `dataset` sequences.  Memory per job on Llama-3-8B (32 layers, LoRA on the
    7 projections): 18 bytes per adapter parameter (fp32 master, two fp32
    moments, fp32 gradient, bf16 copy) and the activations the backward keeps
    (136 KiB per token per layer in bf16: x, h1, q, k, v, attention output, x2,
    h2, gate, up, SwiGLU output)."""
    from packed_adapter_lora_amd.block import proj_dims
    dims = proj_dims(**BLOCK_DIMS)
    per_rank = layers * sum(di + do for di, do in dims.values())
    act_per_token = layers * 2.0 * (6 * 4096 + 2 * 1024 + 3 * 14336)
    jobs = []
    for k in range(n_jobs):
        r = [8, 16, 32, 64][k % 4]
        bs = [1, 2, 4, 8][(k // 4) % 4]
        tokens = bs * seq
        steps = epochs * dataset // bs
        jobs.append({"rank": r, "tokens": tokens, "steps": steps, "mem": 18.0 * r * per_rank + act_per_token * tokens})
    return jobs


def run_plan_bench(args):
    """Plan a 120-job LoRA search on one GPU with the cost model fitted on the
    decoder block (two sizes), and compare the planned makespan with running
    the jobs one at a time."""
    import packed_adapter_lora_amd as P
    layers = 32
    log("fitting the step-time model on the decoder block (1024 and 32768 tokens) ...")
    t_small = time_block_step(1, 1024)
    t_big = time_block_step(32, 1024)
    per_token = (t_big - t_small) / (32768 - 1024)   # seconds per token per layer
    fixed = max(t_small - per_token * 1024, 0.0)      # seconds per step per layer
    jobs = plan_jobs(layers=layers)
    budget = 288e9 - 16.1e9 - 8e9   # HBM minus the bf16 base model and working buffers
    steps = [j["steps"] for j in jobs]
    mem = [j["mem"] for j in jobs]
    own = [j["tokens"] * per_token * layers * 1e3 for j in jobs]  # ms per step
    fixed_ms = fixed * layers * 1e3
    t0 = time.perf_counter()
    assign, npk, makespan = P.plora_plan_packs(steps, mem, own, budget, fixed_ms, 2 ** 26)
    plan_ms = (time.perf_counter() - t0) * 1e3
    seq_ms = sum(s * (fixed_ms + o) for s, o in zip(steps, own))
    lower = fixed_ms * max(steps) + sum(s * o for s, o in zip(steps, own))
    out = {"metric": "planned packing speedup over one job at a time (120 LoRA fine-tuning jobs, one MI355X)",
           "value": round(seq_ms / makespan, 3), "unit": "x", "higher_is_better": True, "n_gpus": 1,
           "data": "synthetic job set; cost model measured on the decoder block",
           "config": {"workload": "llama3_8b_lora_search_120_jobs", "layers": layers, "ranks": [8, 16, 32, 64],
                      "batch_sequences": [1, 2, 4, 8], "sequence": 1024, "memory_budget_GB": round(budget / 1e9, 1)},
           "plan": {"packs": npk, "makespan_h": round(makespan / 3.6e6, 3),
                    "one_at_a_time_h": round(seq_ms / 3.6e6, 3), "lower_bound_h": round(lower / 3.6e6, 3),
                    "planner_ms": round(plan_ms, 2)},
           "cost_model": {"fixed_ms_per_step_per_layer": round(fixed * 1e3, 4),
                          "us_per_token_per_layer": round(per_token * 1e6, 5),
                          "measured": "decoder block fwd+bwd at 1 x 1024 and 32 x 1024 tokens"}}
    print(json.dumps(out), flush=True)


def block_cpu_baseline(hp, seg, ranks, alphas, x, dout, per_segment):
    """fp64 oracle block (forward + backward) on the first `per_segment` tokens
    of the first two adapters' sequences (a bounded sample)."""
    import oracle
    from oracle import block as OB
    rows = np.concatenate([np.arange(seg[i], seg[i] + per_segment) for i in range(2)])
    sub = np.array([0, per_segment, 2 * per_segment] + [2 * per_segment] * (len(ranks) - 2), dtype=np.int64)
    p = dict(hp)
    t0 = time.perf_counter()
    out, c = OB.block_forward(p, x[rows], sub, np.array([0, per_segment, 2 * per_segment], np.int64))
    OB.block_backward(p, c, dout[rows], sub, np.array([0, per_segment, 2 * per_segment], np.int64))
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "first %d tokens of the first 2 adapters' sequences (%d tokens), full Llama-3-8B block dims, "
                      "forward and backward with all 7 projections' dA/dB (the AdamW step, a fixed cost per step "
                      "whatever the tokens, is not in the host sample); %.1f s" % (per_segment, len(rows), dt)}


def write_stats_profile(d, title, name):
    """Kernel-time summary of a rocprofv3 --kernel-trace --stats run (trace/ under d)
    into profiles/<name>."""
    import csv
    import glob
    cmds = json.load(open(os.path.join(d, "commands.json")))
    f = glob.glob(os.path.join(d, "trace", "**", "*kernel_stats.csv"), recursive=True)
    rows = list(csv.DictReader(open(f[0])))
    lines = ["# rocprofv3 kernel statistics, " + title,
             "# command: " + cmds["trace"], "",
             "%6s %12s %12s %7s  %s" % ("calls", "total_ms", "avg_us", "pct", "kernel")]
    for r in rows:
        lines.append("%6s %12.3f %12.1f %7.2f  %s" % (r["Calls"], float(r["TotalDurationNs"]) / 1e6,
                                                      float(r["AverageNs"]) / 1e3, float(r["Percentage"]),
                                                      r["Name"][:110]))
    txt = "\n".join(lines) + "\n"
    open(os.path.join(ROOT, "profiles", name), "w").write(txt)
    print(txt)


BLOCK_COUNTER_CLASSES = (("attn_fwd_kernel", "attn_fwd"), ("attn_bwd_dq_kernel", "attn_bwd_dq"),
                         ("attn_bwd_dkv_kernel", "attn_bwd_dkv"), ("gemm_lora_bf16_pipe<true", "gemm_fwd"),
                         ("gemm_lora_bf16_pipe<false, 4, true>", "gemm_bwd_swiglu"),
                         ("gemm_lora_bf16_pipe<false, 2, true>", "gemm_bwd_swiglu"),
                         ("gemm_lora_bf16_pipe<false", "gemm_bwd"), ("shrink_bf16_pipe", "shrink"),
                         ("wgrad_bf16_pipe", "wgrad"), ("wgrad_prep", "wgrad_prep"), ("rmsnorm", "rmsnorm"),
                         ("swiglu", "swiglu"), ("rope_kernel", "rope"), ("add_kernel", "add"), ("adamw", "adamw"))


def write_block_counters(d):
    """Per-kernel-class counter summary of the decoder block from two rocprofv3
    --pmc runs (p1/, p2/ under d; their commands in d/commands.json) into
    profiles/kernels_llama3_8b_block_counters.txt."""
    import csv
    import glob
    cmds = json.load(open(os.path.join(d, "commands.json")))
    sums = {}
    for run in ("p1", "p2"):
        f = glob.glob(os.path.join(d, run, "**", "*counter_collection.csv"), recursive=True)[0]
        for r in csv.DictReader(open(f)):
            cls = next((c for key, c in BLOCK_COUNTER_CLASSES if key in r["Kernel_Name"]), None)
            if cls is None:
                continue
            sums.setdefault(cls, {}).setdefault(r["Counter_Name"], 0.0)
            sums[cls][r["Counter_Name"]] += float(r["Counter_Value"])
    ratio = lambda a, b: a / b if b else float("nan")
    lines = ["# matrix-core, vector-ALU and LDS counters per kernel class, Llama-3-8B decoder block "
             "(32 adapters x 1024 tokens)",
             "# pass 1: " + cmds["p1"], "# pass 2: " + cmds["p2"],
             "# mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES); valu_active = "
             "SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES;",
             "# lds_wait = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES; conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; "
             "valu/mfma = SQ_INSTS_VALU / SQ_INSTS_MFMA (instructions, summed over the run's dispatches)", "",
             "%-16s %10s %11s %9s %10s %9s" % ("class", "mfma_util", "valu_active", "lds_wait", "conflict", "valu/mfma")]
    order = [c for _, c in BLOCK_COUNTER_CLASSES]
    for cls in sorted(sums, key=lambda c: order.index(c)):
        v = sums[cls]
        lines.append("%-16s %10.3f %11.3f %9.3f %10.4f %9.2f" % (
            cls, ratio(v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0), 4 * v.get("SQ_BUSY_CU_CYCLES", 0)),
            ratio(v.get("SQ_ACTIVE_INST_VALU", 0), v.get("SQ_WAVE_CYCLES", 0)),
            ratio(v.get("SQ_WAIT_INST_LDS", 0), v.get("SQ_WAVE_CYCLES", 0)),
            ratio(v.get("SQ_LDS_BANK_CONFLICT", 0), v.get("SQ_LDS_IDX_ACTIVE", 0)),
            ratio(v.get("SQ_INSTS_VALU", 0), v.get("SQ_INSTS_MFMA", 0))))
    txt = "\n".join(lines) + "\n"
    open(os.path.join(ROOT, "profiles", "kernels_llama3_8b_block_counters.txt"), "w").write(txt)
    print(txt)


def write_profiles(d, workload):
    import workloads
    wl = workloads.config(workload)
    cmds = json.load(open(os.path.join(d, "commands.json")))
    res = rocprof_summary(os.path.join(d, "trace"), os.path.join(d, "fetch"), os.path.join(d, "write"),
                          os.path.join(d, "copy_fetch"), os.path.join(d, "copy_write"), cmds["copy_bytes"],
                          wl.name, cmds, os.path.join(d, "mfma"))
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    open(os.path.join(prof, "kernels_%s_stats.txt" % wl.name), "w").write(res["stats"])
    open(os.path.join(prof, "kernels_%s_hbm_traffic.txt" % wl.name), "w").write(res["traffic_txt"])
    if "mfma_txt" in res:
        open(os.path.join(prof, "kernels_%s_mfma_clock.txt" % wl.name), "w").write(res["mfma_txt"])
        print(res["mfma_txt"])
    if "lds_l2_txt" in res:
        open(os.path.join(prof, "kernels_%s_lds_l2.txt" % wl.name), "w").write(res["lds_l2_txt"])
        print(res["lds_l2_txt"])
    src = {"gemm_fwd": "gemm_bf16.hip", "gemm_bwd": "gemm_bf16.hip", "shrink": "lora_bf16.hip",
           "shrink_sum": "lora_bf16.hip", "wgrad": "lora_bf16.hip", "wgrad_prep": "lora_bf16.hip",
           "reduce": "lora_bf16.hip", "adamw": "optim.hip"}
    tj = {}
    for cls, rec in res["traffic"].items():
        f = os.path.join(ROOT, "packed_adapter_lora_amd", "csrc", src[cls])
        tj[cls] = {"workload": wl.name, "tokens": wl.T, "source": src[cls], "source_sha": source_sha(f),
                   "bytes_per_launch": round(rec["bytes_per_launch"]), "fetch_bytes": round(rec["fetch_bytes"]),
                   "write_bytes": round(rec["write_bytes"]), "fetch_scale": res["scales"][0],
                   "write_scale": res["scales"][1]}
    json.dump(tj, open(os.path.join(prof, "traffic.json"), "w"), indent=1, sort_keys=True)
    print(res["stats"])
    print(res["traffic_txt"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama_up")
    ap.add_argument("--adapters", type=int, default=None)
    ap.add_argument("--cpu-tokens", type=int, default=64, help="oracle sample: tokens per segment")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the MFMA / HBM ceiling probes")
    ap.add_argument("--no-clock", action="store_true", help="skip the power and clock record")
    ap.add_argument("--no-sweep", action="store_true", help="skip the adapter sweep of the default run")
    ap.add_argument("--region-only", action="store_true",
                    help="run only the warm-up and timed steps (for profiler runs: no other passes, sweep or oracle)")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--plan", action="store_true",
                    help="plan a 120-job LoRA search with the packing planner (cost model fitted on the GPU)")
    ap.add_argument("--decode", action="store_true",
                    help="time the forward at decode shapes (--workload decode_up or decode_sq)")
    ap.add_argument("--block", action="store_true",
                    help="time the Llama-3-8B decoder block (LoRA on all 7 projections) instead of the operator")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--rocprof-summary", default=None,
                    help="directory holding rocprofv3 csv runs trace/, fetch/, write/, copy_fetch/, copy_write/: "
                         "write summaries under profiles/ and exit")
    args = ap.parse_args()
    if args.rocprof_summary:
        if args.block and os.path.isdir(os.path.join(args.rocprof_summary, "p1")):
            write_block_counters(args.rocprof_summary)
        elif args.block:
            write_stats_profile(args.rocprof_summary, "Llama-3-8B decoder block, 32 adapters x 1024 tokens",
                                "kernels_llama3_8b_block_stats.txt")
        elif args.decode:
            import workloads
            wl = workloads.config(args.workload)
            write_stats_profile(args.rocprof_summary, "decode-shaped forward %s (%d adapters, %d tokens, "
                                "%d -> %d)" % (wl.name, wl.n_adapters, wl.T, wl.d_in, wl.d_out),
                                "kernels_%s_stats.txt" % wl.name)
        else:
            write_profiles(args.rocprof_summary, args.workload)
        return
    if args.plan:
        if args.gpus != 1:
            print("bench.py measures one GPU only (--gpus %d requested)" % args.gpus, file=sys.stderr)
            sys.exit(2)
        run_plan_bench(args)
        return
    if args.decode:
        if args.gpus != 1:
            print("bench.py measures one GPU only (--gpus %d requested)" % args.gpus, file=sys.stderr)
            sys.exit(2)
        run_decode_bench(args)
        return
    if args.block:
        if args.gpus != 1:
            print("bench.py measures one GPU only (--gpus %d requested)" % args.gpus, file=sys.stderr)
            sys.exit(2)
        run_block_bench(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the packed-LoRA operator here has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        n = args.copy_probe // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4}), flush=True)
        return

    wl = workloads.config(args.workload, n_adapters=args.adapters)
    log("workload %s: T=%d d_in=%d d_out=%d N=%d R=%d" % (wl.name, wl.T, wl.d_in, wl.d_out, wl.n_adapters, wl.R))
    import packed_adapter_lora_amd as P
    log("step 1: timed region (%d steps after %d warm-up, per-kernel events on)" % (args.steps, args.warmup))
    sec, kern, inp, stp = run_bench(wl, args.steps, args.warmup)
    dev = stp.dev
    tokens_per_s = wl.T / sec
    dom = max(("gemm_fwd", "gemm_bwd"), key=lambda k: kern[k]["mean_ms"])
    flops = gemm_flops(wl, dom)
    achieved = flops / (kern[dom]["mean_ms"] * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": load_traffic(dom, wl), "kernel": dom,
            "flops_per_launch": flops, "mean_launch_ms": round(kern[dom]["mean_ms"], 4)}
    whole = step_flops(wl) / sec / 1e12
    if args.region_only:
        args.no_ceilings = args.no_clock = args.no_sweep = args.no_cpu = True
    step_ms = {"timed_region_mean": round(sec * 1e3, 4)}
    overhead, opt = None, None
    if not args.region_only:
        step_ms, overhead, opt = extra_passes(P, wl, stp, dev, args, sec)
    ceil = None
    if not args.no_ceilings:
        log("step 6: measured ceilings (sustained MFMA, HBM copy/read)")
        ceil = measure_ceilings()
        roof["peak_measured"] = ceil["mfma_bf16_tflops"]
        roof["frac_of_measured"] = round(achieved / ceil["mfma_bf16_tflops"], 4)
    clock = None
    if not args.no_clock:
        log("step 7: power and clock while the step runs")
        clock = clock_record(stp)
    sweep = None
    if not args.no_sweep and wl.name == "llama_up" and wl.n_adapters == 32:
        log("step 8: adapter sweep (2..32 adapters x 2048 tokens, 4096->14336 and 4096->4096)")
        sweep = adapter_sweep(wl, dev, max(5, args.steps // 2))
    del stp
    torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu:
        log("step 9: timing the oracle on the host ...")
        cpu = cpu_baseline(wl, inp, args.cpu_tokens)
    out = {
        "metric": "packed LoRA fwd+bwd tokens/sec at %d adapters" % wl.n_adapters,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded normal draws; no dataset or checkpoint)",
        "config": {"workload": workload_label(wl),
            "d_in": wl.d_in, "d_out": wl.d_out, "n_adapters": wl.n_adapters, "tokens": wl.T,
            "ranks": sorted(set(wl.ranks.tolist())), "sum_ranks": wl.R},
        "roofline": roof,
        "cpu_baseline": cpu,
        "step_ms": step_ms,
        "lora_overhead": overhead,
        "whole_step_tflops": round(whole, 1),
        "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in kern.items()},
        "ceilings": ceil,
        "clock": clock,
        "adapter_sweep": sweep,
    }
    if opt:
        # the per-adapter AdamW step over the packed panels, timed after (not in) the step above
        out["optimizer"] = {"kernel": "adamw", "bound": "hbm", "ms_per_call": round(opt["ms_per_call"], 4),
                            "bytes_per_call": opt["bytes_per_call"], "achieved": round(opt["achieved_GBps"], 1),
                            "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(opt["achieved_GBps"] / PEAK_HBM_GBS, 4)}
    print(json.dumps(out), flush=True)

    if args.sweep:
        for n in (2, 4, 8, 16, 32):
            w2 = workloads.config(args.workload, n_adapters=n)
            s2, k2, _, st2 = run_bench(w2, args.steps, args.warmup)
            del st2
            s3 = run_loop_bench(w2, max(3, args.steps // 4), 2)
            torch.cuda.empty_cache()
            print(json.dumps({"sweep": True, "workload": w2.name, "n_adapters": n, "tokens": w2.T,
                              "tokens_per_s": round(w2.T / s2, 1), "ms_per_step": round(s2 * 1e3, 4),
                              "adapter_by_adapter_tokens_per_s": round(w2.T / s3, 1),
                              "packing_gain": round(s3 / s2, 3),
                              "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in k2.items()}}),
                  flush=True)


def extra_passes(P, wl, stp, dev, args, sec):
    """The passes after the timed region: per-step event timings without the
    library's per-kernel events, the same with the caches flushed, the
    frozen path alone (LoRA overhead) and the per-adapter AdamW step."""
    import torch
    log("step 2: the same step without per-kernel events (per-step event timings)")
    _, per = timed_steps(stp, args.steps, 2)
    step_ms = {"timed_region_mean": round(sec * 1e3, 4), "unprofiled": summary_ms(per)}
    log("step 3: with L2 and the Infinity Cache flushed before every step")
    flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device="cuda")
    _, perf = timed_steps(stp, args.steps, 2, flush=flush)
    del flush
    step_ms["cache_flushed"] = summary_ms(perf)
    log("step 4: frozen path only (no adapters) on the same tokens")
    d0 = P.Desc([0], [], [], wl.d_in, wl.d_out, wl.dtype, n_tokens=wl.T)
    s0 = Stepper(P, d0, {k: dev[k] for k in ("X", "W", "dY")}, wl.T, wl.d_in, wl.d_out, 0)
    _, per0 = timed_steps(s0, args.steps, 2)
    del s0
    frozen = summary_ms(per0)
    overhead = {"frozen_ms_per_step": frozen["median"],
                "lora_overhead_ms": round(step_ms["unprofiled"]["median"] - frozen["median"], 4),
                "lora_overhead_frac": round((step_ms["unprofiled"]["median"] - frozen["median"]) /
                                            step_ms["unprofiled"]["median"], 4)}
    opt = None
    if wl.n_adapters:
        log("step 5: per-adapter AdamW on the step's gradients")
        opt = run_adamw(P, wl, stp.d, dev, stp.dA, stp.dB, args.steps, args.warmup)
    return step_ms, overhead, opt


def slice_inputs(dev, wl_n):
    """Device inputs of the first N adapters of a workload whose per-adapter
    draws and 2048-row chunks do not depend on N: the first T_N token rows and
    the first R_N rank rows are exactly the N-adapter workload's inputs."""
    return {"W": dev["W"], "A": dev["A"][:wl_n.R], "B": dev["B"][:wl_n.R], "X": dev["X"][:wl_n.T],
            "dY": dev["dY"][:wl_n.T]}


def adapter_sweep(wl, dev, steps):
    """Tokens/s of the packed step at N = 2..32 adapters of 2048 tokens on the
    4096->14336 and 4096->4096 shapes, against the same tokens computed
    adapter by adapter (median of per-step events; the loop by wall clock)."""
    import torch
    import packed_adapter_lora_amd as P
    import workloads
    res = {}
    shapes = [("llama_up", dev)]
    sq = workloads.config("llama_sq", n_adapters=32)
    inp_sq = workloads.make_inputs(sq, which=("W", "B", "dY"))
    dt = dev["X"].dtype
    dev_sq = {"W": torch.from_numpy(inp_sq["W"]).to("cuda").to(dt), "A": dev["A"],  # A and X: the same draws
              "B": torch.from_numpy(inp_sq["B"]).to("cuda").to(dt), "X": dev["X"],
              "dY": torch.from_numpy(inp_sq["dY"]).to("cuda").to(dt)}
    del inp_sq
    shapes.append(("llama_sq", dev_sq))
    for name, dv in shapes:
        rows = []
        for n in (2, 4, 8, 16, 32):
            w2 = workloads.config(name, n_adapters=n)
            sub = slice_inputs(dv, w2)
            stp = Stepper(P, P.Desc.from_workload(w2), sub, w2.T, w2.d_in, w2.d_out, w2.R)
            _, per = timed_steps(stp, steps, 2)
            del stp
            med = summary_ms(per)["median"]
            loop = run_loop_bench(w2, max(3, steps // 2), 1, dev=sub)
            rows.append({"n_adapters": n, "tokens": w2.T, "ms_per_step": med,
                         "tokens_per_s": round(w2.T / (med * 1e-3), 1),
                         "adapter_by_adapter_tokens_per_s": round(w2.T / loop, 1),
                         "packing_gain": round(loop / (med * 1e-3), 3)})
        ref = rows[-1]["tokens_per_s"]
        for r in rows:
            r["vs_32"] = round(r["tokens_per_s"] / ref, 3)
        res[name] = rows
        torch.cuda.empty_cache()
    del dev_sq
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
