#!/usr/bin/env python3
"""Benchmark of the LiftQuant decode operator on one MI355X.

Headline (`value`): one batch-1 decode step through the linear layers of a
Llama-3-70B block at 2.4 bits per weight (d = 10, D = 24, bf16 activations,
Hadamard block 1024): QKV (K = 8192 -> N = 10240), gate and up (K = 8192 ->
N = 28672, the same input, one lq_linear_multi call) and down (K = 28672 ->
N = 8192); 236.7 MB of packed signs per step. Every step uses the next of
`--weight-sets` distinct copies of the packed weights, so what a step reads
cannot stay in the 256 MB Infinity Cache (as in a real 80-layer model, whose
weights all differ). The K timed steps are captured once in a HIP graph and
replayed; the sign-product kernel durations come from an eager replay of the
same K steps right after, each launch timed by events its own dispatch
records (events cannot be timed inside a graph).

Also in the line:
  roofline      the dominant kernel (the small-batch sign product) of the
                headline step against 8 TB/s;
  prefill       the 2048-token prefill layer K = 8192 -> N = 28672 (d = 3,
                D = 8) through lq_linear, in TFLOP/s;
  large         the same layer through the lifted large-batch product
                (LQ_ALGO_MFMA_LARGE, sign_mfma_large_kernel);
  configs       every other layer and batch size of the workloads: the
                Llama-3-8B MLP step at batch 1, each Llama-3-70B layer at
                batch 1, 4 and 16, the Qwen-2.5-32B-shaped layers at 16 and
                64, the 8192 x 8192 prefill layer: product-kernel time,
                packed-weight GB/s and TFLOP/s with their fractions of peak,
                and the whole lq_linear time;
  encode        the nearest-neighbour encoders and the Eq. (1) training step;
  cpu_baseline  the CPU oracle on a bounded sample of the headline step.

Synthetic data: packed weights are uniformly random bytes (independent fair
signs), M ~ N(0, 1/D), row scales ~ U[0.5, 1.5], channel scales ~
U[0.8, 1.2], activations ~ N(0, 1) rounded to bf16.

Profiling helpers (the summaries under profiles/ are made with these):
  --phase-log FILE        write the order and number of product launches of
                          each measurement phase (for --summarize-stats)
  --pmc-workload          a 256 MiB device copy (the counter calibration),
                          then a few of each measured call; run it under
                          rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE
  --summarize-pmc F W     per-kernel FETCH_SIZE / WRITE_SIZE of those two
                          runs (their output directories), scaled by the copy
  --summarize-stats DIR   per-kernel calls and durations of a
                          rocprofv3 --kernel-trace --stats run; with
                          --phase-log, the product launches split by phase
  --summarize-util DIR    per-kernel matrix-core and LDS utilisation from a
                          rocprofv3 --pmc run of --pmc-workload with
                          SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA
                          SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP64_PEAK_TFLOPS = 78.6        # MI355X fp64 vector (FMA = 2 flops), TFLOP/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
ROOT = os.path.dirname(os.path.abspath(__file__))
SIGN_KERNEL = "sign_fp6_kernel"
LARGE_KERNEL = "sign_mfma_large_kernel"
WSPACE_KERNEL = "wspace_kernel"
# Kernels that carry the sign product of one lq_linear call (one per call).
PRODUCT_KERNELS = ("sign_fp6_kernel", "sign_fp6_chunked_kernel", "sign_valu_kernel",
                   "sign_mfma_large_kernel",
                   "wspace_kernel", "decode_fused_kernel", "decode_self_kernel",
                   "decode_split_kernel")
# The files of the kernels whose HBM traffic the committed summary holds.
# The source file of each kernel whose traffic the counter summary records
# (with every header, which they share).
TRAFFIC_SOURCES = {"sign_fp6_kernel": "sign_fp6.hip", "prep_kernel": "prep.hip",
                   "sign_mfma_large_kernel": "sign_mfma.hip", "wspace_kernel": "wspace.hip",
                   "xpw_kernel": "wspace.hip"}
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_llama3_70b_b1_step_and_prefill_28672_b2048.txt")
COPY_BYTES = 256 << 20         # the calibration copy of --pmc-workload

HEADLINE = "llama3_70b"
PREFILL_B = 2048

# Phases of the run, in order: (label, product launches); --phase-log.
PHASES = []


def phase(label, launches):
    PHASES.append((label, int(launches)))


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--weight-sets", type=int, default=6,
                   help="distinct copies of the headline step's weights (236.7 MB each)")
    p.add_argument("--config-reps", type=int, default=24,
                   help="calls per timed configuration row")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="approximate CPU time budget of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--decode-algo", default="auto",
                   choices=["auto", "small", "fused", "local", "split", "valu"],
                   help="algorithm of the decode lq_linear calls (lq_linear_ex; auto = lq_linear)")
    p.add_argument("--prefill-algo", default="auto", choices=["auto", "large", "wspace"],
                   help="algorithm of the prefill lq_linear call (lq_linear_ex; auto = lq_linear)")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the 2048-token prefill layer and the large-batch product")
    p.add_argument("--no-configs", action="store_true", help="skip the per-configuration rows")
    p.add_argument("--no-encode", action="store_true",
                   help="skip the encoder and training-step timings")
    p.add_argument("--gate-up", default="multi", choices=["multi", "separate"],
                   help="decode: gate and up (same x) in one lq_linear_multi call, or as two "
                        "lq_linear calls")
    p.add_argument("--eager", action="store_true",
                   help="launch the timed steps eagerly, each sign product timed by its own "
                        "dispatch events (slows the launches down)")
    p.add_argument("--phase-log", metavar="FILE")
    p.add_argument("--pmc-workload", action="store_true",
                   help="calibration copy plus a few of each measured call, for rocprofv3 --pmc")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    p.add_argument("--summarize-util", metavar="PMC_DIR")
    p.add_argument("--summarize-stats", metavar="DIR")
    return p.parse_args()


# ------------------------------------------------------------ profiling aids

def kernel_sources_hash(kernel):
    """Hash of the sources of `kernel` (a key of TRAFFIC_SOURCES): its .hip
    file and every header. Counters taken on other code are stale for it;
    host-only files such as the C-ABI dispatch, and the other kernels'
    files, do not change what it reads or writes."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_matmul_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith(".h") or name == TRAFFIC_SOURCES[kernel]:
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _read_rocprof_rows(d, kind):
    """Rows of a rocprofv3 output directory: ('pmc') counter rows as dicts
    with kernel, counter, value; ('trace') kernel dispatches with name,
    start and duration in ns. Reads the CSV files if present, else the
    SQLite db."""
    import csv
    import glob
    import sqlite3
    rows = []
    if kind == "pmc":
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(fn) as f:
                for r in csv.DictReader(f):
                    rows.append(dict(kernel=r.get("Kernel_Name", ""), counter=r.get("Counter_Name", ""),
                                     value=float(r.get("Counter_Value", "nan")),
                                     dispatch=r.get("Dispatch_Id", "")))
        if rows:
            return rows
        for fn in glob.glob(os.path.join(d, "**", "*results.db"), recursive=True):
            db = sqlite3.connect(fn)
            q = "select name, counter_name, counter_value, dispatch_id from pmc_events"
            try:
                for name, cn, v, did in db.execute(q):
                    rows.append(dict(kernel=name, counter=cn, value=float(v), dispatch=did))
            except sqlite3.Error:
                pass
        return rows
    for fn in glob.glob(os.path.join(d, "**", "*results.db"), recursive=True):
        db = sqlite3.connect(fn)
        for name, s0, e0 in db.execute("select name, start, end from kernels"):
            rows.append(dict(kernel=name, start=float(s0), duration=float(e0) - float(s0)))
    if not rows:
        for fn in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            with open(fn) as f:
                for r in csv.DictReader(f):
                    s0, e0 = float(r["Start_Timestamp"]), float(r["End_Timestamp"])
                    rows.append(dict(kernel=r["Kernel_Name"], start=s0, duration=e0 - s0))
    return rows


def _short(name):
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0].strip()


def summarize_stats(d, phase_log=None):
    """Per-kernel calls and durations. With `phase_log` (the --phase-log of
    the profiled run), also the product-kernel dispatches split by phase, in
    dispatch order, each phase's average next to the kernels it ran."""
    rows = _read_rocprof_rows(d, "trace")
    agg = {}
    for r in rows:
        agg.setdefault(_short(r["kernel"]), []).append(r["duration"])
    lines = ["kernel | calls | avg us | min us | max us | total us"]
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{k} | {len(v)} | {sum(v) / len(v) / 1e3:.3f} | {min(v) / 1e3:.3f} | "
                     f"{max(v) / 1e3:.3f} | {sum(v) / 1e3:.1f}")
    if phase_log:
        with open(phase_log) as f:
            phases = json.load(f)
        prod = sorted((r for r in rows if any(p in r["kernel"] for p in PRODUCT_KERNELS)),
                      key=lambda r: r["start"])
        need = sum(n for _, n in phases)
        lines.append("")
        lines.append(f"product-kernel dispatches by phase ({len(prod)} in the trace, "
                     f"{need} in the phase log)")
        if len(prod) == need:
            at = 0
            for label, n in phases:
                part = prod[at:at + n]
                at += n
                if not part:
                    continue
                names = sorted({_short(r["kernel"]) for r in part})
                avg = sum(r["duration"] for r in part) / n / 1e3
                lines.append(f"{label} | {n} launches | avg {avg:.3f} us | {', '.join(names)}")
        else:
            lines.append("phase log and trace disagree; phases not split")
    return "\n".join(lines)


def summarize_pmc(fetch_dir, write_dir):
    """Per-kernel average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) and the
    calibration factors: the known size of the --pmc-workload copy over what
    each counter reads for that copy (its largest copy dispatch)."""
    out, copy = {}, {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = {}
        for r in _read_rocprof_rows(d, "pmc"):
            if r["counter"] != counter:
                continue
            k = _short(r["kernel"])
            per.setdefault(k, []).append(r["value"])
            if "copyBuffer" in k:
                copy[counter] = max(copy.get(counter, 0.0), r["value"])
        out[counter] = {k: sum(v) / len(v) for k, v in per.items() if "copyBuffer" not in k}
    lines = [f"sources {k} {kernel_sources_hash(k)}" for k in sorted(TRAFFIC_SOURCES)]
    lines.append(f"copy_bytes {COPY_BYTES}")
    if "FETCH_SIZE" in copy and "WRITE_SIZE" in copy:
        lines.append(f"copy_fetch_kib {copy['FETCH_SIZE']:.1f}")
        lines.append(f"copy_write_kib {copy['WRITE_SIZE']:.1f}")
        lines.append(f"fetch_factor {COPY_BYTES / 1024.0 / copy['FETCH_SIZE']:.4f}")
        lines.append(f"write_factor {COPY_BYTES / 1024.0 / copy['WRITE_SIZE']:.4f}")
    for k in sorted(out["FETCH_SIZE"]):
        if not k.startswith("lq::"):
            continue
        lines.append(f"kernel {k} fetch_kib {out['FETCH_SIZE'][k]:.1f} "
                     f"write_kib {out['WRITE_SIZE'].get(k, float('nan')):.1f}")
    return "\n".join(lines)


XCDS, CUS, SIMDS_PER_CU = 8, 256, 4


def summarize_util(d):
    """Per-kernel averages over dispatches of the counters of one rocprofv3
    --pmc run, and what they give: the matrix pipe busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES, summed over the 1024 SIMDs, over the kernel's
    cycles: GRBM_GUI_ACTIVE summed over the 8 XCDs, divided by 8), LDS busy
    and bank-conflict fractions (SQ_LDS_IDX_ACTIVE and SQ_LDS_BANK_CONFLICT,
    summed over compute units, over the same cycles times 256), and cycles
    per MFMA instruction per SIMD."""
    per = {}
    for r in _read_rocprof_rows(d, "pmc"):
        k = _short(r["kernel"])
        if not k.startswith("lq::"):
            continue
        per.setdefault(k, {}).setdefault(r["counter"], []).append(r["value"])
    lines = ["kernel | dispatches | gpu cycles | mfma busy | mfma insts | cycles per mfma "
             "per SIMD | lds busy | lds bank-conflict cycles"]
    for k in sorted(per):
        c = {n: sum(v) / len(v) for n, v in per[k].items()}
        if "GRBM_GUI_ACTIVE" not in c or c.get("SQ_INSTS_MFMA", 0) == 0:
            continue
        cyc = c["GRBM_GUI_ACTIVE"] / XCDS
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (cyc * CUS * SIMDS_PER_CU)
        per_simd = c["SQ_VALU_MFMA_BUSY_CYCLES"] / c["SQ_INSTS_MFMA"]
        lds = c.get("SQ_LDS_IDX_ACTIVE", float("nan")) / (cyc * CUS)
        bank = c.get("SQ_LDS_BANK_CONFLICT", float("nan")) / (cyc * CUS)
        n = len(next(iter(per[k].values())))
        lines.append(f"{k} | {n} | {cyc:.0f} | {busy:.3f} | {c['SQ_INSTS_MFMA']:.0f} | "
                     f"{per_simd:.1f} | {lds:.3f} | {bank:.3f}")
    return "\n".join(lines)


def traffic_from_summary(kernel):
    """HBM bytes per launch of the kernel instance(s) whose name contains
    `kernel` (averaged over them) from the committed counter summary, or
    None when there is none or it was taken on other sources."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    import re
    kv, kern, src = {}, {}, {}
    for line in text.splitlines():
        parts = line.split()
        if len(parts) == 3 and parts[0] == "sources":
            src[parts[1]] = parts[2]
        if len(parts) >= 2 and parts[0] in ("fetch_factor", "write_factor"):
            kv[parts[0]] = parts[1]
        m = re.match(r"^kernel (.*) fetch_kib ([0-9.]+) write_kib ([0-9.]+)$", line)
        if m and kernel in m.group(1):
            kern[m.group(1)] = (float(m.group(2)), float(m.group(3)))
    if kernel not in TRAFFIC_SOURCES or src.get(kernel) != kernel_sources_hash(kernel) or not kern:
        return None
    ff, wf = float(kv["fetch_factor"]), float(kv["write_factor"])
    f = sum(v[0] for v in kern.values()) / len(kern)
    w = sum(v[1] for v in kern.values()) / len(kern)
    return round((f * ff + w * wf) * 1024.0, 1)


class HipEvents:
    """Raw hipEvent_t handles (the same HIP runtime torch and liblq use)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


# ------------------------------------------------------------ workloads

ALGO_NAMES = {0: "AUTO", 1: "VALU", 2: "MFMA_SMALL", 3: "MFMA_LARGE", 4: "FUSED",
              5: "FUSED_LOCAL", 6: "WSPACE", 7: "FUSED_SPLIT"}
ALGO_KERNEL = {1: "sign_valu_kernel", 2: SIGN_KERNEL, 3: LARGE_KERNEL, 4: "decode_fused_kernel",
               5: "decode_self_kernel", 6: WSPACE_KERNEL, 7: "decode_split_kernel"}


class LayerSets:
    """`n_sets` distinct copies of the packed weights (and r, c) of the
    named layers of one workload on the GPU, with one M per workload (the
    pages' single global mapping matrix per rate)."""

    def __init__(self, torch, lq, wl_name, names, n_sets, seed):
        from workloads import WORKLOADS
        wl = WORKLOADS[wl_name]
        by_name = {s.name: s for s in wl.layers}
        self.wl = wl
        self.specs = [(n, by_name[base]) for n, base in names]
        dev = "cuda"
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        s0 = self.specs[0][1]
        self.M = (torch.randn(s0.d, s0.D, device=dev, generator=gen) / s0.D ** 0.5).contiguous()
        self.sets = []
        for _ in range(n_sets):
            row = {}
            for pname, s in self.specs:
                nbytes = lq.lq_packed_size(s.N, s.K, s.d, s.D)
                packed = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev, generator=gen)
                r = torch.rand(s.N, device=dev, generator=gen) + 0.5
                c = torch.rand(s.K, device=dev, generator=gen) * 0.4 + 0.8
                st = lq.layer_struct(s.N, s.K, s.d, s.D, s.hb, packed, self.M, c, r)
                row[pname] = dict(name=pname, spec=s, packed=packed, r=r, c=c, struct=st, bytes=nbytes)
            self.sets.append(row)
        self.gen = gen

    def x(self, torch, K, B):
        return torch.randn(B, K, device="cuda", generator=self.gen).to(torch.bfloat16)


SPIN_MS_PER_CALL = 0.25      # host time to enqueue one timed call, generously
_SPIN_CYCLES_PER_MS = []


def spin_gpu(torch, ms):
    """Keep the current stream busy for about `ms` milliseconds (torch's
    bounded spin kernel, calibrated once with events). Without that kernel
    the replay is not queued ahead and its launches wait on the host."""
    if not hasattr(torch.cuda, "_sleep"):
        return
    if not _SPIN_CYCLES_PER_MS:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_MS.append(1_000_000 / max(a.elapsed_time(b), 1e-3))
    torch.cuda._sleep(int(min(ms, 200.0) * _SPIN_CYCLES_PER_MS[0]))


def time_calls(torch, lq, ev, fn, reps, warmup, label, eager=False):
    """Time `reps` calls fn(i), i = 0..reps-1, each enqueuing exactly one
    product launch per lq call it makes; `fn` returns the number of lq calls
    (product launches) it made. The timed calls run as one HIP graph replay
    (or eagerly with --eager); the product-kernel durations come from an
    eager replay of the same calls with dispatch events. Returns
    (ms per call, [kernel durations in ms], launches per call)."""
    n = 0
    for i in range(warmup):
        n += fn(i)
    torch.cuda.synchronize()
    phase(f"{label}: warm-up", n)
    per_call = n // max(warmup, 1)
    n_launch = per_call * reps
    starts, stops = ev.create(n_launch), ev.create(n_launch)
    if eager:
        lq.lq_profile_events(starts, stops)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(reps):
            fn(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        lq.lq_profile_events([], [])
        phase(f"{label}: timed eager calls with dispatch events", n_launch)
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                fn(i)
        g.replay()                      # the first replay uploads the graph (untimed)
        torch.cuda.synchronize()
        phase(f"{label}: graph upload replay", n_launch)
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        phase(f"{label}: timed graph replay", n_launch)
        # Queue the replay behind a spin kernel, so that its launches run
        # back to back from a full queue as in the graph replay rather than
        # each waiting for the host to enqueue it.
        spin_gpu(torch, SPIN_MS_PER_CALL * reps)
        lq.lq_profile_events(starts, stops)
        for i in range(reps):
            fn(i)
        torch.cuda.synchronize()
        lq.lq_profile_events([], [])
        phase(f"{label}: eager replay with dispatch events", n_launch)
        del g
    durs = [ev.elapsed_ms(a, b) for a, b in zip(starts, stops)]
    ev.destroy(starts)
    ev.destroy(stops)
    return (t1 - t0) * 1e3 / reps, durs, per_call


def workspace(torch, lq, structs, B, algo=None, multi=None):
    need = 0
    for st in structs:
        a = lq.LQ_ALGO_AUTO if algo is None else algo
        need = max(need, lq.lq_linear_workspace_size_ex(st, B, torch.bfloat16, a))
    if multi:
        need = max(need, lq.lq_linear_multi_workspace_size(multi, B, torch.bfloat16))
    return torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")   # zeroed control area


DECODE_ALGOS = {"auto": None, "small": "LQ_ALGO_MFMA_SMALL", "fused": "LQ_ALGO_FUSED",
                "local": "LQ_ALGO_FUSED_LOCAL", "split": "LQ_ALGO_FUSED_SPLIT",
                "valu": "LQ_ALGO_VALU"}


def decode_step_fn(torch, lq, sets, order, x_in, ys, ws, grouped, algo):
    """A decode step over the layers `order` (names; a tuple of two names =
    layers on the same input, grouped in one lq_linear_multi call)."""
    def call(l, x):
        if algo is not None and l.get("algo_ok", {}).get(algo, True):
            try:
                lq.lq_linear_ex(l["struct"], x, 1, ys[l["name"]], algo, ws)
                return
            except lq.LQError:          # does not apply to this layer: lq_linear's choice
                l.setdefault("algo_ok", {})[algo] = False
        lq.lq_linear(l["struct"], x, 1, ys[l["name"]], ws)

    def step(i):
        row = sets.sets[i % len(sets.sets)]
        n = 0
        for item in order:
            if isinstance(item, tuple):
                ls = [row[nm] for nm in item]
                if grouped:
                    lq.lq_linear_multi([l["struct"] for l in ls], x_in[item[0]], 1,
                                       [ys[nm] for nm in item], ws)
                    n += 1
                else:
                    for l in ls:
                        call(l, x_in[item[0]])
                        n += 1
            else:
                call(row[item], x_in[item])
                n += 1
        return n
    return step


def run_decode_step(args, torch, lq, ev, wl_name, names, order, n_sets, label, seed):
    algo_name = DECODE_ALGOS[args.decode_algo]
    algo = None if algo_name is None else getattr(lq, algo_name)
    sets = LayerSets(torch, lq, wl_name, names, n_sets, seed)
    first = sets.sets[0]
    x_in = {nm: sets.x(torch, first[nm]["spec"].K, 1) for nm, _ in names}
    ys = {nm: torch.empty((1, first[nm]["spec"].N), dtype=torch.bfloat16, device="cuda")
          for nm, _ in names}
    grouped = args.gate_up == "multi" and algo is None
    multi = None
    for item in order:
        if isinstance(item, tuple):
            multi = [first[nm]["struct"] for nm in item]
    algos = [lq.LQ_ALGO_AUTO] + ([algo] if algo is not None else [])
    need = 16
    for nm, _ in names:
        for a in algos:
            try:
                need = max(need, lq.lq_linear_workspace_size_ex(first[nm]["struct"], 1,
                                                                torch.bfloat16, a))
            except lq.LQError:
                pass
    if multi:
        need = max(need, lq.lq_linear_multi_workspace_size(multi, 1, torch.bfloat16))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    step = decode_step_fn(torch, lq, sets, order, x_in, ys, ws, grouped, algo)
    ms, durs, per_step = time_calls(torch, lq, ev, step, args.steps, args.warmup, label,
                                    eager=args.eager)
    step_bytes = sum(l["bytes"] for l in first.values())
    # launch j of a step reads the packed bytes of its layers
    launch_layers = []
    for item in order:
        if isinstance(item, tuple) and grouped:
            launch_layers.append(list(item))
        elif isinstance(item, tuple):
            launch_layers += [[nm] for nm in item]
        else:
            launch_layers.append([item])
    per_launch = []
    for j, lay in enumerate(launch_layers):
        d = durs[j::per_step]
        nb = sum(first[nm]["bytes"] for nm in lay)
        us = sum(d) / len(d) * 1e3
        per_launch.append(dict(layers="+".join(lay), packed_bytes=nb, kernel_us=round(us, 3),
                               gbs=round(nb / (us * 1e-6) / 1e9, 1),
                               frac=round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)))
    kern_ms = sum(durs) / len(durs)
    bytes_per_launch = step_bytes / per_step
    res = dict(ms_step=ms, gbs=step_bytes / (ms * 1e-3) / 1e9, kern_ms=kern_ms,
               achieved=bytes_per_launch / (kern_ms * 1e-3) / 1e9, step_bytes=step_bytes,
               bytes_per_launch=bytes_per_launch, per_launch=per_launch, n_sets=n_sets,
               grouped=grouped, launches_per_step=per_step)
    del sets, ws
    torch.cuda.empty_cache()
    return res


HEADLINE_NAMES = [("qkv", "qkv"), ("gate", "gate_up"), ("up", "gate_up"), ("down", "down")]
HEADLINE_ORDER = ["qkv", ("gate", "up"), "down"]


def run_config_rows(args, torch, lq, ev):
    """Product-kernel and lq_linear times of every layer and batch size of
    the workloads other than the headline step. Each layer rotates over
    enough distinct weight copies that a pass touches >= 600 MB (twice and
    more the 256 MB Infinity Cache)."""
    rows = []
    plan = [("llama3_70b", ("gate_up", "down", "qkv"), (1, 4, 16)),
            ("qwen25_32b", ("up", "down"), (16, 64)),
            ("prefill", ("sq",), (PREFILL_B,))]
    for wl_name, names, batches in plan:
        for nm in names:
            from workloads import WORKLOADS
            spec = {s.name: s for s in WORKLOADS[wl_name].layers}[nm]
            n_sets = 2 if wl_name == "prefill" else -(-600_000_000 // (spec.N * spec.L // 8))
            sets = LayerSets(torch, lq, wl_name, [(nm, nm)], n_sets, seed=11)
            structs = [row[nm]["struct"] for row in sets.sets]
            for B in batches:
                ws = workspace(torch, lq, structs[:1], B)
                x = sets.x(torch, spec.K, B)
                y = torch.empty((B, spec.N), dtype=torch.bfloat16, device="cuda")

                def fn(i, structs=structs, x=x, y=y, ws=ws, B=B):
                    lq.lq_linear(structs[i % len(structs)], x, B, y, ws)
                    return 1
                reps = max(args.config_reps, n_sets) if B <= 64 else 6
                label = f"{wl_name} {nm} B={B}"
                ms, durs, _ = time_calls(torch, lq, ev, fn, reps, 2, label)
                algo = lq.lq_linear_algo(structs[0], B, torch.bfloat16)
                row = config_row(wl_name, nm, spec, B, algo, ms, durs)
                row["weight_sets"] = n_sets
                rows.append(row)
                print(f"[bench] {label}: kernel {row['kernel_us']:.2f} us "
                      f"({row['gbs']:.0f} GB/s, {row['kernel_tflops']:.1f} TFLOP/s)",
                      file=sys.stderr, flush=True)
                del ws, x, y
            del sets, structs
            torch.cuda.empty_cache()
    return rows


def config_row(wl_name, nm, s, B, algo, ms, durs):
    kus = sum(durs) / len(durs) * 1e3
    nbytes = s.N * s.L // 8
    lifted = 2.0 * B * s.N * s.L
    dense = 2.0 * B * s.N * s.Kpad
    kflops = dense if algo == 6 else lifted          # W space multiplies over K'
    gbs = nbytes / (kus * 1e-6) / 1e9
    tf = kflops / (kus * 1e-6) / 1e12
    return dict(workload=f"{wl_name} {nm}", K=s.K, N=s.N, d=s.d, D=s.D, L=s.L, B=B,
                algo=ALGO_NAMES[algo], kernel=ALGO_KERNEL[algo], packed_bytes=nbytes,
                kernel_us=round(kus, 3), linear_us=round(ms * 1e3, 3),
                gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4),
                kernel_tflops=round(tf, 2), frac_bf16=round(tf / BF16_PEAK_TFLOPS, 4),
                lifted_tflops_linear=round(lifted / (ms * 1e-3) / 1e12, 2),
                kernel_flops=kflops)


def run_prefill(args, torch, lq, ev, algo_name, label, reps=6):
    """The 8192 -> 28672 prefill layer (d = 3, D = 8) at B = 2048."""
    algo = None if algo_name is None else getattr(lq, algo_name)
    sets = LayerSets(torch, lq, "prefill", [("wide", "wide")], 1, seed=1)
    l = sets.sets[0]["wide"]
    s, st = l["spec"], l["struct"]
    B = PREFILL_B
    a = lq.LQ_ALGO_AUTO if algo is None else algo
    ws = workspace(torch, lq, [st], B, algo=a)
    x = sets.x(torch, s.K, B)
    y = torch.empty(B, s.N, dtype=torch.bfloat16, device="cuda")

    def fn(i):
        if algo is None:
            lq.lq_linear(st, x, B, y, ws)
        else:
            lq.lq_linear_ex(st, x, B, y, algo, ws)
        return 1
    ms, durs, _ = time_calls(torch, lq, ev, fn, reps, 2, label)
    resolved = lq.lq_linear_algo(st, B, torch.bfloat16, a)
    row = config_row("prefill", "wide", s, B, resolved, ms, durs)
    del sets, ws, x, y
    torch.cuda.empty_cache()
    return row


def run_encode(torch, lq, reps=3):
    """lq_encode at the 2.4-bit rate (d = 10, D = 24: 2^24 sign vectors per
    block) on 4096 blocks and at the prefill rate (d = 3, D = 8) on a whole
    8192 x 8192 layer's blocks; lq_train_m_step (d = 3, D = 8) on 65536
    Gaussian samples. Kernel time from torch events on the stream the
    library launches on (its current stream)."""
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)

    def orth(d, D):
        q, r = torch.linalg.qr(torch.randn(D, D, device=dev, generator=gen, dtype=torch.float64))
        return (q * torch.sign(torch.diagonal(r))[None, :])[:, :d].T.contiguous().float()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / reps
    out = []
    for d, D, n, label in ((10, 24, 4096, "2.4-bit rate (d=10, D=24), 4096 blocks"),
                           (3, 8, 8192 * 2731, "2.67-bit rate (d=3, D=8), the 8192x8192 layer's 22.4M blocks")):
        M = orth(d, D)
        w = torch.randn(n, d, device=dev, generator=gen)
        signs = torch.empty(n, D, dtype=torch.int8, device=dev)
        ms = timed(lambda: lq.lq_encode(w, n, d, D, M, signs))
        flops = float(n) * (1 << D) * 4 * d        # per visited vector: d updates + d distance FMAs
        out.append(dict(workload=label, d=d, D=D, blocks=n, ms=ms, blocks_per_s=n / (ms * 1e-3),
                        tflops=flops / (ms * 1e-3) / 1e12))
    # the 2^(D-d) pseudo-inverse-initialised search: LQ-24/10 and LQ-32/16
    for d, D, n, label in ((10, 24, 65536, "pseudo-inverse search, 2.4-bit rate (d=10, D=24: 2^14 "
                                           "candidates per block), 65536 blocks"),
                           (16, 32, 16384, "pseudo-inverse search, 2-bit LQ-32/16 (2^16 candidates "
                                           "per block), 16384 blocks")):
        M = orth(d, D)
        w = torch.randn(n, d, device=dev, generator=gen)
        signs = torch.empty(n, D, dtype=torch.int8, device=dev)
        ws = torch.zeros(lq.lq_encode_pinv_workspace_size(d, D), dtype=torch.uint8, device=dev)
        ms = timed(lambda: lq.lq_encode_pinv(w, n, d, D, M, signs, None, ws))
        # per candidate: 2d updates, d^2 residual and d distance FMAs
        flops = float(n) * (1 << (D - d)) * 2 * (d * d + 3 * d)
        out.append(dict(workload=label, d=d, D=D, blocks=n, ms=ms, blocks_per_s=n / (ms * 1e-3),
                        tflops=flops / (ms * 1e-3) / 1e12, search="pinv"))
    d, D, n = 3, 8, 65536
    M = orth(d, D)
    w = torch.randn(n, d, device=dev, generator=gen)
    loss = torch.zeros(1, device=dev)
    ws = torch.zeros(lq.lq_train_m_step_workspace_size(n, d, D), dtype=torch.uint8, device=dev)
    ms_train = timed(lambda: lq.lq_train_m_step(M, w, n, d, D, 0.01, loss, ws))
    return out, dict(workload=f"one Eq. (1) step, d={d}, D={D}, {n} Gaussian samples", ms=ms_train)


def encode_cpu_baseline():
    """The oracle's exhaustive search on a small sample of the same blocks."""
    import numpy as np
    from oracle import liftquant_ref as ref
    rng = np.random.default_rng(3)
    res = []
    for d, D, n, fn, search in ((10, 24, 1, ref.encode_nn, "exhaustive"),
                                (3, 8, 20000, ref.encode_nn, "exhaustive"),
                                (10, 24, 20, ref.encode_pinv, "pinv"),
                                (16, 32, 8, ref.encode_pinv, "pinv")):
        M = ref.orthonormal_rows(rng.standard_normal((D, D)), d)
        w = rng.standard_normal((n, d))
        t0 = time.perf_counter()
        fn(w, M)
        dt = time.perf_counter() - t0
        res.append(dict(d=d, D=D, blocks=n, search=search, seconds=round(dt, 3),
                        blocks_per_s=round(n / dt, 3)))
    return res


def cpu_threads():
    """Threads the oracle's numpy uses (its BLAS pool)."""
    try:
        import numpy  # noqa: F401  (loads the BLAS pool threadpoolctl inspects)
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def host_cpu():
    """Logical CPUs this process may run on, all online ones, and the model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return dict(usable=usable, online=os.cpu_count() or 1, model=model)


def cpu_baseline(budget_s):
    """The oracle as it stands, on rows sampled from the layers of the
    headline step (QKV, gate, up, down of the Llama-3-70B block, batch 1)."""
    import numpy as np
    from oracle import liftquant_ref as ref
    from workloads import WORKLOADS, make_layer
    threads = cpu_threads()
    wl = WORKLOADS[HEADLINE]
    by = {s.name: s for s in wl.layers}
    inputs = {nm: make_layer(s, wl, B_max=1) for nm, s in by.items()}
    step = [by["qkv"], by["gate_up"], by["gate_up"], by["down"]]

    def run(rows):
        nbytes = 0
        t = 0.0
        for s in step:
            li = inputs[s.name]
            idx = np.arange(rows)
            signs = li.signs_rows(idx)
            t0 = time.perf_counter()
            ref.linear(li.x(1), li.c, s.hb, li.M, signs, li.row_scale[idx])
            t += time.perf_counter() - t0
            nbytes += rows * s.L // 8
        return nbytes, t

    rows = 32
    nb, t = run(rows)
    reps = 1
    if t < budget_s / 4:
        rows = int(min(4096, max(32, rows * budget_s / 2 / max(t, 1e-3))) // 16 * 16)
        nb, t = run(rows)
        reps = max(1, int(budget_s / max(t, 1e-3)))        # repeat the sample up to the budget
        for _ in range(reps - 1):
            nb2, t2 = run(rows)
            nb += nb2
            t += t2
    cpu = host_cpu()
    return dict(value=round(nb / t / 1e9, 6), unit="GB/s", cores=threads, kind="oracle",
                nproc=cpu["usable"], online_cpus=cpu["online"], cpu_model=cpu["model"],
                sample=f"oracle linear() on the first {rows} rows of each of QKV, gate, up and "
                       f"down of the Llama-3-70B block (B=1, d=10, D=24), {reps} times: {nb} "
                       f"packed bytes in {t:.2f} s; cores = the oracle's BLAS threads")


def pmc_workload(args, torch, lq):
    """The calibration copy, then a few of each measured call (eagerly)."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    sets = LayerSets(torch, lq, HEADLINE, HEADLINE_NAMES, 3, seed=0)
    first = sets.sets[0]
    x_in = {nm: sets.x(torch, first[nm]["spec"].K, 1) for nm, _ in HEADLINE_NAMES}
    ys = {nm: torch.empty((1, first[nm]["spec"].N), dtype=torch.bfloat16, device="cuda")
          for nm, _ in HEADLINE_NAMES}
    multi = [first["gate"]["struct"], first["up"]["struct"]]
    ws = workspace(torch, lq, [first[nm]["struct"] for nm, _ in HEADLINE_NAMES], 1, multi=multi)
    step = decode_step_fn(torch, lq, sets, HEADLINE_ORDER, x_in, ys, ws, True, None)
    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    del sets, ws
    for algo_name in (None, "LQ_ALGO_MFMA_LARGE"):
        algo = None if algo_name is None else getattr(lq, algo_name)
        sets = LayerSets(torch, lq, "prefill", [("wide", "wide")], 1, seed=1)
        l = sets.sets[0]["wide"]
        s, st = l["spec"], l["struct"]
        a = lq.LQ_ALGO_AUTO if algo is None else algo
        ws = workspace(torch, lq, [st], PREFILL_B, algo=a)
        x = sets.x(torch, s.K, PREFILL_B)
        y = torch.empty(PREFILL_B, s.N, dtype=torch.bfloat16, device="cuda")
        lq.lq_linear_ex(st, x, PREFILL_B, y, a, ws)
        torch.cuda.synchronize()
        del sets, ws, x, y
    print("pmc workload done", flush=True)


def main():
    args = parse_args()
    if args.summarize_stats:
        print(summarize_stats(args.summarize_stats, args.phase_log))
        return
    if args.summarize_pmc:
        print(summarize_pmc(*args.summarize_pmc))
        return
    if args.summarize_util:
        print(summarize_util(args.summarize_util))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch
    import bit_matmul_amd as lq
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.pmc_workload:
        pmc_workload(args, torch, lq)
        return
    ev = HipEvents()
    dec = run_decode_step(args, torch, lq, ev, HEADLINE, HEADLINE_NAMES, HEADLINE_ORDER,
                          args.weight_sets, "Llama-3-70B decode step B=1", seed=0)
    print(f"[bench] headline step: {dec['ms_step'] * 1e3:.2f} us, {dec['gbs']:.1f} GB/s",
          file=sys.stderr, flush=True)
    grouped = dec["grouped"]
    out = {
        "metric": "LiftQuant linear: packed-weight HBM GB/s (batch 1) and TFLOP/s (batch 2048)",
        "value": round(dec["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3-70B block decode at 2.4 bit (d=10, D=24), batch 1, bf16 "
                        "activations, Hadamard block 1024: QKV K=8192->N=10240, gate and up "
                        "K=8192->N=28672, down K=28672->N=8192; one step = the four projections"
                        + (" (QKV in one lq_linear call, gate and up, which read the same x, in "
                           "one lq_linear_multi call, down in one lq_linear call)" if grouped
                           else " as lq_linear calls"),
            "global_batch": 1,
            "weight_sets": dec["n_sets"],
            "packed_bytes_per_step": dec["step_bytes"],
            "graph": not args.eager,
            "decode_algo": args.decode_algo,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": f"sign product (lq {SIGN_KERNEL})",
            "achieved": round(dec["achieved"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec["achieved"] / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_summary(SIGN_KERNEL),
            "avg_launch_us": round(dec["kern_ms"] * 1e3, 3),
            "launches_per_step": dec["launches_per_step"],
            "per_launch": dec["per_launch"],
            "timing": "hipEvents recorded by the dispatch of every sign-product launch of an "
                      "eager replay of the K timed steps, queued behind a spin kernel so that "
                      "its launches run back to back as in the timed graph replay",
            "algorithmic_bytes_per_launch": dec["bytes_per_launch"],
        },
    }
    if not args.no_prefill:
        algo_name = {"auto": None, "large": "LQ_ALGO_MFMA_LARGE",
                     "wspace": "LQ_ALGO_WSPACE"}[args.prefill_algo]
        pf = run_prefill(args, torch, lq, ev, algo_name, "prefill 8192->28672 B=2048")
        print(f"[bench] prefill: {pf['linear_us']:.1f} us per lq_linear", file=sys.stderr, flush=True)
        lifted = 2.0 * pf["B"] * pf["N"] * pf["L"]
        out["prefill"] = {
            "metric": "TFLOP/s (batch 2048), lifted flops 2*B*N*L per lq_linear call",
            "workload": f"prefill K={pf['K']} N={pf['N']} d={pf['d']} D={pf['D']} B={pf['B']}",
            "algo": pf["algo"],
            "kernel": pf["kernel"],
            "value": pf["lifted_tflops_linear"],
            "unit": "TFLOP/s",
            "ms_per_linear": round(pf["linear_us"] / 1e3, 4),
            "lifted_flops": lifted,
            "note": ("value counts the 2*B*N*L flops of the lifted product for the whole call; "
                     "it is not a rate the matrix cores ran at when the W-space product (D/d "
                     "times fewer flops) runs: that rate is roofline.achieved"),
            "roofline": {"bound": "mfma", "achieved": pf["kernel_tflops"],
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": pf["frac_bf16"],
                         "kernel_flops_per_launch": pf["kernel_flops"],
                         "flops_convention": ("2*B*N*K' (dense-equivalent: the W-space "
                                              "product multiplies over K')"
                                              if pf["algo"] == "WSPACE" else "2*B*N*L"),
                         "avg_launch_us": pf["kernel_us"],
                         "traffic": traffic_from_summary(pf["kernel"])},
        }
        lg = run_prefill(args, torch, lq, ev, "LQ_ALGO_MFMA_LARGE",
                         "prefill 8192->28672 B=2048, lifted product")
        out["large"] = {
            "metric": "TFLOP/s of the lifted large-batch product (2*B*N*L per launch)",
            "workload": f"prefill K={lg['K']} N={lg['N']} d={lg['d']} D={lg['D']} B={lg['B']}, "
                        "LQ_ALGO_MFMA_LARGE",
            "kernel": LARGE_KERNEL,
            "ms_per_linear": round(lg["linear_us"] / 1e3, 4),
            "roofline": {"bound": "mfma", "achieved": lg["kernel_tflops"],
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": lg["frac_bf16"],
                         "kernel_flops_per_launch": lg["kernel_flops"],
                         "avg_launch_us": lg["kernel_us"],
                         "traffic": traffic_from_summary(LARGE_KERNEL)},
        }
    if not args.no_configs:
        step8 = run_decode_step(args, torch, lq, ev, "llama3_8b_mlp",
                                [("gate", "gate_up"), ("up", "gate_up"), ("down", "down")],
                                [("gate", "up"), "down"], 24, "Llama-3-8B MLP decode step B=1",
                                seed=2)
        rows = run_config_rows(args, torch, lq, ev)
        out["configs"] = {
            "note": "kernel_us = the product kernel (event-timed by its dispatch, eager replay); "
                    "linear_us = one whole lq_linear call (graph replay); gbs = packed bytes / "
                    "kernel_us; kernel_tflops = the kernel's flops (2*B*N*L lifted, 2*B*N*K' "
                    "for W space) / kernel_us",
            "llama3_8b_mlp_step_b1": {
                "gbs_per_step": round(step8["gbs"], 1), "ms_per_step": round(step8["ms_step"], 6),
                "packed_bytes_per_step": step8["step_bytes"], "per_launch": step8["per_launch"],
                "weight_sets": step8["n_sets"]},
            "rows": rows,
        }
    if not args.no_encode:
        enc, train = run_encode(torch, lq)
        big = enc[0]
        out["encode"] = {
            "metric": "blocks/s encoded (the nearest-neighbour search of Eq. (1)'s inner minimisation: "
                      "exhaustive over 2^D, or the 2^(D-d) pseudo-inverse-initialised search)",
            "workloads": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in e.items()}
                          for e in enc],
            "kernel": "encode_kernel",
            "roofline": {"bound": "alu", "achieved": round(big["tflops"], 2),
                         "peak": FP64_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(big["tflops"] / FP64_PEAK_TFLOPS, 4),
                         "workload": big["workload"],
                         "flops": "4 d fp64 flops per visited sign vector (2^D per block)",
                         "traffic": None},
            "train_step": {"workload": train["workload"], "ms": round(train["ms"], 4)},
        }
        if not args.no_cpu_baseline:
            out["encode"]["cpu_baseline"] = {"kind": "oracle", "cores": cpu_threads(),
                                             "samples": encode_cpu_baseline()}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    if args.phase_log:
        with open(args.phase_log, "w") as f:
            json.dump(PHASES, f)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
