#!/usr/bin/env python3
"""Benchmark of the LiftQuant decode operator on one MI355X.

A step is one decode token through the three MLP projections of a
Llama-3-8B layer at 2.4 bits per weight (d = 10, D = 24): gate and up
(K = 4096 -> N = 14336) and down (K = 14336 -> N = 4096), batch 1, bf16
activations, each a full lq_linear call (whitening, lift, sign product).
Every step uses the next of `--weight-sets` distinct copies of the packed
weights, so the 52.9 MB of packed bits a step reads cannot stay in the
256 MB Infinity Cache (like a real 32-layer model, whose weights are all
different). The K timed steps are captured once in a HIP graph and replayed;
the sign-product kernel durations come from an eager replay of the same K
steps right after, each launch timed by events its own dispatch records
(recording them inside the timed region would slow it down).

Printed (one JSON line): whole-step packed-weight throughput in GB/s
(`value`), the roofline of the dominant kernel (the sign product), timed
with HIP events around each of its launches inside the timed graph, and the
CPU oracle's rate on a bounded sample of the same workload. With
The 2048-token prefill layer (d = 3, D = 8) is timed too, in TFLOP/s (its
own object in the line; `--no-prefill` skips it), and so are the
nearest-neighbour encoder and the training step of M (`encode` object;
`--no-encode` skips it).

Synthetic data: packed weights are uniformly random bytes (i.e. independent
fair signs), M ~ N(0, 1/D), row scales ~ U[0.5, 1.5], channel scales ~
U[0.8, 1.2], activations ~ N(0, 1) rounded to bf16.

Profiling helpers (the summaries under profiles/ are made with these):
  --pmc-workload          a 256 MiB device copy (the counter calibration),
                          then a few eager decode steps; run it under
                          rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE
  --summarize-pmc F W     per-kernel FETCH_SIZE / WRITE_SIZE of those two
                          runs (their output directories), scaled by the copy
  --summarize-stats DIR   per-kernel calls and durations of a
                          rocprofv3 --kernel-trace --stats run
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
# The files of the kernels whose HBM traffic the committed summary holds.
TRAFFIC_SOURCES = ("sign_fp6.hip", "prep.hip", "sign_mfma.hip", "wspace.hip")
LARGE_KERNEL = "sign_mfma_large_kernel"
WSPACE_KERNEL = "wspace_kernel"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_llama3_8b_mlp_b1_and_prefill_8192_b2048.txt")
COPY_BYTES = 256 << 20         # the calibration copy of --pmc-workload


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--weight-sets", type=int, default=24)
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="approximate CPU time budget of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--decode-algo", default="auto",
                   choices=["auto", "small", "fused", "local", "split", "valu"],
                   help="algorithm of the decode lq_linear calls (lq_linear_ex; auto = lq_linear)")
    p.add_argument("--prefill-algo", default="auto", choices=["auto", "large", "wspace"],
                   help="algorithm of the prefill lq_linear call (lq_linear_ex; auto = lq_linear)")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the 2048-token prefill layer (TFLOP/s)")
    p.add_argument("--no-encode", action="store_true",
                   help="skip the encoder and training-step timings")
    p.add_argument("--gate-up", default="multi", choices=["multi", "separate"],
                   help="decode: gate and up (same x) in one lq_linear_multi call, or as two "
                        "lq_linear calls")
    p.add_argument("--eager", action="store_true",
                   help="launch the timed steps eagerly, each sign product timed by its own "
                        "dispatch events (slows the launches down)")
    p.add_argument("--pmc-workload", action="store_true",
                   help="calibration copy plus a few eager decode steps, for rocprofv3 --pmc")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    p.add_argument("--summarize-util", metavar="PMC_DIR")
    p.add_argument("--summarize-stats", metavar="DIR")
    p.add_argument("--profiled-steps", type=int, default=None,
                   help="with --summarize-stats: the --steps of the profiled run")
    return p.parse_args()


# ------------------------------------------------------------ profiling aids

def kernel_sources_hash():
    """Hash of the sources of the kernels the counter summary covers (their
    .hip files and every header; a summary taken on other code is stale).
    Host-only files such as the C-ABI dispatch, and kernels the summary does
    not cover, do not change what these kernels read or write."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_matmul_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith(".h") or name in TRAFFIC_SOURCES:
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _read_rocprof_rows(d, kind):
    """Rows of a rocprofv3 output directory: ('pmc') counter rows as dicts
    with kernel, counter, value; ('trace') kernel dispatches with name and
    duration in ns. Reads the CSV files if present, else the SQLite db."""
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
        for name, dur in db.execute("select name, duration from kernels"):
            rows.append(dict(kernel=name, duration=float(dur)))
    for fn in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                rows.append(dict(kernel=r["Kernel_Name"],
                                 duration=float(r["End_Timestamp"]) - float(r["Start_Timestamp"])))
    return rows


def _short(name):
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0].strip()


def summarize_stats(d, steps=None):
    """Per-kernel calls and durations. With `steps` (the --steps of the
    profiled bench run), also the sign-product dispatches split by phase:
    the graph's timed replay and the eager replay whose dispatch events give
    bench.py's kernel durations (the last 3 * steps sign launches)."""
    rows = _read_rocprof_rows(d, "trace")
    agg = {}
    for r in rows:
        a = agg.setdefault(_short(r["kernel"]), [])
        a.append(r["duration"])
    lines = ["kernel | calls | avg us | min us | max us | total us"]
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{k} | {len(v)} | {sum(v) / len(v) / 1e3:.3f} | {min(v) / 1e3:.3f} | "
                     f"{max(v) / 1e3:.3f} | {sum(v) / 1e3:.1f}")
    if steps:
        import glob
        import sqlite3
        sign = []
        for fn in glob.glob(os.path.join(d, "**", "*results.db"), recursive=True):
            db = sqlite3.connect(fn)
            sign += [(s0, e0) for n, s0, e0 in db.execute("select name, start, end from kernels")
                     if SIGN_KERNEL in n]
        sign.sort()
        dur = [e0 - s0 for s0, e0 in sign]
        n = 3 * steps
        if len(dur) >= 2 * n:
            timed, replay = dur[-2 * n:-n], dur[-n:]
            lines.append("")
            lines.append(f"{SIGN_KERNEL}, graph timed replay ({n} launches): avg "
                         f"{sum(timed) / n / 1e3:.3f} us")
            lines.append(f"{SIGN_KERNEL}, eager replay with dispatch events ({n} launches): avg "
                         f"{sum(replay) / n / 1e3:.3f} us")
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
    lines = [f"sources {kernel_sources_hash()}",
             f"copy_bytes {COPY_BYTES}"]
    if "FETCH_SIZE" in copy and "WRITE_SIZE" in copy:
        lines.append(f"copy_fetch_kib {copy['FETCH_SIZE']:.1f}")
        lines.append(f"copy_write_kib {copy['WRITE_SIZE']:.1f}")
        lines.append(f"fetch_factor {COPY_BYTES / 1024.0 / copy['FETCH_SIZE']:.4f}")
        lines.append(f"write_factor {COPY_BYTES / 1024.0 / copy['WRITE_SIZE']:.4f}")
    for k in sorted(out["FETCH_SIZE"]):
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


def traffic_from_summary(kernel=SIGN_KERNEL):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when there is none or it was taken on other sources."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    import re
    kv, kern = {}, {}
    for line in text.splitlines():
        parts = line.split()
        if len(parts) >= 2 and parts[0] in ("sources", "fetch_factor", "write_factor"):
            kv[parts[0]] = parts[1]
        m = re.match(r"^kernel (.*) fetch_kib ([0-9.]+) write_kib ([0-9.]+)$", line)
        if m and kernel in m.group(1):
            kern[m.group(1)] = (float(m.group(2)), float(m.group(3)))
    if kv.get("sources") != kernel_sources_hash() or not kern:
        return None
    ff, wf = float(kv["fetch_factor"]), float(kv["write_factor"])
    f = sum(v[0] for v in kern.values()) / len(kern)
    w = sum(v[1] for v in kern.values()) / len(kern)
    return round((f * ff + w * wf) * 1024.0, 1)


def pmc_workload(torch, lq):
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    specs, layers, x_in, ys, ws, M = build_decode_case(torch, lq, 4)
    for i in range(3):                           # the decode step as the benchmark runs it
        gate, up, down = layers[i % len(layers)]
        lq.lq_linear_multi([gate["struct"], up["struct"]], x_in["gate"], 1, [ys["gate"], ys["up"]], ws)
        lq.lq_linear(down["struct"], x_in["down"], 1, ys["down"], ws)
    torch.cuda.synchronize()
    pf = build_prefill_case(torch, lq)
    lq.lq_linear(pf["struct"], pf["x"], pf["B"], pf["y"], pf["ws"])
    torch.cuda.synchronize()
    print("pmc workload done", flush=True)


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


def build_decode_case(torch, lq, n_sets, seed=0):
    from workloads import WORKLOADS, make_layer
    wl = WORKLOADS["llama3_8b_mlp"]
    gate_spec, down_spec = wl.layers
    specs = [("gate", gate_spec), ("up", gate_spec), ("down", down_spec)]
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    host = {s.name: make_layer(s, wl, B_max=1) for s in (gate_spec, down_spec)}
    M = torch.from_numpy(host[gate_spec.name].M).to(dev)        # one global mapping matrix
    layers = []   # [set][proj] -> dict
    for _ in range(n_sets):
        row = []
        for pname, s in specs:
            nbytes = lq.lq_packed_size(s.N, s.K, s.d, s.D)
            packed = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev, generator=gen)
            r = torch.rand(s.N, device=dev, generator=gen) + 0.5
            c = torch.rand(s.K, device=dev, generator=gen) * 0.4 + 0.8
            st = lq.layer_struct(s.N, s.K, s.d, s.D, s.hb, packed, M, c, r)
            row.append(dict(name=pname, spec=s, packed=packed, r=r, c=c, struct=st, bytes=nbytes))
        layers.append(row)
    x_in = {
        "gate": torch.from_numpy(host[gate_spec.name].x(1)).to(dev).to(torch.bfloat16),
        "down": torch.from_numpy(host[down_spec.name].x(1)).to(dev).to(torch.bfloat16),
    }
    ys = {p: torch.empty((1, s.N), dtype=torch.bfloat16, device=dev) for p, s in specs}
    def need(st, a):
        try:
            return lq.lq_linear_workspace_size_ex(st, 1, torch.bfloat16, a)
        except lq.LQError:                                     # does not apply to this layer
            return 0
    ws_bytes = max(need(layers[0][i]["struct"], a) for i in range(3)
                   for a in (lq.LQ_ALGO_AUTO, lq.LQ_ALGO_MFMA_SMALL, lq.LQ_ALGO_FUSED_SPLIT))
    ws_bytes = max(ws_bytes, lq.lq_linear_multi_workspace_size(
        [layers[0][0]["struct"], layers[0][1]["struct"]], 1, torch.bfloat16))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)      # zeroed control area
    return specs, layers, x_in, ys, ws, M


def run_decode(args, torch, lq, ev):
    specs, layers, x_in, ys, ws, M = build_decode_case(torch, lq, args.weight_sets)
    n_sets = len(layers)
    step_bytes = sum(l["bytes"] for l in layers[0])

    algo = {"auto": None, "small": lq.LQ_ALGO_MFMA_SMALL, "fused": lq.LQ_ALGO_FUSED,
            "local": lq.LQ_ALGO_FUSED_LOCAL, "split": lq.LQ_ALGO_FUSED_SPLIT,
            "valu": lq.LQ_ALGO_VALU}[args.decode_algo]

    def call(l, x):
        # An algorithm that does not apply to a layer falls back to lq_linear's choice.
        if algo is not None and l.get("algo_ok", {}).get(algo, True):
            try:
                lq.lq_linear_ex(l["struct"], x, 1, ys[l["name"]], algo, ws)
                return
            except lq.LQError:
                l.setdefault("algo_ok", {})[algo] = False
        lq.lq_linear(l["struct"], x, 1, ys[l["name"]], ws)

    # gate and up read the same x: one lq_linear_multi call (one preparation
    # and one product launch for both) unless another algorithm is forced
    grouped = args.gate_up == "multi" and algo is None
    ys_gu = [ys["gate"], ys["up"]]

    def step(i):
        gate, up, down = layers[i % n_sets]
        if grouped:
            lq.lq_linear_multi([gate["struct"], up["struct"]], x_in["gate"], 1, ys_gu, ws)
        else:
            call(gate, x_in["gate"])
            call(up, x_in["gate"])
        call(down, x_in["down"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    per_step = 2 if grouped else 3              # product launches per step
    n_launch = per_step * K
    starts, stops = ev.create(n_launch), ev.create(n_launch)
    if args.eager:
        lq.lq_profile_events(starts, stops)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            step(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                step(i)
        g.replay()                      # first replay uploads the graph (untimed)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    lq.lq_profile_events([], [])
    timing = ("hipEvents recorded by the dispatch of every sign-product launch inside the "
              "timed region")
    try:
        durs = [ev.elapsed_ms(a, b) for a, b in zip(starts, stops)]
    except RuntimeError:
        # Fallback: the same K steps launched eagerly right after the timed
        # region, each sign-product kernel bracketed by events.
        timing = ("hipEvents recorded by the dispatch of every sign-product launch of an eager "
                  "replay of the K steps")
        lq.lq_profile_events(starts, stops)
        for i in range(K):
            step(i)
        torch.cuda.synchronize()
        lq.lq_profile_events([], [])
        durs = [ev.elapsed_ms(a, b) for a, b in zip(starts, stops)]
    ev.destroy(starts)
    ev.destroy(stops)

    ms_step = (t1 - t0) * 1e3 / K
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    kern_ms = sum(durs) / len(durs)
    # N*L/8 of the layers a product launch reads, averaged over the launches
    bytes_per_launch = step_bytes / per_step
    achieved = bytes_per_launch / (kern_ms * 1e-3) / 1e9
    per_proj = {}
    names = ["gate+up", "down"] if grouped else [p for p, _ in specs]
    for j, pname in enumerate(names):
        d = durs[j::per_step]
        per_proj[pname] = round(sum(d) / len(d) * 1e3, 3)
    return dict(ms_step=ms_step, gbs=gbs, kern_ms=kern_ms, achieved=achieved,
                step_bytes=step_bytes, bytes_per_launch=bytes_per_launch, per_proj_us=per_proj,
                n_sets=n_sets, timing=timing, grouped=grouped)


def build_prefill_case(torch, lq, algo=None):
    """The 2048-token prefill layer (8192 -> 8192, d = 3, D = 8) on the GPU."""
    from workloads import WORKLOADS
    s = WORKLOADS["prefill"].layers[0]
    B = 2048
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    nbytes = lq.lq_packed_size(s.N, s.K, s.d, s.D)
    packed = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev, generator=gen)
    M = (torch.randn(s.d, s.D, device=dev, generator=gen) / s.D ** 0.5).contiguous()
    r = torch.rand(s.N, device=dev, generator=gen) + 0.5
    c = torch.rand(s.K, device=dev, generator=gen) * 0.4 + 0.8
    st = lq.layer_struct(s.N, s.K, s.d, s.D, s.hb, packed, M, c, r)
    x = torch.randn(B, s.K, device=dev, generator=gen).to(torch.bfloat16)
    y = torch.empty(B, s.N, dtype=torch.bfloat16, device=dev)
    a = lq.LQ_ALGO_AUTO if algo is None else algo
    ws = torch.zeros(lq.lq_linear_workspace_size_ex(st, B, torch.bfloat16, a), dtype=torch.uint8,
                     device=dev)
    return dict(spec=s, B=B, packed=packed, M=M, r=r, c=c, struct=st, x=x, y=y, ws=ws)


PREFILL_ALGOS = {"auto": None, "large": "LQ_ALGO_MFMA_LARGE", "wspace": "LQ_ALGO_WSPACE"}


def run_prefill(args, torch, lq, ev, steps=10):
    name = PREFILL_ALGOS[args.prefill_algo]
    algo = None if name is None else getattr(lq, name)
    pf = build_prefill_case(torch, lq, algo)
    s, B, st, x, y, ws = pf["spec"], pf["B"], pf["struct"], pf["x"], pf["y"], pf["ws"]

    def call():
        if algo is None:
            lq.lq_linear(st, x, B, y, ws)
        else:
            lq.lq_linear_ex(st, x, B, y, algo, ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    starts, stops = ev.create(steps), ev.create(steps)
    lq.lq_profile_events(starts, stops)
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lq.lq_profile_events([], [])
    durs = [ev.elapsed_ms(a, b) for a, b in zip(starts, stops)]
    ev.destroy(starts)
    ev.destroy(stops)
    flops = 2.0 * B * s.N * s.L
    dense = 2.0 * B * s.N * s.Kpad
    kern_ms = sum(durs) / len(durs)
    ms = (t1 - t0) * 1e3 / steps
    # The timed kernel and its algorithmic flops: the lifted product does
    # 2 B N L, the W-space one 2 B N K' (the dense-equivalent product).
    ws_path = lq.lq_linear_algo(st, B, torch.bfloat16,
                                lq.LQ_ALGO_AUTO if algo is None else algo) == lq.LQ_ALGO_WSPACE
    kflops = dense if ws_path else flops
    return dict(workload=f"prefill K={s.K} N={s.N} d={s.d} D={s.D} B={B}",
                tflops_linear=flops / (ms * 1e-3) / 1e12, ms_linear=ms,
                kernel_ms=kern_ms, kernel_tflops=kflops / (kern_ms * 1e-3) / 1e12,
                kernel=WSPACE_KERNEL if ws_path else LARGE_KERNEL,
                kernel_flops=kflops, lifted_flops=flops, dense_equiv_flops=dense)


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
    for d, D, n in ((10, 24, 1), (3, 8, 20000)):
        M = ref.orthonormal_rows(rng.standard_normal((D, D)), d)
        w = rng.standard_normal((n, d))
        t0 = time.perf_counter()
        ref.encode_nn(w, M)
        dt = time.perf_counter() - t0
        res.append(dict(d=d, D=D, blocks=n, seconds=round(dt, 3), blocks_per_s=round(n / dt, 3)))
    return res


def cpu_threads():
    """Threads the oracle's numpy uses (its BLAS pool)."""
    try:
        import numpy  # noqa: F401  (loads the BLAS pool threadpoolctl inspects)
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def cpu_baseline(budget_s):
    """The oracle as it stands, on rows sampled from the same three layers."""
    import numpy as np
    from oracle import liftquant_ref as ref
    from workloads import WORKLOADS, make_layer
    threads = cpu_threads()
    wl = WORKLOADS["llama3_8b_mlp"]
    gate, down = wl.layers
    inputs = {s.name: make_layer(s, wl, B_max=1) for s in (gate, down)}

    def run(rows):
        nbytes = 0
        t = 0.0
        for s in (gate, gate, down):
            li = inputs[s.name]
            idx = np.arange(rows)
            signs = li.signs_rows(idx)
            t0 = time.perf_counter()
            ref.linear(li.x(1), li.c, s.hb, li.M, signs, li.row_scale[idx])
            t += time.perf_counter() - t0
            nbytes += rows * s.L // 8
        return nbytes, t

    rows = 64
    nb, t = run(rows)
    reps = 1
    if t < budget_s / 4:
        rows = int(min(4096, max(64, rows * budget_s / max(t, 1e-3))) // 16 * 16)
        nb, t = run(rows)
        reps = max(1, int(budget_s / max(t, 1e-3)))        # repeat the sample up to the budget
        for _ in range(reps - 1):
            nb2, t2 = run(rows)
            nb += nb2
            t += t2
    return dict(value=round(nb / t / 1e9, 6), unit="GB/s", cores=threads, kind="oracle",
                sample=f"oracle linear() on the first {rows} rows of each of gate, up and down "
                       f"(B=1, d=10, D=24), {reps} times: {nb} packed bytes in {t:.2f} s")


def main():
    args = parse_args()
    if args.summarize_stats:
        print(summarize_stats(args.summarize_stats, args.profiled_steps))
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
        pmc_workload(torch, lq)
        return
    ev = HipEvents()
    dec = run_decode(args, torch, lq, ev)
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
            "workload": "Llama-3-8B MLP decode at 2.4 bit (d=10, D=24): gate and up "
                        "K=4096->N=14336, down K=14336->N=4096, batch 1, bf16 activations, "
                        "Hadamard block 1024; one step = the three projections"
                        + (" (gate and up, which read the same x, in one lq_linear_multi "
                           "call; down in one lq_linear call)" if dec["grouped"]
                           else " as three lq_linear calls"),
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
            "traffic": traffic_from_summary(),
            "avg_launch_us": round(dec["kern_ms"] * 1e3, 3),
            "per_layer_avg_us": dec["per_proj_us"],
            "timing": dec["timing"],
            "algorithmic_bytes_per_launch": dec["bytes_per_launch"],
        },
    }
    if not args.no_prefill:
        pf = run_prefill(args, torch, lq, ev)
        out["prefill"] = {
            "metric": "TFLOP/s (batch 2048), lifted flops 2*B*N*L",
            "workload": pf["workload"],
            "algo": args.prefill_algo,
            "kernel": pf["kernel"],
            "kernel_flops_per_launch": pf["kernel_flops"],
            "value": round(pf["tflops_linear"], 2),
            "unit": "TFLOP/s",
            "ms_per_linear": round(pf["ms_linear"], 4),
            "roofline": {"bound": "mfma", "achieved": round(pf["kernel_tflops"], 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(pf["kernel_tflops"] / BF16_PEAK_TFLOPS, 4),
                         "avg_launch_us": round(pf["kernel_ms"] * 1e3, 2),
                         "traffic": traffic_from_summary(pf["kernel"])},
        }
    if not args.no_encode:
        enc, train = run_encode(torch, lq)
        big = enc[0]
        out["encode"] = {
            "metric": "blocks/s encoded (exhaustive nearest-neighbour search, Eq. (1) inner minimisation)",
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
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
