#!/usr/bin/env python3
"""Benchmark of the sparse MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config mixtral_prefill] [--only]

A step is one whole layer forward (router, gating, grouping, expert FFNs,
combine) over one resident batch of synthetic inputs.  Prints one JSON line:
throughput in tokens/s over exactly K timed steps, the roofline of the dominant
kernel (the grouped gate/up projection; for decode-sized batches the bytes of
the distinct experts it reads) from HIP events recorded around that kernel on
the layer's stream during the timed steps, per-stage device times from a second,
untimed pass with an event at every stage boundary, and the CPU oracle timed on
a bounded sample of the same layer.  The headline is the Mixtral-shaped prefill
layer; the default run then measures the decode batch, the DeepSeek-V3 shape and
the skewed layer with capacity the same way, under "configs" (--only skips them).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import re
import sys
import statistics
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + % bf16 MFMA peak (prefill); % HBM GB/s (decode)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded (same soname)."""

    # timing-only events: no system-scope fence (cache writeback and invalidate) when recorded
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self) -> int:
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def record(self, ev: int, stream: int) -> None:
        rc = self.hip.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def destroy(self, ev: int) -> None:
        self.hip.hipEventDestroy(ev)


def algorithmic_counts(cfg, counts, weight_bytes: float = None):
    """Flops and bytes of one layer call by the definitions (not the implementation).

    flops: router 2*T*d*N; per kept (token, expert) slot 2*nm*d*d_ff (nm = 3 SwiGLU, 2 ReLU);
    the shared expert adds 2*nm*d*d_ff per token.  bytes: the weights of the distinct experts
    touched (plus the shared expert), the router weights, x and y.
    ffn_in: the gate/up (or W1) projection alone, per launch."""
    import numpy as np
    nm = 3 if cfg.ffn == "swiglu" else 2
    nm_in = nm - 1
    eb = cfg.elem_bytes
    wb = eb if weight_bytes is None else weight_bytes    # bytes per expert weight
    kept = int(np.sum(counts))
    touched = int(np.sum(counts > 0))
    rows_sh = cfg.T if cfg.has_shared else 0
    flops = 2.0 * cfg.T * cfg.d * cfg.N + 2.0 * nm * cfg.d * cfg.d_ff * (kept + rows_sh)
    w_expert = nm * cfg.d * cfg.d_ff * wb
    bytes_ = (touched + (1 if cfg.has_shared else 0)) * w_expert + cfg.N * cfg.d * eb + 2 * cfg.T * cfg.d * eb
    ffn_in_flops = 2.0 * nm_in * cfg.d * cfg.d_ff * (kept + rows_sh)
    ffn_in_bytes = ((touched + (1 if cfg.has_shared else 0)) * nm_in * cfg.d * cfg.d_ff * wb
                    + cfg.T * cfg.d * eb + (kept + rows_sh) * cfg.d_ff * eb)
    return dict(flops=flops, bytes=bytes_, touched=touched, kept=kept,
                ffn_in_flops=ffn_in_flops, ffn_in_bytes=ffn_in_bytes)


FFN_SOURCE = os.path.join(ROOT, "mixture_experts_layer_48_amd", "csrc", "ffn.hip")
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    """Short hash of the grouped-GEMM source: counter figures are only reused while it is unchanged."""
    import hashlib
    with open(FFN_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch of the in-projection kernel from the committed counter summary
    (profiles/ffn_in_<workload>_traffic.txt), or None if there is none or the kernel source
    changed since the counters were taken."""
    path = os.path.join(TRAFFIC_DIR, f"ffn_in_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for ln in f:
            if "=" in ln and not ln.startswith("#"):
                k, v = ln.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def summarize_pmc(fetch_dir: str, write_dir: str, copy_bytes: int, workload: str, command: str) -> str:
    """Text summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch):
    each counter is scaled by what it reads for a plain copy of copy_bytes."""
    import csv
    import glob
    import statistics

    def per_kernel(d, counter):
        out = {}
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(fn)):
                if r["Counter_Name"] == counter:
                    out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")

    def pick_in_projection(d):
        # the gate/up (or W1) stage, one launch of each of its kernels per layer call: the tiled
        # GEMM, the weight-streaming kernel, or both (the tiled GEMM beside a weight stream for
        # the small experts), SwiGLU or ReLU mode; the stage's bytes are their sum
        ks = sorted(k for k in d if re.search(r"ffn_(bf16|skinny)_kernel<[01][,>]", k))
        if not ks:
            return float("nan"), "none"
        return sum(statistics.mean(d[k]) for k in ks), " + ".join(ks)

    def largest(d, key):
        # the calibration copy is by far the largest copy dispatch of the run
        vals = [v for k, vs in d.items() if key in k for v in vs]
        return max(vals) if vals else float("nan")

    copy_f, copy_w = largest(fetch, "copy"), largest(write, "copy")
    f_scale = copy_bytes / (copy_f * 1024.0)
    w_scale = copy_bytes / (copy_w * 1024.0)
    (ffn_f, kname), (ffn_w, _) = pick_in_projection(fetch), pick_in_projection(write)
    hbm = ffn_f * 1024.0 * f_scale + ffn_w * 1024.0 * w_scale
    lines = [
        f"# HBM traffic of the grouped in-projection stage ({kname}), {workload}",
        f"# command: {command}",
        "# FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by bytes/KiB it reads",
        f"# for a plain device copy of {copy_bytes} bytes in the same run.",
        f"workload = {workload}",
        f"copy_bytes = {copy_bytes}",
        f"copy_fetch_kib = {copy_f:.1f}",
        f"copy_write_kib = {copy_w:.1f}",
        f"fetch_scale = {f_scale:.4f}",
        f"write_scale = {w_scale:.4f}",
        f"ffn_in_fetch_kib_per_dispatch = {ffn_f:.1f}",
        f"ffn_in_write_kib_per_dispatch = {ffn_w:.1f}",
        f"hbm_bytes_per_launch = {hbm:.0f}",
        f"kernel_source_sha256_16 = {kernel_source_hash()}",
    ]
    for name, vals in sorted(fetch.items()):
        lines.append(f"# fetch_kib {statistics.mean(vals):14.1f}  {name[:90]}")
    for name, vals in sorted(write.items()):
        lines.append(f"# write_kib {statistics.mean(vals):14.1f}  {name[:90]}")
    return "\n".join(lines) + "\n"


def summarize_counters(pmc_dir: str, workload: str, command: str) -> str:
    """Text summary of one rocprofv3 --pmc run: every counter's mean per dispatch for each kernel,
    and for the MFMA kernels the matrix-core utilisation SQ_VALU_MFMA_BUSY_CYCLES /
    (GRBM_GUI_ACTIVE x SIMDs), the shader clock GRBM_GUI_ACTIVE / duration, and the share of wave
    cycles spent waiting (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES) and waiting on LDS."""
    import csv
    import glob
    import statistics
    vals = {}
    durs = {}
    for fn in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(fn)):
            k = r["Kernel_Name"]
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    for fn in glob.glob(os.path.join(pmc_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(fn)):
            durs.setdefault(r["Kernel_Name"], []).append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    simds, xcds = 256 * 4, 8
    lines = [f"# rocprofv3 counters per dispatch (mean over dispatches), {workload}",
             f"# command: {command}",
             "# Values are summed over the counter's instances (GRBM_GUI_ACTIVE over the 8 XCDs, so active cycles",
             "# = GRBM_GUI_ACTIVE / 8).  mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (active cycles * 1024 SIMDs), as",
             "# rocprofv3's MfmaUtil; clock = active cycles / kernel duration; wait = SQ_WAIT_INST_ANY /",
             "# SQ_WAVE_CYCLES; lds_wait = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES"]
    for k in sorted(vals, key=lambda k: -statistics.mean(durs.get(k, [0.0]))):
        c = {n: statistics.mean(v) for n, v in vals[k].items()}
        d = statistics.mean(durs[k]) if k in durs else float("nan")
        lines.append(f"kernel {k[:110]}")
        lines.append(f"  dispatches {len(next(iter(vals[k].values())))}, mean duration {d / 1e3:.1f} us")
        for n in sorted(c):
            lines.append(f"  {n} = {c[n]:.6g}")
        g = c.get("GRBM_GUI_ACTIVE", 0.0) / xcds
        if g and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            lines.append(f"  mfma_util = {c['SQ_VALU_MFMA_BUSY_CYCLES'] / (g * simds):.4f}")
        if g and d == d and d > 0:
            lines.append(f"  clock_ghz = {g / d:.3f}")
        if c.get("SQ_WAVE_CYCLES"):
            if "SQ_WAIT_INST_ANY" in c:
                lines.append(f"  wait = {c['SQ_WAIT_INST_ANY'] / c['SQ_WAVE_CYCLES']:.4f}")
            if "SQ_WAIT_INST_LDS" in c:
                lines.append(f"  lds_wait = {c['SQ_WAIT_INST_LDS'] / c['SQ_WAVE_CYCLES']:.4f}")
    return "\n".join(lines) + "\n"


def summarize_stats(stats_csv: str, workload: str, command: str, note: str = "") -> str:
    """Text table of a rocprofv3 --kernel-trace --stats run (its kernel_stats.csv): calls, mean,
    min and max duration and share of the total per kernel, longest total first."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel statistics, {workload}", f"# command: {command}"]
    if note:
        lines.append(f"# {note}")
    lines.append(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel")
    for r in rows:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} {float(r['MinNs']) / 1e3:10.1f} "
                     f"{float(r['MaxNs']) / 1e3:10.1f} {float(r['Percentage']):6.2f}  {r['Name'][:100]}")
    return "\n".join(lines) + "\n"


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, sample_tokens: int, one_core_tokens: int):
    """The plain C++ float64 oracle (oracle/moe_oracle.cpp), as it stands, on the same layer and
    weights (host copies of the device tensors, bf16 read in place): routing of every token, then
    the expert FFNs and combine of the first `sample_tokens` tokens on all host cores this process
    may use, and of the first `one_core_tokens` on one core.  tokens/s counts the sampled tokens."""
    import oracle.cpp as OC
    host = {k: (None if v is None else v.cpu()) for k, v in inp.items()}
    shared = (host["sh_gate"], host["sh_up"], host["sh_down"]) if cfg.has_shared else None
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)

    def run(threads, S):
        OC.set_threads(threads)
        t0 = time.perf_counter()
        OC.forward(host["x"], host["w_router"], host["w_up"], host["w_down"], cfg.k, cfg.ffn, cfg.gating,
                   w_gate=host["w_gate"], logit_bias=host["logit_bias"], capacity_factor=cfg.capacity_factor,
                   shared=shared, tokens=list(range(S)))
        return time.perf_counter() - t0

    S = min(sample_tokens, cfg.T)
    S1 = min(one_core_tokens, cfg.T)
    dt = run(cores, S)
    dt1 = run(1, S1)
    OC.set_threads(cores)
    return {"value": S / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"C++ float64 oracle: routing of all {cfg.T} tokens, expert FFNs and combine of the first "
                      f"{S} tokens of the same layer and weights on {cores} threads, {dt:.1f} s",
            "one_core": {"value": S1 / dt1, "unit": "tokens/s", "cores": 1,
                         "sample": f"first {S1} tokens on one thread, {dt1:.1f} s"},
            "cpu_model": cpu_model(), "nproc": os.cpu_count()}


def ep_layout_timing(M, cfg, desc, inp, routing, hip, steps: int, G: int = 8):
    """Device time of the expert-parallel layouts for one rank of a G-way placement (contiguous
    expert blocks; this batch's routing as every source's): send layout + packing of the rows,
    receive layout of rank 0 (G copies of the counts), and the unpack of its expert outputs.
    Outside the layer step; bytes are the rows moved (read + write)."""
    import torch
    G = min(G, cfg.N)
    owner = [e * G // cfg.N for e in range(cfg.N)]
    T, k, N, d = cfg.T, cfg.k, cfg.N, cfg.d
    i32 = dict(dtype=torch.int32, device="cuda")
    outs = [torch.empty(n, **i32) for n in (N, N + 1, G, G + 1, T * k, T * k)]
    send_buf = torch.empty((T * k, d), dtype=cfg.torch_dtype, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = hip.create(), hip.create()
        hip.record(a, stream)
        for _ in range(steps):
            fn()
        hip.record(b, stream)
        torch.cuda.synchronize()
        us = hip.elapsed_ms(a, b) * 1e3 / steps
        hip.destroy(a)
        hip.destroy(b)
        return us

    disp = lambda: M.moe_ep_dispatch(desc, routing["idx"], owner, G, *outs, inp["x"], send_buf)  # noqa: E731
    dispatch_us = timed(disp)
    layout_us = timed(lambda: M.moe_ep_dispatch(desc, routing["idx"], owner, G, *outs))
    kept = int(outs[3][G].item())
    rc = outs[0].repeat(G).view(G, N).contiguous()
    R = int(rc[:, [e for e in range(N) if owner[e] == 0]].sum().item())
    nl = sum(1 for e in range(N) if owner[e] == 0)
    ro, lo = torch.empty(G + 1, **i32), torch.empty(nl + 1, **i32)
    rp, ri = torch.empty(max(R, 1), **i32), torch.empty(max(R, 1), **i32)
    recv_us = timed(lambda: M.moe_ep_receive_layout(N, G, owner, 0, rc, R, ro, lo, rp, ri))
    yg = torch.empty((max(R, 1), d), dtype=torch.float32, device="cuda")
    ret = torch.empty_like(yg)
    unpack_us = timed(lambda: M.moe_ep_unpack(G, R, d * 4, ro, ri, yg, ret))
    eb = cfg.elem_bytes
    return {"G": G, "owner": "contiguous", "rows_sent": kept, "rows_received_rank0": R,
            "dispatch_and_pack_us": dispatch_us, "dispatch_layout_us": layout_us,
            "pack_gbs": 2 * kept * d * eb / max(dispatch_us - layout_us, 1e-3) / 1e3,
            "receive_layout_us": recv_us, "unpack_us": unpack_us,
            "unpack_gbs": 2 * R * d * 4 / max(unpack_us, 1e-3) / 1e3}


def measure(M, W, hip, cfg, steps: int, warmup: int, weights: str = "native", extras: bool = True):
    """Time `steps` layer forwards of one configuration (after `warmup` untimed ones) and derive
    its throughput, roofline fractions and per-stage device times.  Returns (result dict,
    inputs, routing) -- the inputs stay resident for the CPU baseline."""
    import torch

    inp = W.make_inputs(cfg, "cuda")
    desc = M.make_desc(cfg.T, cfg.d, cfg.N, cfg.k, cfg.d_ff, cfg.dtype, cfg.ffn, cfg.gating,
                       cfg.capacity_factor, cfg.has_shared)
    qweights = M.quantize_weights_q4(inp) if weights == "int4" else None
    layer = M.MoELayer(desc, inp, qweights=qweights)
    routing = layer.routing_buffers()
    y = torch.empty((cfg.T, cfg.d), dtype=cfg.torch_dtype, device="cuda")
    nev = M.MOE_NUM_STAGES + 1

    for _ in range(warmup):
        layer.forward(inp["x"], y=y, out_routing=routing)
    # Timed region: the only events recorded are the two around the dominant kernel (the
    # in-projection, stage 3), for its live duration.
    in_ev = [(hip.create(), hip.create()) for _ in range(steps)]
    only_in = [[None] * 3 + [a, b] + [None] * (nev - 5) for a, b in in_ev]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        layer.forward(inp["x"], y=y, out_routing=routing, events=only_in[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1000.0 / steps
    ffn_in_ms = sum(hip.elapsed_ms(a, b) for a, b in in_ev) / steps
    # Stage breakdown: a second pass with an event at every stage boundary (not timed; the
    # events themselves add a few microseconds per call).
    events = [[hip.create() for _ in range(nev)] for _ in range(steps)]
    for i in range(steps):
        layer.forward(inp["x"], y=y, out_routing=routing, events=events[i])
    torch.cuda.synchronize()
    stage_ms = [sum(hip.elapsed_ms(ev[s], ev[s + 1]) for ev in events) / steps
                for s in range(M.MOE_NUM_STAGES)]
    step_dev = sorted(hip.elapsed_ms(ev[0], ev[-1]) for ev in events)
    step_dev_ms = sum(step_dev) / steps
    for ev in events + [list(p) for p in in_ev]:
        for e in ev:
            hip.destroy(e)

    counts = routing["counts"].cpu().numpy()
    alg = algorithmic_counts(cfg, counts, weight_bytes=0.5 + 4.0 / 128 if qweights is not None else None)
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    ai = alg["ffn_in_flops"] / alg["ffn_in_bytes"]
    if cfg.dtype == "f32":
        roof = {"bound": "alu", "achieved": alg["ffn_in_flops"] / (ffn_in_ms * 1e-3) / 1e12,
                "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s"}
    elif ai >= ridge:
        roof = {"bound": "mfma", "achieved": alg["ffn_in_flops"] / (ffn_in_ms * 1e-3) / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": alg["ffn_in_bytes"] / (ffn_in_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_from_profile(cfg.name) if qweights is None else None
    roof["kernel"] = ("ffn_in (grouped gate/up projection)" if qweights is None
                      else "ffn_in (gate/up projection, int4 weight stream)")
    roof["ms_per_launch"] = ffn_in_ms
    res = {
        "workload": cfg.name,
        "ms_per_step": ms_per_step,
        "tokens_per_s": cfg.T * steps / (t1 - t0),
        "tflops": alg["flops"] / (ms_per_step * 1e-3) / 1e12,
        "mfma_frac": alg["flops"] / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "gbs_distinct_experts": alg["bytes"] / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac": alg["bytes"] / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "experts_touched": alg["touched"], "device_ms_per_step": step_dev_ms,
        "device_ms_median": statistics.median(step_dev), "device_ms_min": step_dev[0],
        # the time the binding roofline allows, max(flops / MFMA peak, bytes / HBM peak), over the
        # measured time
        "roofline_time_frac": max(alg["flops"] / (PEAK_BF16_TFLOPS * 1e12),
                                  alg["bytes"] / (PEAK_HBM_GBS * 1e9)) / (ms_per_step * 1e-3),
        "stages_ms": dict(zip(M.STAGE_NAMES, stage_ms)),
        "roofline": roof,
        "config": {"T": cfg.T, "d": cfg.d, "N": cfg.N, "k": cfg.k, "d_ff": cfg.d_ff, "ffn": cfg.ffn,
                   "gating": cfg.gating, "capacity_factor": cfg.capacity_factor,
                   "shared_expert": cfg.has_shared, "expert_weights": weights},
    }
    if extras:
        # Routing statistics of the same routing (outside the layer step): device time per call
        # between two events around `steps` back-to-back calls.
        st_out = None
        ev_a, ev_b = hip.create(), hip.create()
        layer.routing_stats(routing)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream().cuda_stream
        hip.record(ev_a, stream)
        for _ in range(steps):
            st_out = layer.routing_stats(routing)
        hip.record(ev_b, stream)
        torch.cuda.synchronize()
        stats_us = hip.elapsed_ms(ev_a, ev_b) * 1e3 / steps
        hip.destroy(ev_a)
        hip.destroy(ev_b)
        st_vals = st_out["stats"].cpu().numpy().tolist()
        # algorithmic bytes: logits, indices and counts read once, the statistics written
        st_bytes = cfg.T * cfg.N * 4 + cfg.T * cfg.k * 4 + cfg.N * 4 + M.MOE_NUM_STATS * 8 + 3 * 4
        res["routing_stats"] = {"us_per_call": stats_us, "gbs": st_bytes / (stats_us * 1e-6) / 1e9,
                                "values": dict(zip(M.STAT_NAMES, st_vals)),
                                "top3": st_out["top3"].cpu().numpy().tolist()}
        res["ep_layout"] = ep_layout_timing(M, cfg, desc, inp, routing, hip, steps)
    del layer, y, qweights
    return res, inp, routing


# The other layer shapes of the metric, measured after the headline one in the default run: the
# decode batch (scored on HBM bandwidth of the distinct experts it reads), the DeepSeek-V3 shape and
# the skewed layer with capacity (scored on MFMA and on HBM).
SECONDARY = ("mixtral_decode", "deepseek_v3", "skewed_capacity")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral_prefill")
    ap.add_argument("--only", action="store_true",
                    help="measure --config alone (without the other layer shapes of the default run)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--weights", choices=("native", "int4"), default="native",
                    help="expert weights: the layer dtype, or int4 codes + fp32 group scales (0.53125 B each)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_MIB", "COMMAND"),
                    help="print the traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("PMC_DIR", "COMMAND"),
                    help="print the per-kernel counter summary of one rocprofv3 --pmc run and exit")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("STATS_CSV", "COMMAND", "NOTE"),
                    help="print the kernel table of one rocprofv3 --kernel-trace --stats run and exit")
    args = ap.parse_args(argv)
    if args.summarize_pmc:
        fd, wd, mib, cmd = args.summarize_pmc
        sys.stdout.write(summarize_pmc(fd, wd, int(mib) << 20, args.config, cmd))
        return 0
    if args.summarize_counters:
        d, cmd = args.summarize_counters
        sys.stdout.write(summarize_counters(d, args.config, cmd))
        return 0
    if args.summarize_stats:
        f, cmd, note = args.summarize_stats
        sys.stdout.write(summarize_stats(f, args.config, cmd, note))
        return 0
    if args.gpus != 1:
        print(f"bench.py: the library runs one GPU's share of the layer; --gpus {args.gpus} is not "
              f"supported (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import mixture_experts_layer_48_amd as M
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    cfg = W.CONFIGS[args.config]
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    hip = HipEvents()
    res, inp, _ = measure(M, W, hip, cfg, args.steps, args.warmup, args.weights)
    print(f"# {cfg.name}: {res['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
    out = {
        "metric": METRIC,
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype if args.weights == "native" else "bf16 activations, int4 expert weights",
        "data": "synthetic (seeded Gaussian inputs and weights of the layer's shapes)",
        "config": dict(workload=cfg.name, **res["config"]),
        "layer": {k: res[k] for k in ("tflops", "mfma_frac", "gbs_distinct_experts", "hbm_frac",
                                      "experts_touched", "device_ms_per_step", "device_ms_median",
                                      "device_ms_min", "roofline_time_frac")},
        "stages_ms": res["stages_ms"],
        "routing_stats": res["routing_stats"],
        "ep_layout": res["ep_layout"],
        "roofline": res["roofline"],
        "cpu_baseline": None,
        "configs": {},
    }
    if not args.no_cpu_baseline:
        # samples sized for roughly 10-20 s of oracle work each, on 16 host cores and on one
        default_sample = {"tiny_fp32": 128, "mixtral_prefill": 768, "mixtral_decode": 16,
                          "deepseek_v3": 256, "skewed_capacity": 2048}.get(cfg.name, 64)
        S = args.cpu_sample_tokens or default_sample
        out["cpu_baseline"] = cpu_baseline(cfg, inp, S, max(1, S // 16))
    del inp
    torch.cuda.empty_cache()
    if not args.only and args.weights == "native" and cfg.name == "mixtral_prefill":
        for name in SECONDARY:
            r2, inp2, _ = measure(M, W, hip, W.CONFIGS[name], args.steps, args.warmup, extras=False)
            print(f"# {name}: {r2['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
            r2.pop("workload")
            out["configs"][name] = r2
            del inp2
            torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
