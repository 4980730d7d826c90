"""Benchmark of the attention forward hot path on one MI355X.

One step = one pass of the whole hot path over the long-context GQA workload
(batch 1, 32 query heads / 8 kv heads, seq 32768, head_dim 128, causal GQA,
synthetic fp16 inputs already resident in HBM; the largest of the five
workloads, 8.8 TFLOP per attention call):
    attn_quantize_k        (K channel mean, smoothing, per-block INT8 K)
    attn_fwd_int8_fused_q  (per-block INT8 Q in the kernel, INT8 QK^T,
                            online softmax, FP16 P.V)
    attn_fwd_fp16          (the exact FP16 FlashAttention-style baseline)

Printed: ONE JSON line.  `value` is the INT8 (SageAttention-form) path's
attention throughput, quantisation included: FLOP / (t_quantize_k +
t_fwd_int8_fused_q), with FLOP = 4*B*Hq*S^2*D/2 (causal) and the per-call
times taken with HIP events on the launch stream inside the timed steps.  The
FP16 path and the INT8 forward alone are reported beside it, each as TFLOPS and
as a fraction of MI355X's published dense MFMA peak (fp16 2.5 PFLOP/s, int8
5.0 POP/s, and for the INT8 path the harmonic blend of the two, its QK^T half
running at the INT8 rate and its P.V half at the FP16 rate).

`paths.configs` times the same three calls on each of the five workloads (the
tiny MHA, the 8192-token LLM prefill, the video-diffusion MHA, the long GQA
and the batched MQA) in the same process.  Outside the timed steps the line
also carries, on the headline workload, the two-call INT8 path
(attn_quantize_qk + attn_fwd_int8), the FP8 alternative and the 8-bit P.V
ablation; the KV-cache decode kernels (batch 16, one query over an 8192-token
cache) as GB/s against HBM; and the tile-masked forwards under the APB layout
of the 8192-token prefill (1024 anchor, 2048 passing, 5120 local tokens).

`roofline` describes the dominant kernel of the step; `mfma_loop` gives, as
context for its published peak, the rate a dense MFMA loop sustains on this
device (libattn_probe.so), and `hbm_read` the bandwidth a plain streaming read
of a 4 GiB buffer reaches, context for the 8 TB/s of the HBM-bound kernels;
`cpu_baseline` times the CPU oracle (fp64, plain
loops) on a bounded, seeded sample of the headline workload's query rows, on
this machine's host cores, and `parity_sample` compares the GPU outputs with
it on those rows.

Each timed section is preceded by untimed calls for CLOCK_WARM_MS of busy
time (the clocks ramp up after the GPU idled while the CPU drew the inputs),
then the W warm-up steps, then exactly K timed steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--no-configs] [--no-cpu] [--clock-warm-ms MS] [--only-step]
       python bench.py --decode-only [--decode-reps N]      (profiling)
       python bench.py --copy-calibration BYTES             (HBM counter scale)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"fp16": 2500.0, "int8": 5000.0}
PEAK_BLEND = 2.0 / (1.0 / PEAK_TFLOPS["int8"] + 1.0 / PEAK_TFLOPS["fp16"])
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "long_gqa"
APB_WORKLOAD = "llm_prefill_gqa"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload block paths.configs")
    ap.add_argument("--only-step", action="store_true",
                    help="only the warm-up and timed steps of the workload (for profiling): no "
                         "other paths, configs, decode, APB, MFMA loop or CPU baseline")
    ap.add_argument("--config-steps", type=int, default=10,
                    help="timed steps per workload in paths.configs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (HBM counter calibration)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the KV-cache decode measurement (one JSON line; for profiling)")
    ap.add_argument("--decode-reps", type=int, default=20, help="timed calls per decode kernel")
    ap.add_argument("--clock-warm-ms", type=float, default=CLOCK_WARM_MS,
                    help="untimed busy time before each timed section")
    return ap.parse_args()


def counters_for(kernel_tag: str, workload: str):
    """HBM traffic of a kernel from the committed rocprofv3 counter summary, or
    None when the summary is missing or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    # the kernel is its source file plus the headers it includes, hashed in the listed order
    h = hashlib.sha256()
    for name in vals.get("source", "attn_fwd.hip").split():
        h.update(open(os.path.join(ROOT, "bit_quantized_exact_amd", "csrc", name), "rb").read())
    sha = h.hexdigest()
    if vals.get("source_sha256") != sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# The chip's clocks ramp up over tens to hundreds of milliseconds after an
# idle spell (the inputs are drawn on the CPU while the GPU idles); measured,
# the first path timed after one ran up to 15 % slow with a few warm-up calls.
# Each timed section is therefore preceded by this much busy time.
CLOCK_WARM_MS = 300.0


def clock_warm(fn, min_ms=None, batch=4):
    """Call fn (batches of `batch` calls) until at least min_ms (default
    CLOCK_WARM_MS) of wall time has passed with the GPU busy; returns the
    number of calls (untimed)."""
    import torch

    if min_ms is None:
        min_ms = CLOCK_WARM_MS

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(batch):
            fn()
        n += batch
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            return n


def algorithmic_bytes(w):
    """Bytes each call must move (every tensor read or written once)."""
    B, Hq, Hkv, S, D = w.batch, w.heads_q, w.heads_kv, w.seq, w.head_dim
    nq, nk = B * Hq * S * D, B * Hkv * S * D
    kscales = 4 * B * Hkv * math.ceil(S / 64)
    return {
        "fwd_fp16": 2 * (2 * nq + 2 * nk),                       # Q, K, V read; O written
        "fwd_int8": 2 * nq + nk + 2 * nk + 2 * nq + kscales,     # fp16 Q, int8 K, fp16 V, O, K scales
        "quantize_k": 2 * 2 * nk + nk + kscales,                 # K read twice, int8 K and scales written
    }


def time_core(w, steps, warmup, tensors=None):
    """Times the step's three calls (attn_quantize_k, attn_fwd_int8_fused_q,
    attn_fwd_fp16) on workload w with HIP events on the launch stream: a clock
    warm-up, `warmup` untimed steps, then `steps` timed ones.  Returns the mean
    per-call milliseconds, the wall time of the timed steps and the device
    tensors (inputs and outputs)."""
    import torch

    import bit_quantized_exact_amd as A
    from bit_quantized_exact_amd.inputs import make_qkv

    if tensors is None:
        q, k, v = make_qkv(w)
        dev = torch.device("cuda:0")
        qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
        del q, k, v
    else:
        qd, kd, vd = tensors
    # outputs and workspace allocated once: the timed steps only launch kernels
    kz = A.quantize_k(kd, with_mean=False)
    o8 = torch.empty_like(qd)
    o16 = torch.empty_like(qd)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        A.quantize_k(kd, out=kz, with_mean=False)
        if evs:
            evs[1].record(stream)
        A.fwd_int8_fused_q(qd, kz, vd, causal=w.causal, out=o8)
        if evs:
            evs[2].record(stream)
        A.fwd_fp16(qd, kd, vd, causal=w.causal, out=o16)
        if evs:
            evs[3].record(stream)

    prewarm_calls = clock_warm(step, batch=1)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = lambda a, b: float(np.mean([e[a].elapsed_time(e[b]) for e in ev]))
    return dict(ms_q=mean(0, 1), ms_8=mean(1, 2), ms_16=mean(2, 3), wall=wall, prewarm=prewarm_calls,
                qd=qd, kd=kd, vd=vd, kz=kz, o8=o8, o16=o16)


def config_entry(w, t):
    """The per-workload record of paths.configs."""
    flop = w.flops()
    tf = lambda ms: flop / (ms * 1e-3) / 1e12
    by = algorithmic_bytes(w)
    e2e = tf(t["ms_q"] + t["ms_8"])
    return {
        "shape": {"batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv, "seq": w.seq,
                  "head_dim": w.head_dim, "causal": w.causal},
        "flop": flop,
        "int8": {"tflops": round(e2e, 2), "ms": round(t["ms_q"] + t["ms_8"], 4),
                 "frac_int8_peak": round(e2e / PEAK_TFLOPS["int8"], 4),
                 "frac_blended_peak": round(e2e / PEAK_BLEND, 4)},
        "int8_fwd_only": {"tflops": round(tf(t["ms_8"]), 2), "ms": round(t["ms_8"], 4),
                          "frac_int8_peak": round(tf(t["ms_8"]) / PEAK_TFLOPS["int8"], 4),
                          "frac_blended_peak": round(tf(t["ms_8"]) / PEAK_BLEND, 4)},
        "fp16": {"tflops": round(tf(t["ms_16"]), 2), "ms": round(t["ms_16"], 4),
                 "frac_fp16_peak": round(tf(t["ms_16"]) / PEAK_TFLOPS["fp16"], 4)},
        "quantize_k": {"ms": round(t["ms_q"], 4),
                       "gbs": round(by["quantize_k"] / (t["ms_q"] * 1e-3) / 1e9, 1),
                       "frac_hbm_peak": round(by["quantize_k"] / (t["ms_q"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "int8_speedup_over_fp16": round(t["ms_16"] / (t["ms_q"] + t["ms_8"]), 3),
        # HBM bytes per call over the algorithmic bytes, from the committed
        # counter summaries of this workload (null where none or stale)
        "traffic_over_algorithmic": {tag: (None if tr is None else round(tr / by[tag], 3))
                                     for tag, tr in ((k, counters_for(k, w.name)) for k in by)},
    }


def run_workload(name, steps, warmup, cpu=False, cpu_seconds=12.0, configs=True, config_steps=10):
    import torch

    import bit_quantized_exact_amd as A
    from bit_quantized_exact_amd.inputs import WORKLOADS, make_qkv

    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    dev = torch.device("cuda:0")
    t = time_core(w, steps, warmup, tensors=tuple(torch.from_numpy(x).to(dev) for x in (q, k, v)))
    if not cpu:
        del q, k, v
    qd, kd, vd, o8, o16 = t["qd"], t["kd"], t["vd"], t["o8"], t["o16"]
    ms_q, ms_8, ms_16, wall = t["ms_q"], t["ms_8"], t["ms_16"], t["wall"]
    stream = torch.cuda.current_stream()

    # the two-call INT8 path (separate Q quantisation), timed after the steps
    qz = A.quantize_qk(qd, kd, with_mean=False)
    for _ in range(max(1, warmup)):
        A.quantize_qk(qd, kd, out=qz, with_mean=False)
        A.fwd_int8(qz, vd, causal=w.causal, out=o8)
    tc = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    n2 = max(1, min(steps, 10))
    tc[0].record(stream)
    for _ in range(n2):
        A.quantize_qk(qd, kd, out=qz, with_mean=False)
    tc[1].record(stream)
    for _ in range(n2):
        A.fwd_int8(qz, vd, causal=w.causal, out=o8)
    tc[2].record(stream)
    torch.cuda.synchronize()
    ms_qqk = tc[0].elapsed_time(tc[1]) / n2
    ms_8u = tc[1].elapsed_time(tc[2]) / n2
    # the FP8 alternative (E4M3 Q/K, FP16 P.V) and the 8-bit P.V ablation
    # (INT8 Q/K, E4M3 P and V): the comparisons the SageAttention article draws
    of8 = torch.empty_like(qd)
    opv8 = torch.empty_like(qd)
    qz8 = A.quantize_qk_fp8(qd, kd, with_mean=False)
    vz8 = A.quantize_v_fp8(vd)
    for _ in range(max(1, warmup)):
        A.fwd_fp8(qz8, vd, causal=w.causal, out=of8)
        A.fwd_int8_pv8(qz, vz8, causal=w.causal, out=opv8)
    te = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    te[0].record(stream)
    for _ in range(n2):
        A.quantize_qk_fp8(qd, kd, workspace=qz8["workspace"], with_mean=False)
    te[1].record(stream)
    for _ in range(n2):
        A.fwd_fp8(qz8, vd, causal=w.causal, out=of8)
    te[2].record(stream)
    for _ in range(n2):
        A.quantize_v_fp8(vd, workspace=vz8["workspace"])
    te[3].record(stream)
    for _ in range(n2):
        A.fwd_int8_pv8(qz, vz8, causal=w.causal, out=opv8)
    te[4].record(stream)
    torch.cuda.synchronize()
    ms_qf8, ms_f8, ms_qv8, ms_pv8 = (te[i].elapsed_time(te[i + 1]) / n2 for i in range(4))
    A.quantize_qk_fp8(qd, kd, workspace=qz8["workspace"], with_mean=False)
    A.fwd_fp8(qz8, vd, causal=w.causal, out=of8)
    A.quantize_v_fp8(vd, workspace=vz8["workspace"])
    A.fwd_int8_pv8(qz, vz8, causal=w.causal, out=opv8)
    A.fwd_int8_fused_q(qd, t["kz"], vd, causal=w.causal, out=o8)   # o8 is compared below
    del qz8, vz8, qz
    flop = w.flops()
    tf = lambda ms: flop / (ms * 1e-3) / 1e12
    int8_e2e = tf(ms_q + ms_8)
    by = algorithmic_bytes(w)

    kernels = {
        "fwd_fp16": dict(ms=ms_16, peak=PEAK_TFLOPS["fp16"]),
        "fwd_int8": dict(ms=ms_8, peak=PEAK_BLEND),
        "quantize_k": dict(ms=ms_q, peak=None),
    }
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    kd_ = kernels[dom]
    if dom == "quantize_k":
        achieved = by[dom] / (kd_["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    elif dom == "fwd_fp16":
        achieved = tf(kd_["ms"])
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS["fp16"],
                "unit": "TFLOP/s", "frac": achieved / PEAK_TFLOPS["fp16"]}
    else:
        achieved = tf(kd_["ms"])
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BLEND,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BLEND,
                "peak_note": "int8 QK^T at 5.0 POP/s and fp16 PV at 2.5 PFLOP/s, harmonic blend"}
    roof["kernel"] = {"fwd_fp16": "attn_fwd_fp16", "fwd_int8": "attn_fwd_int8_fused_q",
                      "quantize_k": "attn_quantize_k"}[dom]
    roof["traffic"] = counters_for(dom, name)
    roof["algorithmic_bytes"] = by[dom]
    roof["flop_per_launch"] = flop if dom != "quantize_k" else 0.0

    B, Hq, Hkv, S, D = w.batch, w.heads_q, w.heads_kv, w.seq, w.head_dim
    rec = {
        "metric": "attention fwd TFLOPS (INT8 & FP16 paths) and % of gfx950 MFMA peak, 1 GPU",
        "value": round(int8_e2e, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "clock_warmup": {"ms": CLOCK_WARM_MS, "steps": t["prewarm"],
                         "note": "untimed steps before the warm-up steps, until the clocks have ramped"},
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "heads_q": Hq, "heads_kv": Hkv, "seq": S,
                   "head_dim": D, "causal": w.causal,
                   "value_is": "INT8 path: FLOP / (t_quantize_k + t_fwd_int8_fused_q)"},
        "paths": {
            "int8": {"tflops": round(int8_e2e, 2), "ms": round(ms_q + ms_8, 4),
                     "fwd_only_tflops": round(tf(ms_8), 2), "fwd_ms": round(ms_8, 4),
                     "quantize_ms": round(ms_q, 4),
                     "quantize_gbs": round(by["quantize_k"] / (ms_q * 1e-3) / 1e9, 1),
                     "quantize_frac_hbm_peak": round(by["quantize_k"] / (ms_q * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "two_call_tflops": round(tf(ms_qqk + ms_8u), 2),
                     "two_call_quantize_qk_ms": round(ms_qqk, 4),
                     "two_call_fwd_int8_ms": round(ms_8u, 4),
                     "frac_int8_peak": round(int8_e2e / PEAK_TFLOPS["int8"], 4),
                     "frac_blended_peak": round(int8_e2e / PEAK_BLEND, 4),
                     "fwd_only_frac_blended_peak": round(tf(ms_8) / PEAK_BLEND, 4),
                     "fwd_traffic": counters_for("fwd_int8", name),
                     "fwd_algorithmic_bytes": by["fwd_int8"],
                     "quantize_traffic": counters_for("quantize_k", name)},
            "fp16": {"tflops": round(tf(ms_16), 2), "ms": round(ms_16, 4),
                     "frac_fp16_peak": round(tf(ms_16) / PEAK_TFLOPS["fp16"], 4)},
            "int8_speedup_over_fp16": round(ms_16 / (ms_q + ms_8), 3),
            "fp8_qk": {"fwd_tflops": round(tf(ms_f8), 2), "fwd_ms": round(ms_f8, 4),
                       "quantize_qk_fp8_ms": round(ms_qf8, 4),
                       "two_call_tflops": round(tf(ms_qf8 + ms_f8), 2),
                       "fwd_frac_blended_peak": round(tf(ms_f8) / PEAK_BLEND, 4),
                       "peak_note": "fp8 QK^T at 5.0 PFLOP/s and fp16 PV at 2.5, harmonic blend"},
            "int8_pv8": {"fwd_tflops": round(tf(ms_pv8), 2), "fwd_ms": round(ms_pv8, 4),
                         "quantize_v_fp8_ms": round(ms_qv8, 4),
                         "fwd_frac_peak": round(tf(ms_pv8) / PEAK_TFLOPS["int8"], 4),
                         "peak_note": "int8 QK^T and fp8 PV, both 5.0 P(FL)OP/s"},
        },
        "roofline": {k_: (round(v_, 4) if isinstance(v_, float) else v_) for k_, v_ in roof.items()},
        "cpu_baseline": None,
    }
    if cpu:
        rec["cpu_baseline"], rec["parity_sample"] = cpu_baseline(w, q, k, v, o8, o16, cpu_seconds,
                                                                 extra={"fp8_qk": of8, "int8_pv8": opv8})
        del q, k, v
    del of8, opv8
    own = config_entry(w, t)
    del t, qd, kd, vd, o8, o16
    torch.cuda.empty_cache()
    if configs:
        rec["paths"]["configs"] = {}
        for cname, cw in WORKLOADS.items():
            if cname == name:
                rec["paths"]["configs"][cname] = dict(own, timed_steps=steps, note="the headline steps")
                continue
            ct = time_core(cw, config_steps, max(1, warmup // 2))
            rec["paths"]["configs"][cname] = dict(config_entry(cw, ct), timed_steps=config_steps)
            if cname == APB_WORKLOAD:
                rec["paths"]["apb_masked"] = run_apb(ct["qd"], ct["kd"], ct["vd"], cw)
            del ct
            torch.cuda.empty_cache()
    rec["paths"]["decode"] = run_decode()
    rec["mfma_loop"] = run_mfma_loop()
    rec["hbm_read"] = run_hbm_read()
    return rec


def run_hbm_read(nbytes=1 << 32, reps=10, per_cu=(1, 2, 3, 4)):
    """Practical HBM read bandwidth of this device: streaming passes over a
    4 GiB buffer (16 times the 256 MB Infinity Cache, so the reads come from
    HBM; attn_probe_hbm_read: non-temporal 16-byte loads, four in flight per
    thread), with 1 to 4 workgroups of 256 threads per compute unit (more bytes
    in flight per compute unit measured slower), each timed with HIP events
    on the launch stream after a clock warm-up; the best shape is reported.
    Context for the HBM-bound kernels (decode, quantisation), whose
    `frac_hbm_peak` stays against the published 8 TB/s."""
    import ctypes

    import torch

    from bit_quantized_exact_amd import probe

    L = probe.lib()
    cus = ctypes.c_int(0)
    if L.attn_probe_compute_units(ctypes.byref(cus)) != 0 or cus.value <= 0:
        return None
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(max(per_cu) * cus.value * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def time_shape(blocks):
        def launch():
            st = L.attn_probe_hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes, blocks,
                                       ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
            if st != 0:
                raise RuntimeError(f"attn_probe_hbm_read failed: {st}")

        clock_warm(launch, min_ms=50, batch=2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    shapes = {n: time_shape(n * cus.value) for n in per_cu}
    best = min(shapes, key=shapes.get)
    ms = shapes[best]
    gbs = nbytes / (ms * 1e-3) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "workgroups_per_cu": best, "ms": round(ms, 4), "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "gbs_by_workgroups_per_cu": {str(n): round(nbytes / (t * 1e-3) / 1e9, 1) for n, t in shapes.items()}}


def run_mfma_loop(iters=20000, reps=5):
    """Sustained matrix-core rate of this device: a dense MFMA loop (four
    independent accumulator chains per wave, two waves per SIMD on every
    compute unit; attn_probe_mfma), timed with HIP events on the launch stream
    after a clock warm-up.  Context for `roofline`, whose peak stays the
    published figure.  `softmax_mix` times the FP16 loop with softmax-like
    vector work beside every MFMA (one exp2 and five FMAs on independent
    registers), that vector work alone, and both together: `hidden_frac` is
    the share of the shorter of the two that runs under the other."""
    import ctypes

    import torch

    from bit_quantized_exact_amd import probe

    L = probe.lib()
    cus = ctypes.c_int(0)
    if L.attn_probe_compute_units(ctypes.byref(cus)) != 0 or cus.value <= 0:
        return None
    blocks = 2 * cus.value
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def time_kind(kind):
        ops = ctypes.c_double(0.0)

        def launch():
            st = L.attn_probe_mfma(kind, blocks, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.byref(ops),
                                   ctypes.c_void_p(stream.cuda_stream))
            if st != 0:
                raise RuntimeError(f"attn_probe_mfma failed: {st}")

        clock_warm(launch, min_ms=100, batch=2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps, ops.value

    out = {"compute_units": cus.value, "waves_per_simd": 2}
    ms = {}
    for kind, key, fkey, peak in ((0, "fp16_tflops", "fp16_frac_of_published_peak", PEAK_TFLOPS["fp16"]),
                                  (1, "int8_tops", "int8_frac_of_published_peak", PEAK_TFLOPS["int8"])):
        t, ops = time_kind(kind)
        ms[kind] = t
        rate = ops / (t * 1e-3) / 1e12
        out[key] = round(rate, 1)
        out[fkey] = round(rate / peak, 4)
    t_both, _ = time_kind(2)
    t_valu, _ = time_kind(3)
    t_mfma = ms[0]
    out["softmax_mix"] = {"mfma_alone_ms": round(t_mfma, 4), "valu_alone_ms": round(t_valu, 4),
                          "both_ms": round(t_both, 4),
                          "hidden_frac": round((t_mfma + t_valu - t_both) / min(t_mfma, t_valu), 3)}
    return out


def run_decode(name="decode_gqa", reps=20, warm_ms=None, cold_reps=15):
    """KV-cache decode (one query per sequence over a cached context): the
    INT8 kernel (cache quantised once beforehand) and the FP16 kernel, each
    timed with HIP events; HBM-bound, so reported as GB/s of algorithmic bytes
    (the cache read once, Q read and O written once) against 8 TB/s.  `us`
    and `gbs` time calls back to back, where part of a cache that does not
    fill the 256 MB Infinity Cache can stay there from one call to the next;
    `us_cold` and `gbs_cold` time single calls, each after a 1 GiB read has
    evicted the cache (the case of a model whose layers each read their own
    cache), median of `cold_reps`."""
    import torch

    import bit_quantized_exact_amd as A
    from bit_quantized_exact_amd.inputs import DECODE_WORKLOADS, make_qkv

    w = DECODE_WORKLOADS[name]
    q, k, v = make_qkv(w)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    kz = A.quantize_k(kd, with_mean=False)
    o8, o16 = torch.empty_like(qd), torch.empty_like(qd)
    ws8 = torch.empty(A.decode_workspace_bytes(A.AttnKvShape(w.batch, w.heads_q, w.heads_kv, w.n_q, w.seq,
                                                              w.head_dim)), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    f8 = lambda: A.decode_int8(qd, kz, vd, causal=w.causal, out=o8, workspace=ws8)
    f16 = lambda: A.decode_fp16(qd, kd, vd, causal=w.causal, out=o16, workspace=ws8)
    res, cold = {}, {}
    evict = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    for tag, fn in (("int8", f8), ("fp16", f16)):
        clock_warm(fn, min_ms=CLOCK_WARM_MS if warm_ms is None else warm_ms, batch=16)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[tag] = e0.elapsed_time(e1) / reps
        ts = []
        for _ in range(cold_reps):
            torch.sum(evict, dtype=torch.int64)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        cold[tag] = float(np.median(ts))
    del evict
    B, Hq, Hkv, Sq, Sk, D = w.batch, w.heads_q, w.heads_kv, w.n_q, w.seq, w.head_dim
    qo = 2 * 2 * B * Hq * Sq * D
    bytes8 = B * Hkv * Sk * D + 2 * B * Hkv * Sk * D + qo + 4 * B * Hkv * math.ceil(Sk / 64)
    bytes16 = 2 * 2 * B * Hkv * Sk * D + qo
    out = {"workload": name, "batch": B, "heads_q": Hq, "heads_kv": Hkv, "seq_q": Sq, "seq_kv": Sk,
           "head_dim": D, "causal": w.causal}
    for tag, nbytes in (("int8", bytes8), ("fp16", bytes16)):
        ms = res[tag]
        gbs = nbytes / (ms * 1e-3) / 1e9
        gbs_c = nbytes / (cold[tag] * 1e-3) / 1e9
        out[tag] = {"us": round(ms * 1e3, 2), "algorithmic_bytes": nbytes, "gbs": round(gbs, 1),
                    "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                    "us_cold": round(cold[tag] * 1e3, 2), "gbs_cold": round(gbs_c, 1),
                    "frac_hbm_peak_cold": round(gbs_c / HBM_PEAK_GBS, 4),
                    "tokens_per_s": round(B * Sq / (ms * 1e-3), 1),
                    "tflops": round(w.flops() / (ms * 1e-3) / 1e12, 2)}
    out["int8_speedup_over_fp16"] = round(res["fp16"] / res["int8"], 3)
    return out


def run_apb(qd, kd, vd, w, anchor=1024, passing=2048, reps=10):
    """The LLM-prefill shape under the APB tile mask (keys [anchor | passing |
    local]): the FP16 and INT8 masked forwards; FLOP over the visible pairs."""
    import torch

    import bit_quantized_exact_amd as A

    qz = A.quantize_qk(qd, kd, with_mean=False)
    S = w.seq
    csr = A.block_mask_csr(S, A.apb_block_mask(S, anchor, passing))
    o = torch.empty_like(qd)
    stream = torch.cuda.current_stream()
    res = {}
    for tag, fn in (("fp16", lambda: A.fwd_fp16_masked(qd, kd, vd, csr, out=o)),
                    ("int8", lambda: A.fwd_int8_masked(qz, vd, csr, out=o))):
        clock_warm(fn, min_ms=100.0, batch=2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[tag] = e0.elapsed_time(e1) / reps
    rows = np.r_[0:anchor, anchor + passing:S]
    pairs = float((rows + 1).sum())
    flop = 4.0 * w.batch * w.heads_q * w.head_dim * pairs
    out = {"workload": w.name, "anchor": anchor, "passing": passing, "local": S - anchor - passing,
           "mask_tiles_listed": csr["nnz"]}
    for tag in ("fp16", "int8"):
        out[tag] = {"ms": round(res[tag], 4), "tflops": round(flop / (res[tag] * 1e-3) / 1e12, 2)}
    return out


def cpu_baseline(w, q, k, v, o8, o16, target_s, extra=None):
    """Time the CPU oracle (fp64 exact attention) on sampled query rows of the
    same workload and compare the GPU outputs on those rows."""
    from oracle import oracle as O

    threads = len(os.sched_getaffinity(0))
    rng = np.random.default_rng([w.seed, 1234])

    def row_flop(rows):
        vis = (rows + 1) if w.causal else np.full(rows.shape, w.seq)
        return float(4.0 * w.head_dim * vis.sum() * w.batch * w.heads_q)

    def timed(rows):
        t = time.perf_counter()
        out = O.attention(q, k, v, causal=w.causal, rows=rows, nthreads=threads)
        return out, time.perf_counter() - t

    # calibrate on 128 rows (several per thread, so that the threads' share
    # is as even as in the sample), then size the sample for about target_s
    ncal = min(w.seq, 128)
    cal = np.sort(rng.choice(w.seq, ncal, replace=False)).astype(np.int32)
    _, tc = timed(cal)
    n = int(min(w.seq, max(ncal, ncal * target_s / max(tc, 1e-3))))
    rows = np.sort(rng.choice(w.seq, n, replace=False)).astype(np.int32)
    out, dt = timed(rows)
    fl = row_flop(rows)
    g8 = o8.cpu().numpy()[:, :, rows].astype(np.float64)
    g16 = o16.cpu().numpy()[:, :, rows].astype(np.float64)
    a, b = g8.ravel(), out.ravel()
    parity = {
        "rows": int(n) * w.batch * w.heads_q,
        "fp16_max_abs": float(np.abs(g16 - out).max()),
        "int8_cos": float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b))),
        "int8_rel_l1": float(np.abs(a - b).sum() / np.abs(b).sum()),
    }
    for key, t in (extra or {}).items():
        a = t.cpu().numpy()[:, :, rows].astype(np.float64).ravel()
        parity[f"{key}_cos"] = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
        parity[f"{key}_rel_l1"] = float(np.abs(a - b).sum() / np.abs(b).sum())
    base = {
        "value": round(fl / dt / 1e12, 6),
        "unit": "TFLOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{n} of {w.seq} query rows (uniform random, seeded) of every one of the "
                   f"{w.batch * w.heads_q} (batch, head) pairs; fp64 exact attention; "
                   f"{fl / 1e9:.1f} GFLOP in {dt:.2f} s"),
        "seconds": round(dt, 3),
        "full_workload_seconds_extrapolated": round(w.flops() / (fl / dt), 1),
        "extrapolation_note": "the whole workload's oracle time at the sample's rate (extrapolated, not run)",
    }
    return base, parity


def copy_calibration(nbytes: int):
    """A plain elementwise copy (torch.neg on fp16) of nbytes, read once and
    written once: the reference that scales rocprofv3's FETCH_SIZE/WRITE_SIZE."""
    import torch
    n = nbytes // 2
    src = torch.ones(n, dtype=torch.float16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 2, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    global CLOCK_WARM_MS
    CLOCK_WARM_MS = args.clock_warm_ms
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the hot path "
              "shards by kv-head groups with no communication, so it is measured per GPU.",
              file=sys.stderr)
        sys.exit(2)
    if args.decode_only:
        print(json.dumps(run_decode(reps=args.decode_reps)), flush=True)
        return
    if args.only_step:
        from bit_quantized_exact_amd.inputs import WORKLOADS
        w = WORKLOADS[args.workload]
        t = time_core(w, args.steps, args.warmup)
        print(json.dumps({"workload": args.workload, "steps": args.steps, "ms_quantize_k": round(t["ms_q"], 4),
                          "ms_fwd_int8_fused_q": round(t["ms_8"], 4), "ms_fwd_fp16": round(t["ms_16"], 4)}),
              flush=True)
        return
    rec = run_workload(args.workload, args.steps, args.warmup, cpu=not args.no_cpu,
                       cpu_seconds=args.cpu_seconds, configs=not args.no_configs,
                       config_steps=args.config_steps)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
