#!/usr/bin/env python3
"""Benchmark of the causal self-attention hot path on one MI355X.

One step = one pass of the training hot path at the d20 shape
(B=32, T=2048, H=10, D=128, bf16): the forward (o, lse) and the backward
(delta, dk/dv, dq) through the C ABI.  Inputs are the seeded synthetic
tensors of the `workloads` module, resident in HBM before timing starts.
Each measured section first runs its call back to back, untimed, for
--ramp-seconds (default 0.3 s; reported as "clock_ramp_s"): after the
host-side input setup the GPU has idled and its clocks are down, and a K-step
run that starts after an idle gap of 10 ms or more measures about 8% slower
than the same steps back to back, which is the state of a training loop.
Then W untimed warmup steps, then exactly K timed steps between
torch.cuda.synchronize() calls; per-kernel durations come from HIP events
recorded on the launch stream around every kernel of every fourth timed step
(--kernel-events-every: an event between two kernels adds a few
microseconds, about 1% of the step when every step carries them).

The single-token decode over the ragged d20 cache (B=64, H=10, lengths
uniform in [1, 2048]) is timed in its own loop and reported under "decode";
it rotates three separately allocated caches so that no call finds its
cache in the 256 MB Infinity Cache; the same step with the new token's
append and the QK norm + rotary embedding folded in is reported beside it
("with_append_rope_us").  The call time comes from HIP events
around each call; the split/combine breakdown from a second loop that also
records an event between the two kernels (which adds a gap of its own).

The same d20 step with a sliding window (--window, default 1024: the short
"S" layers of nanochat's SSSL pattern; the pages give no window length, so
half the context is this benchmark's choice) and the windowed decode are
timed the same way and reported under "sliding_window" (FLOPs and bytes
counted over the visible (query, key) pairs only).

Prefill over a KV cache (16 sequences, a 512-token chunk each over caches of
U[0, 1536] rows, T_cap 2048, d20 heads; the chat-prefill shape of the
inference engine, sizes chosen here) is timed and reported under "prefill"
(append + attention, FLOPs over the visible pairs), and again with the QK norm
and rotary embedding folded in, next to the prologue kernel followed by the
prefill ("with_qk_norm_rope").

The attention prologue (RMS normalisation + rotary embedding of q and k at
the d20 shape, forward and backward, and the value-embedding gate on the d20
key/value heads) is timed and reported under "prologue" (algorithmic bytes:
every tensor read or written once, plus the cos/sin tables), and so is the
d20 step with the whole prologue (its forward kernels, the attention forward
and backward, and the prologue's backward either as its own two kernels or
folded into the attention backward; and with the query rows' normalisation
and rotation folded into the attention forward as well, "folded_fwd_bwd":
"d20_step_with_prologue_ms").

Grouped-query attention (--kv-heads, default 5: two query heads per key/value
head, a choice of this benchmark; the pages give no key/value head count) is
timed the same way on the d20 step and the decode and reported under "gqa".

The same K-step loop then runs --trials more times (default 5); their
per-step times, median and spread are reported under "trials" (the headline
value stays the first timed run), and each kernel's event times carry their
median and range beside the mean.

The fp64 oracle runs once on a bounded sample of the same workload on the
host cores and is reported as "cpu_baseline" (a reported baseline, not the
target).

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("causal attn fwd+bwd TFLOP/s @ d20 (B32,T2048,H10,D128) + % bf16 peak; "
          "decode GB/s")
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e)
        return evs

    def record(self, e, stream):
        assert self.hip.hipEventRecord(e, stream) == 0

    def ms(self, a, b):
        assert self.hip.hipEventSynchronize(b) == 0
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return float(out.value)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_d20.json")
KERNEL_SOURCES = {  # the sources whose text determines each kernel's code
    "fwd": ["fwd_bf16.hip", "device_common.hpp", "internal.hpp"],
    "delta": ["bwd_bf16.hip", "device_common.hpp", "internal.hpp"],
    "dkdv": ["bwd_bf16.hip", "device_common.hpp", "internal.hpp"],
    "dq": ["bwd_bf16.hip", "device_common.hpp", "internal.hpp"],
    "qk_norm_rope_fwd": ["prologue_bf16.hip", "device_common.hpp", "internal.hpp"],
    "qk_norm_rope_bwd": ["prologue_bf16.hip", "device_common.hpp", "internal.hpp"],
    "value_gate_fwd": ["prologue_bf16.hip", "device_common.hpp", "internal.hpp"],
    "value_gate_bwd": ["prologue_bf16.hip", "device_common.hpp", "internal.hpp"],
    "decode_split": ["decode_bf16.hip", "device_common.hpp", "internal.hpp"],
    "decode_combine": ["decode_bf16.hip", "device_common.hpp", "internal.hpp"],
}


def source_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "causal_self_attention_mha_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel):
    """HBM bytes per launch recorded by the rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (already scaled by the copy-probe calibration), or None when no record
    exists or the kernel's source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(kernel):
        return None
    return int(rec["bytes_per_launch"])


def train_flops(B, T, H, D):
    """Algorithmic FLOPs (causal = half of dense): fwd 2 matmuls, bwd 5."""
    unit = B * H * T * T * D   # one causal matmul: 2 * (T^2 / 2) * D per (b, h)
    return {"fwd": 2 * unit, "delta": 0, "dkdv": 4 * unit, "dq": 1 * unit, "fwd+bwd": 7 * unit}


def design_bytes(B, T, H, D):
    """HBM bytes per launch of the design as built: every operand read once,
    every result written once, including the dS workspace the backward streams
    (dkdv writes dS, bf16 lower-triangular 32 x 32 blocks per head, and dq reads
    it back with K)."""
    t = B * T * H * D * 2          # one bf16 (B, T, H, D) tensor
    r = B * H * T * 4              # one fp32 (B, H, T) row vector
    nblk = (T + 31) // 32
    ds = B * H * nblk * (nblk + 1) // 2 * 32 * 32 * 2
    return {"fwd": 3 * t + t + r, "delta": 2 * t + r, "dkdv": 4 * t + 2 * r + 2 * t + ds,
            "dq": t + ds + t}


def method_bytes(B, T, H, D):
    """HBM bytes per launch of the split-pass method itself (no dS workspace):
    each pass reads its own operands once and writes its results once.
    fwd: q, k, v -> o, lse.  delta: o, dO -> delta.  dkdv: q, k, v, dO, lse,
    delta -> dk, dv.  dq: q, k, v, dO, lse, delta -> dq.  The step-level
    minimum (every tensor of the layer moved once) is under "fwd_min" and
    "bwd_min": q, k, v, o, dO, lse read and dq, dk, dv written."""
    t = B * T * H * D * 2
    r = B * H * T * 4
    return {"fwd": 4 * t + r, "delta": 2 * t + r, "dkdv": 6 * t + 2 * r, "dq": 5 * t + 2 * r,
            "fwd_min": 4 * t + r, "bwd_min": 8 * t + r}


def visible_pairs(T, window):
    """(query, key) pairs per head with j <= i and, given a window, i - j <= window."""
    if window is None or window >= T - 1:
        return T * (T + 1) // 2
    w = window
    return (w + 1) * (w + 2) // 2 - (w + 1) + (T - w) * (w + 1) if T > w else T * (T + 1) // 2


def cpu_baseline(inp, n_heads, dinp=None, n_seqs=0):
    """Time the fp64 oracle (as it stands) on the first n_heads (b, h) heads of
    the training workload, forward and backward separately, and on the first
    n_seqs sequences of the decode workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max(i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas") or 1
    except Exception:  # pragma: no cover
        blas = None
    B, T, H, D = inp.shape
    heads = [(b, h) for b in range(B) for h in range(H)][:n_heads]
    t0 = time.perf_counter()
    oracle.forward(inp.q, inp.k, inp.v, heads=heads)
    t1 = time.perf_counter()
    oracle.backward(inp.q, inp.k, inp.v, inp.do, heads=heads)
    t2 = time.perf_counter()
    unit = len(heads) * T * T * D    # one causal matmul over the sampled heads
    fwd_s, bwd_s = t1 - t0, t2 - t1
    res = {"value": round(7 * unit / (t2 - t0) / 1e12, 6), "unit": "TFLOP/s",
           "cores": int(blas or os.cpu_count()), "kind": "oracle",
           "sample": (f"fp64 numpy oracle fwd then bwd on {len(heads)} of {B * H} (b,h) heads "
                      f"of the d20 workload (T={T}), {t2 - t0:.1f} s wall, algorithmic FLOPs "
                      "as the GPU (fwd 2, bwd 5 causal matmuls)"),
           "seconds": round(t2 - t0, 3), "os_cpu_count": os.cpu_count(), "blas_threads": blas,
           "fwd": {"seconds": round(fwd_s, 3), "TFLOP_per_s": round(2 * unit / fwd_s / 1e12, 6)},
           "bwd": {"seconds": round(bwd_s, 3),
                   "TFLOP_per_s": round(5 * unit / bwd_s / 1e12, 6)}}
    if dinp is not None and n_seqs > 0:
        sl = dinp.seqlens[:n_seqs]
        Hd = dinp.q.shape[1]
        t0 = time.perf_counter()
        oracle.decode(dinp.q[:n_seqs], dinp.k_cache[:n_seqs], dinp.v_cache[:n_seqs], sl)
        dt = time.perf_counter() - t0
        nbytes = int(sl.astype(np.int64).sum()) * Hd * D * 2 * 2
        res["decode"] = {"seconds": round(dt, 3), "sequences": int(n_seqs),
                         "GB_per_s": round(nbytes / dt / 1e9, 3),
                         "sample": f"fp64 oracle decode of {n_seqs} of {len(dinp.seqlens)} "
                                   "sequences of the d20 decode workload, bytes counted as "
                                   "the bf16 cache rows the GPU reads"}
    return res


def sample_sclk(run_load, seconds, period=0.002):
    """Sample the current shader clock (the starred line of the amdgpu driver's
    pp_dpm_sclk file) and the board power (its hwmon power1_input, microwatts,
    beside the power1_cap limit) while run_load() keeps the GPU busy."""
    import glob
    import re
    import threading
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not paths:
        return {"source": None, "note": "no pp_dpm_sclk file readable"}
    samples = {p: [] for p in paths}
    power = {p: [] for p in paths}

    def hwmon_file(p, name):
        found = sorted(glob.glob(os.path.join(os.path.dirname(p), "hwmon", "hwmon*", name)))
        return found[0] if found else None

    pin = {p: hwmon_file(p, "power1_input") for p in paths}
    stop = threading.Event()

    def read_int(path):
        try:
            with open(path) as fh:
                return int(fh.read().strip())
        except (OSError, ValueError):
            return None

    def sampler():
        while not stop.is_set():
            for p in paths:
                if pin[p]:
                    w = read_int(pin[p])
                    if w is not None:
                        power[p].append(w / 1e6)
                try:
                    with open(p) as fh:
                        for line in fh:
                            if line.rstrip().endswith("*"):
                                m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                                if m:
                                    samples[p].append(int(m.group(1)))
                except OSError:
                    pass
            time.sleep(period)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        run_load()
    stop.set()
    th.join()
    # the busiest card is the one under load (other cards idle at a low clock)
    p = max(paths, key=lambda q: (np.median(samples[q]) if samples[q] else -1))
    v = np.array(samples[p], dtype=np.float64)
    if v.size == 0:
        return {"source": p, "note": "no samples"}
    res = {"source": p, "samples": int(v.size), "seconds": seconds,
           "median_MHz": float(np.median(v)), "mean_MHz": round(float(v.mean()), 1),
           "min_MHz": float(v.min()), "max_MHz": float(v.max()),
           "p10_MHz": float(np.percentile(v, 10)), "p90_MHz": float(np.percentile(v, 90))}
    if power[p]:
        w = np.array(power[p], dtype=np.float64)
        cap = hwmon_file(p, "power1_cap")
        cap_w = read_int(cap) if cap else None
        res["power"] = {"source": pin[p], "samples": int(w.size),
                        "median_W": round(float(np.median(w)), 1),
                        "p10_W": round(float(np.percentile(w, 10)), 1),
                        "p90_W": round(float(np.percentile(w, 90)), 1),
                        "max_W": round(float(w.max()), 1),
                        "cap_W": round(cap_w / 1e6, 1) if cap_w else None}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-iters", type=int, default=60)
    ap.add_argument("--cpu-heads", type=int, default=256,
                    help="(b,h) heads in the oracle CPU-baseline sample (0 = skip)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--window", type=int, default=1024,
                    help="sliding-window length for the extra windowed measurement (-1 = skip)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-prologue", action="store_true")
    ap.add_argument("--kernel-events-every", type=int, default=4,
                    help="record the per-kernel HIP events on every N-th timed step (each "
                         "event between two kernels adds a few microseconds to the step)")
    ap.add_argument("--kv-heads", type=int, default=5,
                    help="key/value heads for the extra grouped-query measurement (0 = skip)")
    ap.add_argument("--ramp-seconds", type=float, default=0.3,
                    help="untimed back-to-back calls before each section's warmup, so that "
                         "the GPU's clocks are up after the host-side setup (0 = none)")
    ap.add_argument("--trials", type=int, default=5,
                    help="further runs of the same K timed steps, reported as their spread "
                         "and median (the headline value is the first run)")
    ap.add_argument("--sclk-seconds", type=float, default=1.5,
                    help="seconds of back-to-back d20 steps during which the shader clock "
                         "is sampled from sysfs (0 = skip)")
    ap.add_argument("--depths", default="d12,d26",
                    help="other model depths whose fwd+bwd step is timed as well ('' = none)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="first run a plain device copy of this many MiB (a known-size "
                         "kernel that calibrates HBM byte counters in a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (--gpus {args.gpus} requested); "
              "the attention hot path has no cross-GPU step, see the design notes on sharding",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import causal_self_attention_mha_amd as na
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    lib = na.load_library()
    ev = HipEvents()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    def ramp(fn):
        """Untimed back-to-back calls of fn for --ramp-seconds before a section's
        warmup: after the host-side input setup the GPU has been idle and its
        clocks are down; a short warmup does not bring them back (a K-step run
        after a >= 10 ms idle gap measured about 8% slower than back to back)."""
        t_end = time.perf_counter() + args.ramp_seconds
        n = 0
        while time.perf_counter() < t_end:
            for _ in range(4):
                fn()
            n += 4
            torch.cuda.synchronize()
        log(f"ramp: {n} calls")

    if args.copy_probe_mb > 0:
        n = args.copy_probe_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 2.0, out=dst)  # elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        log(f"copy probe: {n} bytes read + {n} bytes written")
        del src, dst

    # ---------------- training step inputs (resident in HBM)
    cfg = W.CONFIGS[W.HEADLINE]
    B, T, H, D = cfg.B, cfg.T, cfg.H, cfg.D
    log(f"generating d20 inputs B={B} T={T} H={H} D={D}")
    inp = W.make_train_inputs(cfg)

    def dev_t(store):
        return torch.from_numpy(store.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = (dev_t(x) for x in (inp.q_store, inp.k_store, inp.v_store, inp.do_store))
    o = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    ws_bytes = na.bwd_workspace_bytes(B, T, H)     # dS scratch for the dQ GEMM
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    P = ctypes.c_void_p
    ptr = lambda t: P(t.data_ptr())  # noqa: E731

    n_total = args.warmup + args.steps
    evs = [ev.create(5) for _ in range(n_total)]
    ev_arr = [(ctypes.c_void_p * 4)(*[e.value for e in step[1:5]]) for step in evs]

    every = max(1, args.kernel_events_every)

    def instrumented(i):  # timed steps that carry the per-kernel events
        return (i - args.warmup) % every == 0

    timed_ev = [i for i in range(args.warmup, n_total) if instrumented(i)]

    def step(i, window=-1):
        e = evs[i]
        if instrumented(i):
            ev.record(e[0], stream)
        st = lib.na_attn_fwd_window(ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), B, T, H, D,
                                    window, P(stream))
        if st:
            raise RuntimeError(lib.na_last_error().decode())
        st = lib.na_attn_bwd_window(ptr(q), ptr(k), ptr(v), ptr(o), ptr(do), ptr(lse), ptr(dq),
                                    ptr(dk), ptr(dv), ptr(delta), ptr(ws), ws_bytes, B, T, H, D,
                                    window, P(stream),
                                    ctypes.cast(ev_arr[i], P) if instrumented(i) else None)
        if st:
            raise RuntimeError(lib.na_last_error().decode())

    ramp(lambda: step(0))
    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.warmup, n_total):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ["fwd", "delta", "dkdv", "dq"]
    per = {n: [] for n in names}
    step_ms = []
    for i in timed_ev:
        e = evs[i]
        for j, n in enumerate(names):
            per[n].append(ev.ms(e[j], e[j + 1]))
        step_ms.append(ev.ms(e[0], e[4]))
    # ms_per_step: synchronized wall clock over exactly K steps; the HIP-event
    # GPU time per step is reported beside it
    ms_per_step = wall * 1e3 / args.steps
    gpu_ms_per_step = float(np.mean(step_ms))
    fl = train_flops(B, T, H, D)
    tflops = fl["fwd+bwd"] / (ms_per_step * 1e-3) / 1e12
    kern = {}
    for n in names:
        avg = float(np.mean(per[n]))
        kern[n] = {"avg_us": round(avg * 1e3, 2), "min_us": round(min(per[n]) * 1e3, 2),
                   "median_us": round(float(np.median(per[n])) * 1e3, 2),
                   "max_us": round(max(per[n]) * 1e3, 2),
                   "tflops": round(fl[n] / (avg * 1e-3) / 1e12, 2) if fl[n] else None}
    log(f"step {ms_per_step:.3f} ms  {tflops:.1f} TFLOP/s  kernels {kern}")

    # dominant kernel roofline (MFMA bound; algorithmic FLOPs per launch)
    dom = max(("fwd", "dkdv", "dq"), key=lambda n: kern[n]["avg_us"])
    dom_avg_s = kern[dom]["avg_us"] * 1e-6
    achieved = fl[dom] / dom_avg_s / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": recorded_traffic(dom),
                "flops_per_launch": fl[dom],
                "design_bytes_per_launch": design_bytes(B, T, H, D)[dom],
                "method_bytes_per_launch": method_bytes(B, T, H, D)[dom]}

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*0.5 q,k,v; N(0,1)*1e-2 dO; no trained weights)",
        "config": {"workload": "d20 causal self-attention fwd+bwd", "B": B, "T": T, "H": H,
                   "D": D, "causal": True, "parallelism": "single GPU"},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "clock_ramp_s": args.ramp_seconds,
        "wall_s_timed": round(wall, 4),
        "gpu_ms_per_step_events": round(gpu_ms_per_step, 4),
        "kernel_event_steps": len(timed_ev),
        "kernels": kern,
        "roofline": roofline,
    }

    # ---------------- repeated trials of the same K-step loop (spread, median)
    if args.trials > 0:
        ramp(lambda: step(0))
        tr_ms = []
        for _ in range(args.trials):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.warmup, n_total):
                step(i)
            torch.cuda.synchronize()
            tr_ms.append((time.perf_counter() - t0) * 1e3 / args.steps)
        result["trials"] = {
            "count": args.trials, "steps_each": args.steps,
            "ms_per_step": [round(x, 4) for x in tr_ms],
            "median_ms_per_step": round(float(np.median(tr_ms)), 4),
            "min_ms_per_step": round(min(tr_ms), 4), "max_ms_per_step": round(max(tr_ms), 4),
            "median_TFLOP_per_s": round(fl["fwd+bwd"] / (float(np.median(tr_ms)) * 1e-3) / 1e12,
                                        2)}
        log(f"trials {result['trials']}")

    # ---------------- shader clock under the d20 step load
    if args.sclk_seconds > 0:
        def load():
            for i in range(args.warmup, args.warmup + 8):
                step(i)
            torch.cuda.synchronize()
        log(f"sampling the shader clock for {args.sclk_seconds} s of d20 steps")
        result["sclk_under_load"] = sample_sclk(load, args.sclk_seconds)
        log(f"sclk {result['sclk_under_load']}")

    # ---------------- the same step with a sliding window
    wlen = args.window if 0 <= args.window < T - 1 else None
    if wlen is not None:
        log(f"sliding window {wlen}: warmup {args.warmup}, timing {args.steps} steps")
        ramp(lambda: step(0, wlen))
        for i in range(args.warmup):
            step(i, wlen)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.warmup, n_total):
            step(i, wlen)
        torch.cuda.synchronize()
        wwall = time.perf_counter() - t0
        wper = {n: [] for n in names}
        for i in timed_ev:
            for j, n in enumerate(names):
                wper[n].append(ev.ms(evs[i][j], evs[i][j + 1]))
        pairs = visible_pairs(T, wlen)
        wfl = {"fwd": 2, "delta": 0, "dkdv": 4, "dq": 1}
        wfl = {n: c * B * H * pairs * 2 * D for n, c in wfl.items()}
        w_ms = wwall * 1e3 / args.steps
        wk = {}
        for n in names:
            avg = float(np.mean(wper[n]))
            wk[n] = {"avg_us": round(avg * 1e3, 2),
                     "tflops": round(wfl[n] / (avg * 1e-3) / 1e12, 2) if wfl[n] else None}
        w_tf = 7 * B * H * pairs * 2 * D / (w_ms * 1e-3) / 1e12
        result["sliding_window"] = {
            "workload": f"d20 causal self-attention fwd+bwd, sliding window {wlen}",
            "window": wlen, "ms_per_step": round(w_ms, 4), "TFLOP_per_s": round(w_tf, 2),
            "flops_per_step": 7 * B * H * pairs * 2 * D, "visible_pairs_per_head": pairs,
            "kernels": wk}
        log(f"sliding window {wlen}: {w_ms:.3f} ms  {w_tf:.1f} TFLOP/s  kernels {wk}")

    # ---------------- the same step with grouped key/value heads
    hkv = args.kv_heads if 0 < args.kv_heads < H and H % args.kv_heads == 0 else None
    if hkv is not None:
        kg, vg = k[:, :, :hkv].contiguous(), v[:, :, :hkv].contiguous()
        dkg, dvg = torch.empty_like(kg), torch.empty_like(vg)

        def gstep(i):
            e = evs[i]
            if instrumented(i):
                ev.record(e[0], stream)
            st = lib.na_attn_fwd_gqa(ptr(q), ptr(kg), ptr(vg), ptr(o), ptr(lse), B, T, H, hkv, D,
                                     -1, P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())
            st = lib.na_attn_bwd_gqa(ptr(q), ptr(kg), ptr(vg), ptr(o), ptr(do), ptr(lse),
                                     ptr(dq), ptr(dkg), ptr(dvg), ptr(delta), ptr(ws), ws_bytes,
                                     B, T, H, hkv, D, -1, P(stream),
                                     ctypes.cast(ev_arr[i], P) if instrumented(i) else None)
            if st:
                raise RuntimeError(lib.na_last_error().decode())

        log(f"gqa {H}/{hkv} heads: warmup {args.warmup}, timing {args.steps} steps")
        ramp(lambda: gstep(0))
        for i in range(args.warmup):
            gstep(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.warmup, n_total):
            gstep(i)
        torch.cuda.synchronize()
        gwall = time.perf_counter() - t0
        gk = {}
        for j, n in enumerate(names):
            avg = float(np.mean([ev.ms(evs[i][j], evs[i][j + 1]) for i in timed_ev]))
            gk[n] = {"avg_us": round(avg * 1e3, 2),
                     "tflops": round(fl[n] / (avg * 1e-3) / 1e12, 2) if fl[n] else None}
        g_ms = gwall * 1e3 / args.steps
        g_tf = fl["fwd+bwd"] / (g_ms * 1e-3) / 1e12
        result["gqa"] = {"workload": f"d20 causal self-attention fwd+bwd, {H} query heads, "
                                     f"{hkv} key/value heads", "kv_heads": hkv,
                         "ms_per_step": round(g_ms, 4), "TFLOP_per_s": round(g_tf, 2),
                         "kernels": gk}
        log(f"gqa: {g_ms:.3f} ms  {g_tf:.1f} TFLOP/s  kernels {gk}")
        del kg, vg, dkg, dvg

    # ---------------- the other depths of the model family (d12, d26)
    depths = [d for d in args.depths.split(",") if d] if args.depths else []
    if depths:
        result["depths"] = {}
    for dname in depths:
        c = W.CONFIGS[dname]
        dB, dT, dH, dD = c.B, c.T, c.H, c.D
        log(f"{dname}: B={dB} T={dT} H={dH} D={dD}: warmup {args.warmup}, timing {args.steps}")
        din = W.make_train_inputs(c)
        xq, xk, xv, xdo = (dev_t(x) for x in (din.q_store, din.k_store, din.v_store,
                                              din.do_store))
        del din
        xo, xdq, xdk, xdv = (torch.empty_like(xq) for _ in range(4))
        xlse = torch.empty((dB, dH, dT), dtype=torch.float32, device=dev)
        xdelta = torch.empty_like(xlse)
        xwsb = na.bwd_workspace_bytes(dB, dT, dH)
        xws = torch.empty(xwsb, dtype=torch.uint8, device=dev)

        def xstep(i):
            e = evs[i]
            if instrumented(i):
                ev.record(e[0], stream)
            st = lib.na_attn_fwd(ptr(xq), ptr(xk), ptr(xv), ptr(xo), ptr(xlse), dB, dT, dH, dD,
                                 P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())
            st = lib.na_attn_bwd_timed(ptr(xq), ptr(xk), ptr(xv), ptr(xo), ptr(xdo), ptr(xlse),
                                       ptr(xdq), ptr(xdk), ptr(xdv), ptr(xdelta), ptr(xws), xwsb,
                                       dB, dT, dH, dD, P(stream),
                                       ctypes.cast(ev_arr[i], P) if instrumented(i) else None)
            if st:
                raise RuntimeError(lib.na_last_error().decode())

        ramp(lambda: xstep(0))
        for i in range(args.warmup):
            xstep(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.warmup, n_total):
            xstep(i)
        torch.cuda.synchronize()
        xwall = time.perf_counter() - t0
        xfl = train_flops(dB, dT, dH, dD)
        xk_ = {}
        for j, n in enumerate(names):
            avg = float(np.mean([ev.ms(evs[i][j], evs[i][j + 1]) for i in timed_ev]))
            xk_[n] = {"avg_us": round(avg * 1e3, 2),
                      "tflops": round(xfl[n] / (avg * 1e-3) / 1e12, 2) if xfl[n] else None}
        bwd_us = sum(xk_[n]["avg_us"] for n in ("delta", "dkdv", "dq"))
        x_ms = xwall * 1e3 / args.steps
        x_tf = xfl["fwd+bwd"] / (x_ms * 1e-3) / 1e12
        result["depths"][dname] = {
            "workload": f"{dname} causal self-attention fwd+bwd", "B": dB, "T": dT, "H": dH,
            "D": dD, "ms_per_step": round(x_ms, 4), "TFLOP_per_s": round(x_tf, 2),
            "pct_bf16_peak": round(100 * x_tf / PEAK_BF16_TFLOPS, 2),
            "fwd_us": xk_["fwd"]["avg_us"], "bwd_us": round(bwd_us, 2),
            "fwd_TFLOP_per_s": xk_["fwd"]["tflops"],
            "bwd_TFLOP_per_s": round(5 * xfl["dq"] / (bwd_us * 1e-6) / 1e12, 2),
            "kernels": xk_}
        log(f"{dname}: {x_ms:.3f} ms  {x_tf:.1f} TFLOP/s  kernels {xk_}")
        del xq, xk, xv, xdo, xo, xdq, xdk, xdv, xlse, xdelta, xws
        torch.cuda.empty_cache()

    # ---------------- prologue: QK norm + rotary embedding of q and k
    if not args.no_prologue:
        # any angle table serves for timing: seeded random angles
        ct, sn = (torch.from_numpy(a).to(dev) for a in W.make_angle_tables(T, D // 2, seed=1))
        yq, yk, rgq, rgk = (torch.empty_like(q) for _ in range(4))
        rev = ev.create(4)
        eps = ctypes.c_float(1e-6)

        def rfwd():
            st = lib.na_qk_norm_rope_fwd(ptr(q), ptr(k), ptr(yq), ptr(yk), ptr(ct), ptr(sn), None,
                                         B, T, H, H, D, T, eps, P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())

        def rbwd():  # do and v stand in for the gradients of the rotated q and k
            st = lib.na_qk_norm_rope_bwd(ptr(q), ptr(k), ptr(do), ptr(v), ptr(rgq), ptr(rgk),
                                         ptr(ct), ptr(sn), None, B, T, H, H, D, T, eps,
                                         P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())

        ramp(lambda: (rfwd(), rbwd()))
        for _ in range(args.warmup):
            rfwd()
            rbwd()
        torch.cuda.synchronize()
        ev.record(rev[0], stream)
        for _ in range(args.steps):
            rfwd()
        ev.record(rev[1], stream)
        for _ in range(args.steps):
            rbwd()
        ev.record(rev[2], stream)
        f_ms = ev.ms(rev[0], rev[1]) / args.steps
        b_ms = ev.ms(rev[1], rev[2]) / args.steps
        # value-embedding gate on the d20 key/value heads: v, ve = q, k stand-ins
        gt = dev_t(W.make_gate_logits(B, T, H, seed=2)[1])

        def gfwd():
            st = lib.na_value_gate_fwd(ptr(v), ptr(k), ptr(gt), ptr(yq), B, T, H, D, P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())

        def gbwd():
            st = lib.na_value_gate_bwd(ptr(k), ptr(gt), ptr(do), ptr(rgq), ptr(yk), B, T, H, D,
                                       P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())

        ramp(lambda: (gfwd(), gbwd()))
        for _ in range(args.warmup):
            gfwd()
            gbwd()
        ev.record(rev[0], stream)
        for _ in range(args.steps):
            gfwd()
        ev.record(rev[1], stream)
        for _ in range(args.steps):
            gbwd()
        ev.record(rev[2], stream)
        torch.cuda.synchronize()
        gf_ms = ev.ms(rev[0], rev[1]) / args.steps
        gb_ms = ev.ms(rev[1], rev[2]) / args.steps
        vrow = B * T * H * D * 2
        gbytes = B * T * H * 2
        gfb, gbb = 3 * vrow + gbytes, 3 * vrow + 2 * gbytes
        row_bytes = B * T * 2 * H * D * 2          # q and k, bf16
        tab_bytes = 2 * T * (D // 2) * 4
        fb, bb = 2 * row_bytes + tab_bytes, 3 * row_bytes + tab_bytes
        result["prologue"] = {
            "workload": f"QK norm + rotary embedding of q and k: B={B}, T={T}, H={H}, D={D}, "
                        "bf16, fp32 (T, 64) cos/sin tables",
            "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
            "fwd_GB_per_s": round(fb / (f_ms * 1e-3) / 1e9, 1),
            "bwd_GB_per_s": round(bb / (b_ms * 1e-3) / 1e9, 1),
            "fwd_frac_hbm": round(fb / (f_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bwd_frac_hbm": round(bb / (b_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_fwd": fb, "bytes_bwd": bb,
            "traffic_fwd": recorded_traffic("qk_norm_rope_fwd"),
            "traffic_bwd": recorded_traffic("qk_norm_rope_bwd"),
            "value_gate": {"fwd_ms": round(gf_ms, 4), "bwd_ms": round(gb_ms, 4),
                           "fwd_GB_per_s": round(gfb / (gf_ms * 1e-3) / 1e9, 1),
                           "bwd_GB_per_s": round(gbb / (gb_ms * 1e-3) / 1e9, 1),
                           "bytes_fwd": gfb, "bytes_bwd": gbb,
                           "traffic_fwd": recorded_traffic("value_gate_fwd"),
                           "traffic_bwd": recorded_traffic("value_gate_bwd")},
            "calls": args.steps}
        log(f"prologue {result['prologue']}")
        # the d20 step with the prologue: prologue forward (QK norm + rotary
        # embedding of q and k, value-embedding gate of v; k stands in for ve),
        # attention forward and backward, prologue backward as its own kernels
        # or folded into the attention backward's epilogues (na_attn_bwd_rope
        # with the gate)
        tdq, tdk, tdv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        vg, tdve, tdg = torch.empty_like(v), torch.empty_like(v), torch.empty_like(gt)

        def pro_step(folded, folded_fwd=False):
            st = lib.na_value_gate_fwd(ptr(v), ptr(k), ptr(gt), ptr(vg), B, T, H, D, P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())
            if folded_fwd:  # keys by the prologue kernel, queries rotated in the forward
                st = lib.na_attn_fwd_rope(ptr(q), ptr(k), ptr(vg), ptr(ct), ptr(sn), T, eps,
                                          ptr(yq), ptr(yk), ptr(o), ptr(lse), B, T, H, H, D, -1,
                                          P(stream))
            else:
                rfwd()  # yq, yk = rotated q, k
                st = lib.na_attn_fwd(ptr(yq), ptr(yk), ptr(vg), ptr(o), ptr(lse), B, T, H, D,
                                     P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())
            if folded:
                st = lib.na_attn_bwd_rope(ptr(yq), ptr(yk), ptr(vg), ptr(o), ptr(do), ptr(lse),
                                          ptr(q), ptr(k), ptr(ct), ptr(sn), T, eps, ptr(k),
                                          ptr(gt), ptr(tdq), ptr(tdk), ptr(tdv), ptr(tdve),
                                          ptr(tdg), ptr(delta), ptr(ws), ws_bytes, B, T, H, H, D,
                                          -1, P(stream))
            else:
                st = lib.na_attn_bwd(ptr(yq), ptr(yk), ptr(vg), ptr(o), ptr(do), ptr(lse),
                                     ptr(rgq), ptr(rgk), ptr(tdv), ptr(delta), ptr(ws), ws_bytes,
                                     B, T, H, D, P(stream))
                if not st:
                    st = lib.na_qk_norm_rope_bwd(ptr(q), ptr(k), ptr(rgq), ptr(rgk), ptr(tdq),
                                                 ptr(tdk), ptr(ct), ptr(sn), None, B, T, H, H, D,
                                                 T, eps, P(stream))
                if not st:
                    st = lib.na_value_gate_bwd(ptr(k), ptr(gt), ptr(tdv), ptr(tdve), ptr(tdg), B,
                                               T, H, D, P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())

        step_ms = {}
        for name, folded, ffwd in (("folded_bwd", True, False), ("separate_bwd", False, False),
                                   ("folded_fwd_bwd", True, True)):
            ramp(lambda: pro_step(folded, ffwd))
            for _ in range(args.warmup):
                pro_step(folded, ffwd)
            torch.cuda.synchronize()
            ev.record(rev[0], stream)
            for _ in range(args.steps):
                pro_step(folded, ffwd)
            ev.record(rev[1], stream)
            torch.cuda.synchronize()
            step_ms[name] = round(ev.ms(rev[0], rev[1]) / args.steps, 4)
        result["prologue"]["d20_step_with_prologue_ms"] = step_ms
        del yq, yk, rgq, rgk, gt, tdq, tdk, tdv, vg, tdve, tdg

    del q, k, v, do, o, dq, dk, dv, ws
    torch.cuda.empty_cache()

    # ---------------- decode
    dinp_cpu = None
    if not args.no_decode:
        dcfg = W.CONFIGS[W.DECODE]
        log("generating decode inputs")
        dinp = dinp_cpu = W.make_decode_inputs(dcfg)
        Bd, Hd, Tc = dcfg.B, dcfg.H, dcfg.T_cap
        qd = dev_t(dinp.q_store)
        caches = []
        kc0, vc0 = dev_t(dinp.k_store), dev_t(dinp.v_store)
        for r in range(3):
            caches.append((kc0.clone(), vc0.clone()) if r else (kc0, vc0))
        lens = torch.from_numpy(dinp.seqlens).to(dev)
        od = torch.empty_like(qd)
        lsed = torch.empty((Bd, Hd), dtype=torch.float32, device=dev)
        wsb = na.decode_workspace_bytes(Bd, Hd, Tc)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        nd = args.decode_iters
        devs = [ev.create(3) for _ in range(nd + 5)]
        darr = [(ctypes.c_void_p * 3)(*[e.value for e in x]) for x in devs]

        def dstep(i, window=-1, per_kernel=False):
            # per_kernel: the _timed entry records an event between the two
            # kernels (for the split/combine breakdown); otherwise events sit
            # only around the call, so the call time has no event inside it
            kc, vc = caches[i % 3]
            e = devs[i]
            if not per_kernel:
                ev.record(e[0], stream)
            st = lib.na_attn_decode_window(ptr(qd), ptr(kc), ptr(vc), ptr(lens), ptr(od),
                                           ptr(lsed), Bd, Hd, D, Tc, window, ptr(ws), wsb,
                                           P(stream),
                                           ctypes.cast(darr[i], P) if per_kernel else None)
            if st:
                raise RuntimeError(lib.na_last_error().decode())
            if not per_kernel:
                ev.record(e[2], stream)

        ramp(lambda: dstep(0, per_kernel=True))
        for i in range(5):
            dstep(i, per_kernel=True)
        torch.cuda.synchronize()
        for i in range(5, nd + 5):
            dstep(i, per_kernel=True)
        torch.cuda.synchronize()
        split = [ev.ms(devs[i][0], devs[i][1]) for i in range(5, nd + 5)]
        comb = [ev.ms(devs[i][1], devs[i][2]) for i in range(5, nd + 5)]
        for i in range(5):
            dstep(i)
        torch.cuda.synchronize()
        for i in range(5, nd + 5):
            dstep(i)
        torch.cuda.synchronize()
        tot = [ev.ms(devs[i][0], devs[i][2]) for i in range(5, nd + 5)]
        kv_bytes = int(dinp.seqlens.astype(np.int64).sum()) * Hd * D * 2 * 2
        io_bytes = Bd * Hd * D * 2 * 2
        d_ms = float(np.mean(tot))
        gbs = (kv_bytes + io_bytes) / (d_ms * 1e-3) / 1e9
        split_gbs = kv_bytes / (float(np.mean(split)) * 1e-3) / 1e9
        result["decode"] = {
            "workload": "d20 decode B=64 H=10 D=128, lengths U[1,2048], T_cap=2048, bf16",
            "GB_per_s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
            "us_per_call": round(d_ms * 1e3, 2), "kv_bytes": kv_bytes,
            "split_avg_us": round(float(np.mean(split)) * 1e3, 2),
            "combine_avg_us": round(float(np.mean(comb)) * 1e3, 2),
            "split_GB_per_s": round(split_gbs, 1), "iters": nd, "rotated_caches": 3,
            "traffic_split": recorded_traffic("decode_split"),
            "traffic_combine": recorded_traffic("decode_combine"),
        }
        # the engine's per-token step: append the new token's rows (QK norm and
        # rotary embedding folded in), then attend over them with the cache
        act, ast = (torch.from_numpy(a).to(dev) for a in W.make_angle_tables(Tc, D // 2, seed=4))
        dnew = W.make_train_inputs(cfg, B=Bd, T=1, H=Hd, seed=7)
        kn_d, vn_d = dev_t(dnew.k_store), dev_t(dnew.v_store)
        lens_app = torch.from_numpy(np.minimum(dinp.seqlens, Tc - 1).astype(np.int32)).to(dev)
        deps = ctypes.c_float(1e-6)

        def astep(i):
            kc, vc = caches[i % 3]
            e = devs[i]
            ev.record(e[0], stream)
            st = lib.na_attn_decode_append(ptr(qd), ptr(kn_d), ptr(vn_d), ptr(kc), ptr(vc),
                                           ptr(lens_app), ptr(act), ptr(ast), Tc, deps, None,
                                           None, ptr(od), ptr(lsed), Bd, Hd, Hd, D, Tc, -1,
                                           ptr(ws), wsb, P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())
            ev.record(e[2], stream)

        for i in range(5):
            astep(i)
        torch.cuda.synchronize()
        for i in range(5, nd + 5):
            astep(i)
        torch.cuda.synchronize()
        a_ms = float(np.mean([ev.ms(devs[i][0], devs[i][2]) for i in range(5, nd + 5)]))
        result["decode"]["with_append_rope_us"] = round(a_ms * 1e3, 2)
        del kn_d, vn_d
        log(f"decode {result['decode']}")
        if wlen is not None:
            for i in range(5):
                dstep(i, wlen)
            torch.cuda.synchronize()
            for i in range(5, nd + 5):
                dstep(i, wlen)
            torch.cuda.synchronize()
            wtot = [ev.ms(devs[i][0], devs[i][2]) for i in range(5, nd + 5)]
            wkv = int(np.minimum(dinp.seqlens.astype(np.int64), wlen + 1).sum()) * Hd * D * 2 * 2
            w_ms = float(np.mean(wtot))
            w_gbs = (wkv + io_bytes) / (w_ms * 1e-3) / 1e9
            result["sliding_window"]["decode"] = {
                "us_per_call": round(w_ms * 1e3, 2), "kv_bytes": wkv,
                "GB_per_s": round(w_gbs, 1), "pct_hbm_peak": round(100 * w_gbs / PEAK_HBM_GBS, 2)}
            log(f"sliding window decode {result['sliding_window']['decode']}")
        if hkv is not None:
            gcaches = [(kc[:, :, :hkv].contiguous(), vc[:, :, :hkv].contiguous())
                       for kc, vc in caches]

            def gdstep(i):
                kc, vc = gcaches[i % 3]
                ev.record(devs[i][0], stream)
                st = lib.na_attn_decode_gqa(ptr(qd), ptr(kc), ptr(vc), ptr(lens), ptr(od),
                                            ptr(lsed), Bd, Hd, hkv, D, Tc, -1, ptr(ws), wsb,
                                            P(stream), None)
                if st:
                    raise RuntimeError(lib.na_last_error().decode())
                ev.record(devs[i][2], stream)

            for i in range(5):
                gdstep(i)
            torch.cuda.synchronize()
            for i in range(5, nd + 5):
                gdstep(i)
            torch.cuda.synchronize()
            gtot = [ev.ms(devs[i][0], devs[i][2]) for i in range(5, nd + 5)]
            gkv = int(dinp.seqlens.astype(np.int64).sum()) * hkv * D * 2 * 2
            g_ms = float(np.mean(gtot))
            g_gbs = (gkv + io_bytes) / (g_ms * 1e-3) / 1e9
            result.setdefault("gqa", {"kv_heads": hkv})["decode"] = {
                "us_per_call": round(g_ms * 1e3, 2), "kv_bytes": gkv, "GB_per_s": round(g_gbs, 1),
                "pct_hbm_peak": round(100 * g_gbs / PEAK_HBM_GBS, 2)}
            log(f"gqa decode {result['gqa']['decode']}")
            del gcaches
        del caches, kc0, vc0
        torch.cuda.empty_cache()

    # ---------------- prefill over a KV cache
    if not args.no_prefill:
        Bp, Tq, Tcp = 16, 512, 2048
        rng = np.random.default_rng(W.CONFIGS[W.DECODE].seed + 100)
        plens = rng.integers(0, Tcp - Tq + 1, size=Bp).astype(np.int32)
        pin = W.make_train_inputs(cfg, B=Bp, T=Tq)
        pq, pk, pv = (dev_t(x) for x in (pin.q_store, pin.k_store, pin.v_store))
        pkc = torch.zeros((Bp, Tcp, H, D), dtype=torch.bfloat16, device=dev)
        pvc = torch.zeros_like(pkc)
        pl = torch.from_numpy(plens).to(dev)
        po = torch.empty_like(pq)
        plse = torch.empty((Bp, H, Tq), dtype=torch.float32, device=dev)
        pev = ev.create(2)

        def pstep():
            st = lib.na_attn_prefill(ptr(pq), ptr(pk), ptr(pv), ptr(pkc), ptr(pvc), ptr(pl),
                                     ptr(po), ptr(plse), Bp, Tq, H, H, D, Tcp, -1, P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())

        ramp(pstep)
        for _ in range(args.warmup):
            pstep()
        torch.cuda.synchronize()
        ev.record(pev[0], stream)
        for _ in range(args.steps):
            pstep()
        ev.record(pev[1], stream)
        p_ms = ev.ms(pev[0], pev[1]) / args.steps
        pairs = int(sum(Tq * int(L) + Tq * (Tq + 1) // 2 for L in plens))
        pfl = 4 * D * H * pairs  # QK^T and PV, 2 FLOP per multiply-add
        # the same call with the QK-norm + rotary prologue folded in, and the
        # two-step path it replaces (prologue kernel, then the prefill)
        pct, pst = (torch.from_numpy(a).to(dev) for a in W.make_angle_tables(Tcp, D // 2, seed=3))
        pqr, pkr = torch.empty_like(pq), torch.empty_like(pk)
        peps = ctypes.c_float(1e-6)

        def prstep():
            st = lib.na_attn_prefill_rope(ptr(pq), ptr(pk), ptr(pv), ptr(pkc), ptr(pvc), ptr(pl),
                                          ptr(pct), ptr(pst), Tcp, peps, None, None, ptr(po),
                                          ptr(plse), Bp, Tq, H, H, D, Tcp, -1, P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())

        def p2step():
            st = lib.na_qk_norm_rope_fwd(ptr(pq), ptr(pk), ptr(pqr), ptr(pkr), ptr(pct), ptr(pst),
                                         ptr(pl), Bp, Tq, H, H, D, Tcp, peps, P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())
            st = lib.na_attn_prefill(ptr(pqr), ptr(pkr), ptr(pv), ptr(pkc), ptr(pvc), ptr(pl),
                                     ptr(po), ptr(plse), Bp, Tq, H, H, D, Tcp, -1, P(stream))
            if st:
                raise RuntimeError(lib.na_last_error().decode())

        rope_ms = {}
        for name, fn in (("fused", prstep), ("two_step", p2step)):
            ramp(fn)
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            ev.record(pev[0], stream)
            for _ in range(args.steps):
                fn()
            ev.record(pev[1], stream)
            torch.cuda.synchronize()
            rope_ms[name] = ev.ms(pev[0], pev[1]) / args.steps
        result["prefill"] = {
            "workload": f"prefill over a KV cache: B={Bp} chunks of {Tq} tokens, cache lengths "
                        f"U[0,{Tcp - Tq}], T_cap={Tcp}, H={H}, D={D}, bf16 (append + attention)",
            "ms_per_call": round(p_ms, 4), "TFLOP_per_s": round(pfl / (p_ms * 1e-3) / 1e12, 2),
            "visible_pairs": pairs, "calls": args.steps,
            "with_qk_norm_rope": {"fused_ms": round(rope_ms["fused"], 4),
                                  "two_step_ms": round(rope_ms["two_step"], 4)}}
        log(f"prefill {result['prefill']}")
        del pq, pk, pv, pkc, pvc, po, pqr, pkr

    # ---------------- CPU baseline: the oracle on a bounded sample
    if args.cpu_heads > 0:
        log(f"cpu baseline on {args.cpu_heads} heads")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_heads, dinp_cpu,
                                              64 if dinp_cpu is not None else 0)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
