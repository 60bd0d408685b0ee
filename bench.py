#!/usr/bin/env python3
"""Benchmark of the FP8 prefill matmul path on one MI355X.

Workload: the FFN of one prefill at M=2048 tokens (the headline shape: Q4_K
weights, K=3584):
  gate, up : K=3584,  N=18944, Q4_K, one shared FP8 activation quantisation
  down     : K=18944, N=3584,  Q6_K, input SiLU(g)*u
One step is one pass of the whole path over that batch: pack the three
weights (dequantise, absmax, E4M3 encode) in one call with one host wait for
their scales, quantise the FFN input once for gate and up, run gate and up
(one grouped launch), quantise the down input, run down.  Inputs are
synthetic (seeded), resident in HBM before timing.

value = GEMM FLOPs of the step (3 x 2*M*N*K) / measured step time, TFLOP/s.
roofline = the gate+up GEMM launch (one rz_fp8_gemm_group call, 2 x 2*M*N*K
per launch) timed with HIP events on its stream during the timed steps (the
only markers in the timed loop, around that launch on every 4th step),
against the 5.0 PFLOP/s dense FP8 peak; traffic and mfma_counters come from
the committed counter runs of the same kernel (profiles/, null once the
kernel's sources differ from the ones measured); clock = the GFX clock and
board power read from the GPU's metrics (amdsmi, read only) during a 3.5 s
untimed run of the same steps after the timed ones (the firmware refreshes
those values once a second; the readings from 1.05 s on), and the gate+up
rate against the FP8 peak scaled to that clock.  Before the warm-up steps
the step runs untimed for --clock-settle seconds (0.15): from idle the GPU
raises its clock over tens of milliseconds, and a few warm-up steps would
time that ramp instead of the sustained rate.  phases_us comes from a
second, untimed pass of the same steps with markers between all phases.
cpu_baseline = the CPU oracle on a bounded sample of the same workload (see
--help).

Prints one JSON line on stdout; diagnostics go to stderr.

--pack-model instead times the weight packing of the 28-layer 7B-class model
sweep (Q/K/V/O 3584/512/512/3584, gate/up 18944 at K=3584, down 3584 at
K=18944; V and down Q6_K, the rest Q4_K; 196 weights, 4.17 GB of K-quant
blocks -> 6.53 GB of E4M3 codes) after a 1 GiB write that evicts the caches:
all 196 weights in one rz_fp8_pack_weights call, and, for comparison, 196
rz_fp8_pack_weight calls back to back; it prints that measurement's own line.

--gemm-shapes instead times the FP8 GEMM alone at every configuration's
shapes (warm, random E4M3 codes) and the 28-layer M=4096 sweep from them.

--small-m instead times the small-batch routes (GEMV straight from K-quant
blocks, FP8 GEMM, activation quantisation + FP8 GEMM) at N=4608, K=3584.

--fp16-gemm instead times the FP16 cached-weight comparator (fp16 weight
cache, fp16 activation, fp16 MFMA GEMM) beside the FP8 path on the FFN
shapes at M=2048, with both paths' accuracy on the gate GEMM.

--q8-gemm instead times the integer path (Q8_1 activation blocks x Q4_K
weight on the int8 matrix cores) beside the FP8 path, with both paths'
accuracy on the gate GEMM.

--kquant-gemm instead times the FP8 GEMM that encodes the weight from its
K-quant blocks inside the kernel (no FP8 weight cache) beside the cached
path's GEMM, at the model's prefill shapes (warm).

--gemm-clock instead runs the gate+up GEMM launch back to back for a few
seconds each with random E4M3 codes, with constant codes (every product 1.0)
and with random codes again, and reports per phase the launch time, the GFX
clock and board power read from the GPU's metrics meanwhile (amdsmi, read
only; the values change once a second): the clock the MFMA load leaves the
kernel, and its rate at that clock.

--hbm-rates instead times torch's own device kernels on 1 GiB (a max and a
sum that only read, a copy, a fill that only writes), cold (after a 1 GiB
write) and warm, and a 155 MB max right after a 310 MB write (the down
input's absmax after the gate+up GEMM's output): the rates plain kernels
reach on this GPU, beside the 8 TB/s peak the HBM-bound phases are priced
against.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 prefill GEMM TFLOP/s & % FP8 MFMA peak (Q4_K w, M=2048, K=3584)"
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA (at 2.4 GHz)
# per-shape modes: the mean over TIMED_LAUNCHES launches back to back between
# two events (markers between launches would add their own gaps), after
# WARM_LAUNCHES untimed ones; the kernel traces of the same runs give the
# per-launch medians
WARM_LAUNCHES, TIMED_LAUNCHES = 10, 50
CLOCK_PASS_S = 3.5  # seconds of the untimed clock pass (2-3 refreshes of the GPU's metrics after its first second)
HBM_PEAK_TBPS = 8.0  # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")
CLOCK_FILE = os.path.join(ROOT, "profiles", "gemm_clock.json")
KGEMV_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kgemv_traffic.json")
KGEMV_SOURCES = [os.path.join(ROOT, "fp8_prefill_gemm_amd", "csrc", f) for f in ("kgemv.hip", "rz_device.h")]
KERNEL_SOURCES = [os.path.join(ROOT, "fp8_prefill_gemm_amd", "csrc", f)
                  for f in ("gemm.hip", "gemm_common.h", "rz_gemm.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(path=None, sources=None):
    """HBM bytes per launch of the roofline kernel from the committed counter
    runs, or None when they are absent or were taken on a different kernel
    source."""
    try:
        with open(path or TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    return rec.get("bytes_per_launch")


def measured_clock(path=None, sources=None):
    """Sustained core clock and MFMA utilisation of the roofline kernel from
    the committed counter run (GRBM_GUI_ACTIVE per XCD over the launch,
    SQ_VALU_MFMA_BUSY_CYCLES per SIMD), with the fraction of the FP8 peak at
    that clock; None when absent or taken on a different kernel source."""
    try:
        with open(path or CLOCK_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    mhz = float(rec["clock_mhz"])
    return {"mhz": mhz, "mfma_busy_of_active": rec["mfma_busy_of_active"], "launch_us": rec["launch_us"],
            "tflops": rec["tflops"], "frac_at_clock": round(rec["tflops"] / (FP8_PEAK_TFLOPS * mhz / 2400.0), 4),
            "source": rec.get("source")}


class GpuMetrics:
    """GFX clock and board power read every ~5 ms by a thread of this process
    (amdsmi, read only: the calls torch's own clock_rate and power_draw make
    on ROCm) between start() and close().  The values themselves change once
    a second (the firmware's refresh), so a window needs seconds to hold a
    few of them."""

    def __init__(self, device_index=0):
        import threading
        self.samples = []
        self._thread = None
        self.error = None
        self.power_cap_w = None
        self._stop = threading.Event()
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            if len(hs) != 1:
                raise RuntimeError(f"{len(hs)} GPUs visible, cannot tell which one is measured")
            self._h = hs[device_index]
            self._smi = amdsmi
            cap = amdsmi.amdsmi_get_power_cap_info(self._h).get("power_cap")
            self.power_cap_w = cap / 1e6 if isinstance(cap, int) and cap > 0 else None
        except Exception as e:  # no amdsmi, or no permission: no clock in the line
            self.error = repr(e)
        self._thread = None

    def start(self):
        import threading
        if self.error is None and self._thread is None:
            self._stop.clear()
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def _run(self):
        smi, h = self._smi, self._h
        while not self._stop.is_set():
            try:
                mhz = smi.amdsmi_get_clock_info(h, smi.AmdSmiClkType.GFX).get("clk")
                w = smi.amdsmi_get_power_info(h).get("current_socket_power")
            except Exception as e:
                self.error = repr(e)
                return
            self.samples.append((time.monotonic(), mhz if isinstance(mhz, (int, float)) and 0 < mhz < 10000 else None,
                                 w if isinstance(w, (int, float)) and 0 < w < 10000 else None))
            self._stop.wait(0.005)

    def window(self, t0, t1):
        """Mean clock and power over the samples taken in [t0, t1] (time.monotonic())."""
        sel = [x for x in list(self.samples) if t0 <= x[0] <= t1]
        mhz = [x[1] for x in sel if x[1]]
        w = [x[2] for x in sel if x[2]]
        if not mhz:
            return {"error": self.error or "no samples in the window"}
        readings = [x[1:] for i, x in enumerate(sel) if i == 0 or x[1:] != sel[i - 1][1:]]
        return {"gfxclk_mhz": round(sum(mhz) / len(mhz), 1), "gfxclk_mhz_min": round(min(mhz), 1),
                "socket_power_w": round(sum(w) / len(w), 1) if w else None, "power_cap_w": self.power_cap_w,
                "samples": len(sel), "readings": len(readings),
                "readings_mhz_w": [[r[0], r[1]] for r in readings[:8]],
                "source": "amdsmi GFX clock and socket power, read every ~5 ms (the values change once a second)"}

    def close(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=5)
            self._thread = None


def at_clock(tflops, sample, key="gfxclk_mhz"):
    """The rate against the FP8 peak scaled from 2.4 GHz to the measured clock."""
    if not sample or key not in sample:
        return sample
    out = dict(sample)
    out["frac_at_clock"] = round(tflops / (FP8_PEAK_TFLOPS * sample[key] / 2400.0), 4)
    return out


def gemm_clock(args, dev, metrics) -> int:
    """The gate+up launch back to back with random and with constant codes,
    clock and power sampled meanwhile (one line)."""
    import torch

    import fp8_prefill_gemm_amd as rz

    m, k, n = 2048, 3584, 18944
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator().manual_seed(20260)

    def codes(shape):  # E4M3 codes except the NaN codes 0x7F / 0xFF
        a = torch.randint(0, 0x7F, shape, generator=g, dtype=torch.int32)
        sgn = torch.randint(0, 2, shape, generator=g, dtype=torch.int32) << 7
        return (a | sgn).to(torch.uint8).to(dev)

    if metrics is not None:
        metrics.start()
    a, w1, w2 = codes((m, k)), codes((n, k)), codes((n, k))
    one_a = torch.full((m, k), 0x38, dtype=torch.uint8, device=dev)  # 1.0
    one_w = torch.full((n, k), 0x38, dtype=torch.uint8, device=dev)
    sc = torch.tensor([1.0, 0.013, 0, 0], dtype=torch.float32, device=dev)
    ys = [torch.empty((m, n), dtype=torch.float32, device=dev) for _ in range(2)]
    flop = 2.0 * m * 2 * n * k
    rows = {}
    for name, fn in (("random codes", lambda: rz.rz_fp8_gemm_group(a, m, sc, [(w1, 0.007), (w2, 0.008)], ys, stream)),
                     ("constant codes", lambda: rz.rz_fp8_gemm_group(one_a, m, sc, [(one_w, 0.007), (one_w, 0.008)],
                                                                    ys, stream)),
                     ("random codes again", lambda: rz.rz_fp8_gemm_group(a, m, sc, [(w1, 0.007), (w2, 0.008)], ys,
                                                                        stream))):
        time.sleep(1.0)  # idle: the clock and power settle back
        for _ in range(200):  # 50 ms: the clock reaches its steady state under the load
            fn()
        torch.cuda.synchronize()
        t0 = time.monotonic()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launches, busy_ms = 0, 0.0
        while time.monotonic() - t0 < args.clock_seconds:
            for _ in range(50):
                fn()
            launches += 50
            e1.record(stream)
            e1.synchronize()
            busy_ms += e0.elapsed_time(e1)
            e0.record(stream)
        t1 = time.monotonic()
        us = busy_ms * 1e3 / launches
        tf = flop / (us * 1e-6) / 1e12
        rows[name] = at_clock(tf, metrics.window(t0 + 0.3, t1) if metrics else None) or {}
        rows[name].update({"launch_us": round(us, 1), "tflops": round(tf, 1), "frac": round(tf / FP8_PEAK_TFLOPS, 4),
                           "launches": launches})
        log(f"{name}: {rows[name]}")
    print(json.dumps({"metric": "gate+up FP8 GEMM launch back to back: GFX clock, board power and rate",
                      "unit": "TFLOP/s", "higher_is_better": True, "peak": FP8_PEAK_TFLOPS, "rows": rows,
                      "data": "synthetic",
                      "config": {"workload": "M=2048, N=2x18944, K=3584 in one rz_fp8_gemm_group launch; random E4M3 "
                                             "codes (NaN codes excluded) or every code 0x38 (1.0)"}}), flush=True)
    return 0


def cpu_baseline(x_ffn, x_down, gate_blocks, down_blocks, gate, dn, m_rows=128):
    """Time the oracle on a bounded sample of the step: pack the gate and down
    weights, quantise both inputs, compute m_rows output rows of the gate and
    down GEMMs."""
    import numpy as np
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:
        host_cores = os.cpu_count() or 1
    # the GPU machine's CPU share is 16 threads per GPU whatever the affinity
    # mask shows; BLAS gets all of that share
    threads = max(1, min(host_cores, 16))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=threads, user_api="blas")
    except Exception:  # pragma: no cover - threadpoolctl missing
        limiter = None
    from oracle import fp8_path
    t = [time.perf_counter()]
    wg8, dq_g, _ = fp8_path.pack_weight(gate.qtype, gate_blocks, gate.n, gate.k)
    t.append(time.perf_counter())
    wd8, dq_d, _ = fp8_path.pack_weight(dn.qtype, down_blocks, dn.n, dn.k)
    t.append(time.perf_counter())
    a8, _, dq_a = fp8_path.quant_act(x_ffn)
    d8, _, dq_x = fp8_path.quant_act(x_down)
    t.append(time.perf_counter())
    rows = np.linspace(0, x_ffn.shape[0] - 1, m_rows).astype(np.int64)
    fp8_path.gemm_rows(a8, wg8, rows, dq_a, dq_g)
    fp8_path.gemm_rows(d8, wd8, rows, dq_x, dq_d)
    t.append(time.perf_counter())
    if limiter is not None:
        limiter.restore_original_limits()
    flops = 2.0 * m_rows * (gate.n * gate.k + dn.n * dn.k)
    total = t[-1] - t[0]
    log(f"cpu oracle: pack gate {t[1] - t[0]:.2f}s pack down {t[2] - t[1]:.2f}s quant {t[3] - t[2]:.2f}s "
        f"gemm({m_rows} rows x2) {t[4] - t[3]:.2f}s")
    return {
        "value": flops / total / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "host_cores": host_cores,
        "kind": "oracle",
        "sample": (f"oracle (numpy) on a slice of the same step: pack the full {gate.n}x{gate.k} Q4_K gate "
                   f"weight ({t[1] - t[0]:.2f}s) and {dn.n}x{dn.k} Q6_K down weight ({t[2] - t[1]:.2f}s), "
                   f"quantise both full inputs ({t[3] - t[2]:.2f}s), exact gate and down GEMMs for {m_rows} of "
                   f"{x_ffn.shape[0]} output rows ({t[4] - t[3]:.2f}s); value = those rows' 2*m*N*K FLOPs / "
                   f"total time ({total:.1f}s); cores = BLAS threads = the box's CPU share per GPU "
                   f"(16), of {host_cores} cores in the affinity mask"),
    }


def pack_model(args, dev) -> int:
    """Cold-cache packing of every weight of the 28-layer sweep (one line)."""
    import numpy as np
    import torch

    import fp8_prefill_gemm_amd as rz
    import workloads as W

    weights = []  # (name, qtype, n, k, blocks on the device, fp8 output)
    t0 = time.time()
    for layer in range(W.CFG4_LAYERS):
        for grp in W.config_groups(4, layer=layer):
            for g in grp.gemms:
                blocks = torch.from_numpy(W.weight_blocks(g.qtype, g.w_seed, g.n, g.k)).to(dev)
                w8 = torch.empty((g.n, g.k), dtype=torch.uint8, device=dev)
                weights.append((f"{layer}.{g.name}", g.qtype, g.n, g.k, blocks, w8))
        log(f"layer {layer}: {len(weights)} weights resident ({time.time() - t0:.1f} s)")
    kq_bytes = sum(b.numel() for _, _, _, _, b, _ in weights)
    fp8_bytes = sum(n * k for _, _, n, k, _, _ in weights)
    alg_bytes = 2 * kq_bytes + fp8_bytes  # blocks read twice (absmax, encode), codes written once
    ws = rz.workspace(dev)
    stream = torch.cuda.current_stream(dev)
    evict = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    batch = [(qt, blocks, n, k, w8) for _, qt, n, k, blocks, w8 in weights]

    def cold_pass(r, batched):
        evict.fill_(float(r + 1))  # 1 GiB written: the 256 MB MALL and the L2s hold none of the blocks
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if batched:
            rz.rz_fp8_pack_weights(batch, ws, stream)
        else:
            for qt, blocks, n, k, w8 in batch:
                rz.rz_fp8_pack_weight(qt, blocks, n, k, w8, ws, stream)
        e1.record(stream)
        e1.synchronize()
        t = e0.elapsed_time(e1) * 1e-3
        log(f"pass {r} ({'one call' if batched else '196 calls'}): {t * 1e3:.3f} ms, {alg_bytes / t / 1e9:.0f} GB/s")
        return t

    times = [cold_pass(r, True) for r in range(max(1, args.pack_repeats))]
    single = [cold_pass(r, False) for r in range(max(1, args.pack_repeats))]
    t = sorted(times)[len(times) // 2]
    ts = sorted(single)[len(single) // 2]
    out = {"metric": "FP8 weight pack of the 28-layer sweep (196 weights in one call, cold cache)",
           "value": round(alg_bytes / t / 1e9, 1), "unit": "GB/s", "higher_is_better": True,
           "ms": round(t * 1e3, 3), "ms_per_pass": [round(x * 1e3, 3) for x in times],
           "ms_196_single_calls": round(ts * 1e3, 3),
           "algorithmic_bytes": alg_bytes, "kquant_bytes": kq_bytes, "fp8_bytes": fp8_bytes,
           "hbm_frac": round(alg_bytes / t / 1e12 / HBM_PEAK_TBPS, 4), "weights": len(weights),
           "data": "synthetic", "config": {"workload": "28 layers x {q,k,v,o,gate,up,down} at hidden 3584, "
                                                    "kv 512, FFN 18944; v and down Q6_K, the rest Q4_K"}}
    print(json.dumps(out), flush=True)
    return 0


def hbm_rates(args, dev) -> int:
    """Rates of torch's own read, copy and write kernels (one line; median of
    9 runs each, HIP events around one launch)."""
    import torch

    n = 1 << 28  # 1 GiB of fp32
    x = torch.empty(n, dtype=torch.float32, device=dev).normal_()
    y = torch.empty_like(x)
    evict = torch.empty_like(x)

    def timed(fn, cold, before=None):
        ts = []
        for _ in range(9):
            if cold:
                evict.fill_(1.0)  # 1 GiB written: the L2s and the 256 MB MALL hold none of x
            if before is not None:
                before()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return sorted(ts)[len(ts) // 2]

    for _ in range(20):
        y.copy_(x)
    torch.cuda.synchronize()
    gib = n * 4
    rows = {}
    for name, fn, byts in (("amax (read)", lambda: torch.amax(x), gib), ("sum (read)", lambda: x.sum(), gib),
                           ("copy (read + write)", lambda: y.copy_(x), 2 * gib),
                           ("fill (write)", lambda: y.fill_(2.0), gib)):
        for cold in (True, False):
            t = timed(fn, cold)
            rows[f"{name}, {'cold' if cold else 'warm'}"] = {"us": round(t * 1e6, 1),
                                                           "tb_per_s": round(byts / t / 1e12, 2)}
    a = x[:2048 * 18944]
    out = y[:2048 * 37888]
    t = timed(lambda: torch.amax(a), False, before=lambda: out.fill_(3.0))
    rows["amax of 155 MB after a 310 MB write"] = {"us": round(t * 1e6, 1),
                                                   "tb_per_s": round(a.numel() * 4 / t / 1e12, 2)}
    for k, v in rows.items():
        log(f"{k}: {v}")
    print(json.dumps({"metric": "HBM rates of plain device kernels (torch), 1 GiB", "unit": "TB/s",
                      "higher_is_better": True, "peak_tb_per_s": HBM_PEAK_TBPS, "rows": rows,
                      "data": "synthetic", "config": {"workload": "1 GiB fp32 tensors; 155 MB / 310 MB FFN sizes"}}),
          flush=True)
    return 0


def small_m(args, dev) -> int:
    """Small batches at K=3584, N=4608, Q4_K (one line): the GEMV straight from
    the K-quant blocks against the FP8 path (activation quantisation + FP8
    GEMM on the packed weight), warm, HIP events around 200 launches each."""
    import numpy as np
    import torch

    import fp8_prefill_gemm_amd as rz
    import workloads as W

    n, k, reps = 4608, 3584, 200
    stream = torch.cuda.current_stream(dev)
    blocks = torch.from_numpy(W.weight_blocks(W.Q4_K, W.seed_for(5, 0, "up"), n, k)).to(dev)
    w8 = torch.empty((n, k), dtype=torch.uint8, device=dev)
    ws = rz.workspace(dev)
    _, w_scale, _ = rz.rz_fp8_pack_weight(W.Q4_K, blocks, n, k, w8, ws, stream)
    kq_bytes = blocks.numel()

    def timed(fn):
        for _ in range(10):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    rows = {}
    for m in args.small_m:
        x = torch.from_numpy(W.act_student_t(W.seed_for(5, 0, "x_ffn") + m, m, k)).to(dev)
        a8 = torch.empty((rz.rz_pad_m(m), k), dtype=torch.uint8, device=dev)
        sc = torch.empty(2, dtype=torch.float32, device=dev)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        row = {}
        if m <= rz.KGEMV_MAX_M:
            t = timed(lambda: rz.rz_kquant_gemv(W.Q4_K, blocks, n, k, x, y, stream))
            b = kq_bytes + 4 * m * k + 4 * m * n
            row["kquant_gemv"] = {"us": round(t * 1e6, 2), "bytes": b, "gb_s": round(b / t / 1e9, 1),
                                  "hbm_frac": round(b / t / 1e12 / HBM_PEAK_TBPS, 4)}
        rz.rz_fp8_quant_act(x, a8, sc, ws, stream)
        t = timed(lambda: rz.rz_fp8_gemm(a8, w8, m, sc, w_scale, y, stream))
        b = n * k + rz.rz_pad_m(m) * k + 4 * m * n
        row["fp8_gemm"] = {"us": round(t * 1e6, 2), "bytes": b, "gb_s": round(b / t / 1e9, 1)}
        t = timed(lambda: (rz.rz_fp8_quant_act(x, a8, sc, ws, stream),
                           rz.rz_fp8_gemm(a8, w8, m, sc, w_scale, y, stream)))
        row["fp8_quant_plus_gemm_us"] = round(t * 1e6, 2)
        rows[str(m)] = row
        log(f"m={m}: {row}")
    # the down projection's Q6_K weight (N=3584, K=18944) at the same batch sizes
    nd, kd = 3584, 18944
    dblocks = torch.from_numpy(W.weight_blocks(W.Q6_K, W.seed_for(3, 0, "down"), nd, kd)).to(dev)
    q6 = {}
    for m in args.small_m:
        if m > rz.KGEMV_MAX_M:
            continue
        x = torch.from_numpy(W.act_silu_gated(W.seed_for(3, 0, "x_down") + m, m, kd)).to(dev)
        y = torch.empty((m, nd), dtype=torch.float32, device=dev)
        t = timed(lambda: rz.rz_kquant_gemv(W.Q6_K, dblocks, nd, kd, x, y, stream))
        b = dblocks.numel() + 4 * m * kd + 4 * m * nd
        q6[str(m)] = {"us": round(t * 1e6, 2), "bytes": b, "gb_s": round(b / t / 1e9, 1),
                      "hbm_frac": round(b / t / 1e12 / HBM_PEAK_TBPS, 4)}
        log(f"q6k down m={m}: {q6[str(m)]}")
    roof = None
    if "1" in rows and "kquant_gemv" in rows["1"]:
        r1 = rows["1"]["kquant_gemv"]
        roof = {"kernel": "K-quant GEMV at m=1 (N=4608, K=3584, Q4_K), per-call event time over 200 launches",
                "bound": "hbm", "achieved": r1["gb_s"], "peak": HBM_PEAK_TBPS * 1e3, "unit": "GB/s",
                "frac": round(r1["gb_s"] / (HBM_PEAK_TBPS * 1e3), 4),
                "traffic": measured_traffic(KGEMV_TRAFFIC_FILE, KGEMV_SOURCES)}
    out = {"metric": "small-batch matmul at K=3584, N=4608, Q4_K weight (warm)", "unit": "us",
           "roofline": roof,
           "kquant_gemv_q6k_down_n3584_k18944": q6,
           "higher_is_better": False, "rows": rows, "kquant_bytes": kq_bytes, "data": "synthetic",
           "config": {"workload": "edge configuration: N=4608, K=3584, Q4_K; Student-t(3) activations "
                                  "with 8 channels x100", "m": list(args.small_m)}}
    print(json.dumps(out), flush=True)
    return 0


def gemm_shapes(args, dev) -> int:
    """Warm FP8 GEMM time per shape of the five configurations (one line):
    random E4M3 codes (no NaN codes), scales 1, the library's default
    workspace, HIP events around 50 launches after 10 warm-up launches.  Also
    the 28-layer sweep at M=4096 (7 GEMMs per layer, 53.46 TFLOP) from the
    per-shape times."""
    import torch

    import fp8_prefill_gemm_amd as rz

    H, KV, F = 3584, 512, 18944
    shapes = [("cfg1", 16, 256, 512), ("cfg2 q", 512, H, H), ("cfg2 k/v", 512, KV, H),
              ("cfg3 gate/up", 2048, F, H), ("cfg3 down", 2048, H, F),
              ("cfg4 q/o", 4096, H, H), ("cfg4 k/v", 4096, KV, H), ("cfg4 gate/up", 4096, F, H),
              ("cfg4 down", 4096, H, F), ("cfg5 m=1", 1, 4608, H), ("cfg5 m=4", 4, 4608, H),
              ("cfg5 m=37", 37, 4608, H), ("cfg5 m=1000", 1000, 4608, H)]
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(5)

    def codes(rows, cols):
        c = torch.randint(0, 256, (rows, cols), dtype=torch.int32, device=dev, generator=g)
        c = torch.where((c & 0x7F) == 0x7F, c - 1, c)  # 0x7F / 0xFF are E4M3FN NaN codes
        return c.to(torch.uint8)

    sc = torch.ones(2, dtype=torch.float32, device=dev)
    rows = {}
    for name, m, n, k in shapes:
        a = codes(rz.rz_pad_m(m), k)
        w = codes(n, k)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        for _ in range(WARM_LAUNCHES):
            rz.rz_fp8_gemm(a, w, m, sc, 1.0, y, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(TIMED_LAUNCHES):
            rz.rz_fp8_gemm(a, w, m, sc, 1.0, y, stream)
        e1.record(stream)
        e1.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / TIMED_LAUNCHES
        plan = rz.rz_fp8_gemm_plan(m, n, k)
        byts = n * k + rz.rz_pad_m(m) * k + 4 * m * n
        rows[name] = {"m": m, "n": n, "k": k, "us": round(t * 1e6, 2),
                      "tflops": round(2.0 * m * n * k / t / 1e12, 1), "gb_s": round(byts / t / 1e9, 1),
                      "plan": {"bn": plan[0], "bm": plan[1], "threads": plan[2], "workgroups": plan[3]}}
        log(f"{name}: {rows[name]}")
        del a, w, y
    # GEMMs that share an activation, in one rz_fp8_gemm_group launch
    groups = [("cfg3 gate+up grouped", 2048, (F, F), H), ("cfg4 q+k+v grouped", 4096, (H, KV, KV), H),
              ("cfg4 gate+up grouped", 4096, (F, F), H)]
    for name, m, ns, k in groups:
        a = codes(rz.rz_pad_m(m), k)
        ws_ = [(codes(n, k), 1.0) for n in ns]
        ys = [torch.empty((m, n), dtype=torch.float32, device=dev) for n in ns]
        for _ in range(WARM_LAUNCHES):
            rz.rz_fp8_gemm_group(a, m, sc, ws_, ys, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(TIMED_LAUNCHES):
            rz.rz_fp8_gemm_group(a, m, sc, ws_, ys, stream)
        e1.record(stream)
        e1.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / TIMED_LAUNCHES
        plan = rz.rz_fp8_gemm_plan(m, sum(ns), k)
        rows[name] = {"m": m, "n": list(ns), "k": k, "us": round(t * 1e6, 2),
                      "tflops": round(2.0 * m * sum(ns) * k / t / 1e12, 1),
                      "plan": {"bn": plan[0], "bm": plan[1], "threads": plan[2], "workgroups": plan[3]}}
        log(f"{name}: {rows[name]}")
        del a, ws_, ys
    per_layer = sum(rows[nm]["us"] * c for nm, c in (("cfg4 q/o", 2), ("cfg4 k/v", 2), ("cfg4 gate/up", 2),
                                                       ("cfg4 down", 1))) * 1e-6
    per_layer_grouped = sum(rows[nm]["us"] for nm in ("cfg4 q+k+v grouped", "cfg4 q/o", "cfg4 gate+up grouped",
                                                       "cfg4 down")) * 1e-6
    sweep_flop = 28 * 2.0 * 4096 * (2 * H * H + 2 * KV * H + 2 * F * H + H * F)
    out = {"metric": "FP8 GEMM per shape (warm, random E4M3 codes)", "unit": "us", "higher_is_better": False,
           "rows": rows, "sweep_28_layers_m4096": {"ms": round(28 * per_layer * 1e3, 3),
                                                   "tflop": round(sweep_flop / 1e12, 2),
                                                   "tflops": round(sweep_flop / (28 * per_layer) / 1e12, 1)},
           "sweep_28_layers_m4096_grouped": {"ms": round(28 * per_layer_grouped * 1e3, 3),
                                             "tflops": round(sweep_flop / (28 * per_layer_grouped) / 1e12, 1),
                                             "note": "q+k+v and gate+up as one launch each, o and down alone"},
           "data": "synthetic", "config": {"workload": "GEMM shapes of the five configurations"}}
    print(json.dumps(out), flush=True)
    return 0


def kquant_gemm(args, dev) -> int:
    """Warm time of the FP8 GEMM that makes the weight codes from the K-quant
    blocks in the kernel (rz_kquant_fp8_gemm), beside the cached path's GEMM
    on the packed weight (rz_fp8_gemm), per prefill shape of the 7B-class
    model (one line): seeded K-quant blocks and activations, HIP events
    around 50 launches after 10 warm-up launches.  Also the one-pass weight
    scale (rz_kquant_weight_scale, including its host wait) and the weight
    bytes each path keeps resident for the 28-layer model."""
    import torch

    import fp8_prefill_gemm_amd as rz
    import workloads as W

    H, KV, F, L = 3584, 512, 18944, 28
    shapes = [("cfg2 q", 512, W.Q4_K, H, H), ("cfg3 gate/up", 2048, W.Q4_K, F, H),
              ("cfg3 down", 2048, W.Q6_K, H, F), ("cfg4 q/o", 4096, W.Q4_K, H, H),
              ("cfg4 k/v", 4096, W.Q4_K, KV, H), ("cfg4 gate/up", 4096, W.Q4_K, F, H),
              ("cfg4 down", 4096, W.Q6_K, H, F)]
    stream = torch.cuda.current_stream(dev)

    def timed(fn, reps=TIMED_LAUNCHES):
        for _ in range(WARM_LAUNCHES):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    rows = {}
    for name, m, qt, n, k in shapes:
        blocks = torch.from_numpy(W.weight_blocks(qt, 31 + n, n, k)).to(dev)
        a8, sc = rz.rz_fp8_quant_act(torch.from_numpy(W.act_student_t(32 + m, m, k)).to(dev), stream=stream)
        q, dq, _ = rz.rz_kquant_weight_scale(qt, blocks, n, k, stream=stream)
        w8, scale, _ = rz.rz_fp8_pack_weight(qt, blocks, n, k, stream=stream)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        tf = timed(lambda: rz.rz_kquant_fp8_gemm(a8, m, sc, qt, blocks, n, k, q, dq, y, stream))
        tc = timed(lambda: rz.rz_fp8_gemm(a8, w8, m, sc, scale, y, stream))
        t0 = time.perf_counter()
        for _ in range(5):
            rz.rz_kquant_weight_scale(qt, blocks, n, k, stream=stream)
        ts = (time.perf_counter() - t0) / 5
        fl = 2.0 * m * n * k
        rows[name] = {"m": m, "n": n, "k": k, "qtype": "Q4_K" if qt == W.Q4_K else "Q6_K",
                      "fused_us": round(tf * 1e6, 1), "fused_tflops": round(fl / tf / 1e12, 1),
                      "cached_us": round(tc * 1e6, 1), "cached_tflops": round(fl / tc / 1e12, 1),
                      "weight_scale_us": round(ts * 1e6, 1)}
        log(f"{name}: {rows[name]}")
        del blocks, a8, w8, y
    per_layer = {"q/o": (2, W.Q4_K, H, H), "k/v": (2, W.Q4_K, KV, H), "gate/up": (2, W.Q4_K, F, H),
                 "down": (1, W.Q6_K, H, F)}
    kq = sum(c * rz.rz_weight_bytes(qt, n, k) for c, qt, n, k in per_layer.values()) * L
    f8 = sum(c * n * k for c, _, n, k in per_layer.values()) * L
    g = rows["cfg3 gate/up"]
    ach = 2.0 * g["m"] * g["n"] * g["k"] / (g["fused_us"] * 1e-6) / 1e12
    roof = {"kernel": "kq_fp8_gemm_kernel<Q4_K, 256-row tiles> (M=2048, N=18944, K=3584)", "bound": "mfma",
            "achieved": round(ach, 1), "peak": 5000.0, "unit": "TFLOP/s", "frac": round(ach / 5000.0, 4),
            "traffic": None}
    out = {"metric": "FP8 GEMM from K-quant blocks vs cached FP8 weight (warm)", "unit": "us",
           "higher_is_better": False, "rows": rows, "roofline": roof,
           "resident_weight_bytes_28_layers": {"kquant_only": kq, "kquant_plus_fp8_cache": kq + f8},
           "data": "synthetic", "config": {"workload": "prefill GEMM shapes of the 7B-class model"}}
    print(json.dumps(out), flush=True)
    return 0


def fp16_gemm(args, dev) -> int:
    """The FP16 comparator (cached fp16 weight, fp16 activation, fp16 MFMA
    GEMM with fp32 accumulation) beside the FP8 path on the FFN shapes at
    M=2048 (one line): warm GEMM times (HIP events around 50 launches after
    10 warm-up launches), the one-off weight conversion and the per-input
    activation conversion, the resident weight bytes, and the accuracy of
    both paths' gate outputs on 64 rows against a float64 product of the
    fp32 activation and the fp32 dequantised weight (computed here with
    torch in float64 on the GPU from rz_dequant_f32)."""
    import numpy as np
    import torch

    import fp8_prefill_gemm_amd as rz
    import workloads as W

    ffn, down = W.config_groups(3)
    stream = torch.cuda.current_stream(dev)

    def timed(fn, reps=TIMED_LAUNCHES):
        for _ in range(WARM_LAUNCHES):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    rows, acc = {}, {}
    for grp in (ffn, down):
        x = torch.from_numpy(grp.activation()).to(dev)
        m = grp.m
        a16 = rz.rz_fp16_convert_act(x, stream=stream)
        a8, sc = rz.rz_fp8_quant_act(x, stream=stream)
        t_cvt16 = timed(lambda: rz.rz_fp16_convert_act(x, a16, stream))
        t_q8 = timed(lambda: rz.rz_fp8_quant_act(x, a8, sc, stream=stream))
        for gm in grp.gemms:
            blocks = torch.from_numpy(W.weight_blocks(gm.qtype, gm.w_seed, gm.n, gm.k)).to(dev)
            w16 = rz.rz_fp16_pack_weight(gm.qtype, blocks, gm.n, gm.k, stream=stream)
            w8, scale, _ = rz.rz_fp8_pack_weight(gm.qtype, blocks, gm.n, gm.k, stream=stream)
            t_pack16 = timed(lambda: rz.rz_fp16_pack_weight(gm.qtype, blocks, gm.n, gm.k, w16, stream), reps=5)
            y16 = torch.empty((m, gm.n), dtype=torch.float32, device=dev)
            y8 = torch.empty((m, gm.n), dtype=torch.float32, device=dev)
            t16 = timed(lambda: rz.rz_fp16_gemm(a16, w16, m, y16, stream))
            t8 = timed(lambda: rz.rz_fp8_gemm(a8, w8, m, sc, scale, y8, stream))
            fl = 2.0 * m * gm.n * gm.k
            rows[gm.name] = {"m": m, "n": gm.n, "k": gm.k,
                             "fp16_gemm_us": round(t16 * 1e6, 1), "fp16_tflops": round(fl / t16 / 1e12, 1),
                             "fp8_gemm_us": round(t8 * 1e6, 1), "fp8_tflops": round(fl / t8 / 1e12, 1),
                             "fp16_weight_convert_us": round(t_pack16 * 1e6, 1),
                             "act_convert_us": {"fp16": round(t_cvt16 * 1e6, 1), "fp8": round(t_q8 * 1e6, 1)},
                             "weight_bytes": {"fp16": 2 * gm.n * gm.k, "fp8": gm.n * gm.k,
                                              "kquant": int(blocks.numel())}}
            log(f"{gm.name}: {rows[gm.name]}")
            if gm.name == "gate":
                wf = rz.rz_dequant_f32(gm.qtype, blocks, gm.n, gm.k, stream=stream)
                sel = torch.linspace(0, m - 1, 64, device=dev).long()
                ref = x[sel].double() @ wf.double().t()
                den = ref.abs().mean().item()
                for name, yy in (("fp16", y16), ("fp8", y8)):
                    e = (yy[sel].double() - ref).abs()
                    acc[name] = {"mean_abs_err_rel": round(e.mean().item() / den, 6),
                                 "max_abs_err_rel": round(e.max().item() / den, 6)}
                del wf, ref
            del blocks, w16, w8, y16, y8
        del x, a16, a8
    g = rows["gate"]
    ach = 2.0 * g["m"] * g["n"] * g["k"] / (g["fp16_gemm_us"] * 1e-6) / 1e12
    plan = rz.rz_fp8_gemm_plan(g["m"], g["n"], 2 * g["k"])
    roof = {"kernel": f"fp8_gemm_interior_kernel<fp16 operands>, {plan[0]}x{plan[1]} tiles, {plan[3]} persistent workgroups "
                      "(M=2048, N=18944, K=3584)",
            "bound": "mfma", "achieved": round(ach, 1), "peak": 2500.0, "unit": "TFLOP/s",
            "frac": round(ach / 2500.0, 4), "traffic": None}
    out = {"metric": "FP16 cached-weight GEMM vs FP8 GEMM, FFN at M=2048 (warm)", "unit": "us",
           "higher_is_better": False, "rows": rows, "roofline": roof,
           "gate_accuracy_vs_fp64_of_fp32_inputs": acc,
           "dtype": "fp16 (fp32 accumulate) vs fp8_e4m3 (fp32 accumulate)", "data": "synthetic",
           "config": {"workload": "FFN prefill, M=2048: gate/up K=3584 N=18944 Q4_K, down K=18944 N=3584 Q6_K"}}
    print(json.dumps(out), flush=True)
    return 0


# The integer path's vector-ALU bound: every output takes three ALU operations
# per 32-value sub-block (convert the integer block sum, form the scale
# product, fused multiply-add), i.e. 3/32 operation per multiply-add, on
# 256 CUs x 4 SIMDs x 16 lanes at 2.4 GHz (non-packed fp32).
INT_PATH_ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 * (32 / 3) * 2 / 1e12


def q8_gemm(args, dev) -> int:
    """The integer path (Q8_1 activation x Q4_K weight) beside the FP8 path
    on the FFN gate/up shape at M=2048 and M=4096 and the attention Q shape
    (one line): warm times, HIP events around 50 launches after 10 warm-up
    launches, and the accuracy of both paths' outputs on 64 rows against a
    float64 product of the fp32 activation and the fp32 dequantised weight
    (torch float64 on the GPU, from rz_dequant_f32)."""
    import torch

    import fp8_prefill_gemm_amd as rz
    import workloads as W

    stream = torch.cuda.current_stream(dev)

    def timed(fn, reps=TIMED_LAUNCHES):
        for _ in range(WARM_LAUNCHES):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    rows = {}
    for name, m, n, k in [("cfg3 gate/up", 2048, 18944, 3584), ("cfg4 gate/up", 4096, 18944, 3584),
                          ("cfg2 q", 512, 3584, 3584)]:
        x = torch.from_numpy(W.act_normal(41 + m, m, k)).to(dev)
        blocks = torch.from_numpy(W.q4k_blocks(42 + n, n, k)).to(dev)
        q8 = rz.rz_q8_1_quant(x, stream=stream)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        t_q = timed(lambda: rz.rz_q8_1_quant(x, q8, stream))
        t_g = timed(lambda: rz.rz_q8_q4k_gemm(q8, m, blocks, n, k, y, stream))
        a8, sc = rz.rz_fp8_quant_act(x, stream=stream)
        w8, scale, _ = rz.rz_fp8_pack_weight(W.Q4_K, blocks, n, k, stream=stream)
        y8 = torch.empty((m, n), dtype=torch.float32, device=dev)
        t_f = timed(lambda: rz.rz_fp8_gemm(a8, w8, m, sc, scale, y8, stream, ws=None))
        fl = 2.0 * m * n * k
        rows[name] = {"m": m, "n": n, "k": k, "q8_quant_us": round(t_q * 1e6, 1),
                      "q8_gemm_us": round(t_g * 1e6, 1), "q8_gemm_tops": round(fl / t_g / 1e12, 1),
                      "fp8_gemm_us": round(t_f * 1e6, 1), "fp8_gemm_tflops": round(fl / t_f / 1e12, 1)}
        if name == "cfg3 gate/up":
            wf = rz.rz_dequant_f32(W.Q4_K, blocks, n, k, stream=stream)
            sel = torch.linspace(0, m - 1, 64, device=dev).long()
            ref = x[sel].double() @ wf.double().t()
            den = ref.abs().mean().item()
            rows[name]["accuracy_vs_fp64_of_fp32_inputs"] = {
                nm: {"mean_abs_err_rel": round((yy[sel].double() - ref).abs().mean().item() / den, 6),
                     "max_abs_err_rel": round((yy[sel].double() - ref).abs().max().item() / den, 6)}
                for nm, yy in (("q8_1 x q4_k", y), ("fp8", y8))}
            del wf, ref
        log(f"{name}: {rows[name]}")
        del x, blocks, q8, y, a8, w8, y8
    g = rows["cfg3 gate/up"]
    ach = 2.0 * g["m"] * g["n"] * g["k"] / (g["q8_gemm_us"] * 1e-6) / 1e12
    roof = {"kernel": "q8_q4k_gemm_kernel (M=2048, N=18944, K=3584)", "bound": "alu", "achieved": round(ach, 1),
            "peak": round(INT_PATH_ALU_PEAK_TOPS, 1), "unit": "TOPS", "frac": round(ach / INT_PATH_ALU_PEAK_TOPS, 4),
            "int8_mfma_peak_tops": 5000.0, "frac_of_int8_mfma_peak": round(ach / 5000.0, 4), "traffic": None}
    out = {"metric": "Q8_1 x Q4_K integer GEMM vs FP8 GEMM (warm)", "unit": "us", "higher_is_better": False,
           "rows": rows, "roofline": roof, "dtype": "int8 x 4-bit (int32 block sums, fp32 accumulate)",
           "data": "synthetic", "config": {"workload": "prefill GEMM shapes of the 7B-class model, Q4_K weights"}}
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # the defaults time the clocks' steady state: after only a few warm-up
    # steps the GPU is still raising its clock (measured: gate+up launch 0.38
    # of peak after 3 warm-up steps, 0.43 after 10, 0.45-0.46 from 100 on)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle timing (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--pack-model", action="store_true",
                    help="time the cold-cache packing of all 196 weights of the 28-layer sweep instead")
    ap.add_argument("--pack-repeats", type=int, default=3, help="cold passes of --pack-model")
    ap.add_argument("--gemm-shapes", action="store_true",
                    help="instead time the FP8 GEMM alone at every configuration's shapes (warm)")
    ap.add_argument("--small-m", type=int, nargs="*", default=None,
                    help="instead time the small-batch paths at N=4608, K=3584 (Q4_K) for these m")
    ap.add_argument("--fp16-gemm", action="store_true",
                    help="instead time the FP16 cached-weight comparator beside the FP8 path (warm, M=2048 FFN)")
    ap.add_argument("--q8-gemm", action="store_true",
                    help="instead time the integer path (Q8_1 activation x Q4_K weight) beside the FP8 path (warm)")
    ap.add_argument("--gemm-clock", action="store_true",
                    help="instead run the gate+up GEMM back to back with random and constant codes, sampling the "
                         "GFX clock and board power")
    ap.add_argument("--clock-seconds", type=float, default=3.0, help="seconds per --gemm-clock phase")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock pass (the GPU's clock and power readings) after the timed steps")
    ap.add_argument("--clock-settle", type=float, default=0.15,
                    help="seconds of untimed steps before the warm-up steps (the GPU raising its clock from idle)")
    ap.add_argument("--hbm-rates", action="store_true",
                    help="time torch's read, copy and write kernels on 1 GiB instead (HBM rates on this GPU)")
    ap.add_argument("--kquant-gemm", action="store_true",
                    help="instead time the GEMM straight from K-quant blocks beside the cached path (warm)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}), flush=True)
        log("bench.py: only --gpus 1 is supported (the path is measured on one GPU's shard)")
        return 2

    import numpy as np
    import torch

    import fp8_prefill_gemm_amd as rz
    import workloads as W

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        return 1
    rz.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration and (args.pack_model or args.gemm_shapes or args.small_m is not None):
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB write done")
        del src, dst
    if args.hbm_rates:
        return hbm_rates(args, dev)
    # board clock and power readings (refreshed once a second): the default
    # step's clock pass and --gemm-clock
    sampled = not any((args.pack_model, args.gemm_shapes, args.kquant_gemm, args.fp16_gemm, args.q8_gemm,
                       args.small_m is not None)) and not args.no_clock
    metrics = GpuMetrics() if sampled else None
    try:
        return measure(args, dev, metrics)
    finally:
        if metrics is not None:
            metrics.close()


def measure(args, dev, metrics) -> int:
    import numpy as np
    import torch

    import fp8_prefill_gemm_amd as rz
    import workloads as W

    if args.gemm_clock:
        return gemm_clock(args, dev, metrics)
    if args.pack_model:
        return pack_model(args, dev)
    if args.gemm_shapes:
        return gemm_shapes(args, dev)
    if args.kquant_gemm:
        return kquant_gemm(args, dev)
    if args.fp16_gemm:
        return fp16_gemm(args, dev)
    if args.q8_gemm:
        return q8_gemm(args, dev)
    if args.small_m is not None:
        if not args.small_m:
            args.small_m = [1, 2, 3, 4, 8, 37]
        return small_m(args, dev)

    ffn, down = W.config_groups(3)
    gate, up = ffn.gemms
    dn = down.gemms[0]
    M = ffn.m
    log(f"setup: M={M} gate/up N={gate.n} K={gate.k} Q4_K, down N={dn.n} K={dn.k} Q6_K")
    x_ffn_h = ffn.activation()
    x_down_h = down.activation()
    gate_blocks_h = W.weight_blocks(gate.qtype, gate.w_seed, gate.n, gate.k)
    up_blocks_h = W.weight_blocks(up.qtype, up.w_seed, up.n, up.k)
    down_blocks_h = W.weight_blocks(dn.qtype, dn.w_seed, dn.n, dn.k)

    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x_ffn, x_down = to(x_ffn_h), to(x_down_h)
    b_gate, b_up, b_down = to(gate_blocks_h), to(up_blocks_h), to(down_blocks_h)
    u8, f32 = torch.uint8, torch.float32
    w8 = {g.name: torch.empty((g.n, g.k), dtype=u8, device=dev) for g in (gate, up, dn)}
    Mp = rz.rz_pad_m(M)
    a8_ffn = torch.empty((Mp, ffn.k), dtype=u8, device=dev)
    a8_down = torch.empty((Mp, down.k), dtype=u8, device=dev)
    sc_ffn = torch.empty(4, dtype=f32, device=dev)
    sc_down = torch.empty(4, dtype=f32, device=dev)
    y = {g.name: torch.empty((M, g.n), dtype=f32, device=dev) for g in (gate, up, dn)}
    ws = rz.workspace(dev)
    gws_bytes = max(rz.rz_fp8_gemm_workspace_bytes(M, g.n, g.k) for g in (gate, up, dn))
    gws = torch.zeros(max(gws_bytes, 256), dtype=u8, device=dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=f32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB write done")
        del src, dst

    phases = ["pack", "quant_ffn", "gemm_gate_up", "quant_down", "gemm_down"]
    packs = [(g.qtype, blk, g.n, g.k, w8[g.name]) for g, blk in ((gate, b_gate), (up, b_up), (dn, b_down))]

    def step(events=None, gemm_events=None):
        """One pass of the path.  events: 6 markers between the phases
        (diagnostic pass); gemm_events: 2 markers around the gate+up GEMM
        launch (timed pass, for the roofline)."""
        def mark(i):
            if events is not None:
                events[i].record(stream)
        def gmark(i):
            if gemm_events is not None:
                gemm_events[i].record(stream)
        mark(0)
        # the three weights in one call: one host wait for their scales
        (_, s_gate, _), (_, s_up, _), (_, s_down, _) = rz.rz_fp8_pack_weights(packs, ws, stream)
        mark(1)
        rz.rz_fp8_quant_act(x_ffn, a8_ffn, sc_ffn, ws, stream)
        mark(2)
        gmark(0)
        # gate and up share the FP8 activation: one launch for both
        rz.rz_fp8_gemm_group(a8_ffn, M, sc_ffn, [(w8["gate"], s_gate), (w8["up"], s_up)],
                             [y["gate"], y["up"]], stream, gws)
        mark(3)
        gmark(1)
        rz.rz_fp8_quant_act(x_down, a8_down, sc_down, ws, stream)
        mark(4)
        rz.rz_fp8_gemm(a8_down, w8["down"], M, sc_down, s_down, y["down"], stream, gws)
        mark(5)

    # everything the timed pass needs is made before the GPU starts working:
    # the markers, and no garbage collection from here on (a full collection
    # over the interpreter's objects stalls the host for milliseconds, the
    # GPU idles meanwhile and lowers its clock; and the host issues every
    # launch of the next phase after the pack's scale readback)
    every = 4
    gev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in range(0, args.steps, every)}
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    gc.collect()
    gc.disable()
    # clock settle: from idle the GPU raises its clock over tens of
    # milliseconds (measured: gate+up launch 0.38 of peak after 3 steps, 0.43
    # after 10, 0.45-0.46 from 100 on), so the step runs untimed for a fixed
    # time before the warm-up steps, whatever their number
    c0 = time.monotonic()
    settle_steps = 0
    while time.monotonic() - c0 < args.clock_settle:
        step()
        settle_steps += 1
    torch.cuda.synchronize()
    log(f"clock settle: {settle_steps} steps in {time.monotonic() - c0:.3f} s; warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed pass: the only markers are the two around the gate+up GEMM
    # launch, on every 4th step (each marker leaves a 3-6 us gap between
    # kernels, so markers on every step would add ~9 us to each)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(gemm_events=gev.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    log(f"timed {args.steps} steps")
    # clock pass (untimed): the GFX clock and board power under the same
    # steps, read from the GPU's metrics; the firmware refreshes them once a
    # second, so the pass runs for CLOCK_PASS_S seconds and keeps the
    # readings from 1.05 s on (a value read earlier may have been refreshed
    # before the pass, during the setup's idle time)
    clock = None
    if metrics is not None:
        metrics.start()
        r0 = time.monotonic()
        clock_steps = 0
        while time.monotonic() - r0 < CLOCK_PASS_S:
            step()
            clock_steps += 1
        torch.cuda.synchronize()
        clock = metrics.window(r0 + 1.05, time.monotonic())
        metrics.close()
        clock["window"] = f"{clock_steps} untimed steps ({CLOCK_PASS_S} s) after the timed ones, from 1.05 s on"
        log(f"clock pass: {clock}")
    gateup_events_us = float(np.mean([e[0].elapsed_time(e[1]) for e in gev.values()])) * 1e3

    # diagnostic pass (not timed as a whole): markers between every phase
    for i in range(args.steps):
        step(events=ev[i])
    torch.cuda.synchronize()
    gc.enable()

    ms_per_step = (t1 - t0) * 1e3 / max(args.steps, 1)
    ph = {p: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in ev])) * 1e3 for i, p in enumerate(phases)}
    flop = {g.name: 2.0 * M * g.n * g.k for g in (gate, up, dn)}
    step_flop = sum(flop.values())
    value = step_flop / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = {"gate_up": (flop["gate"] + flop["up"]) / (ph["gemm_gate_up"] * 1e-6) / 1e12,
                   "down": flop["down"] / (ph["gemm_down"] * 1e-6) / 1e12}
    gateup_us = gateup_events_us  # the one launch of both GEMMs
    achieved = (flop["gate"] + flop["up"]) / (gateup_us * 1e-6) / 1e12
    plan = rz.rz_fp8_gemm_plan(M, gate.n + up.n, gate.k)
    # HBM-bound phases: algorithmic bytes (blocks read twice + 1 B per weight
    # written; activations read twice as fp32 + 1 B per element written)
    # against the 8 TB/s HBM peak
    Mp_ffn = rz.rz_pad_m(M)
    algo = {
        "pack": (2 * gate_blocks_h.nbytes + gate.n * gate.k + 2 * up_blocks_h.nbytes + up.n * up.k
                 + 2 * down_blocks_h.nbytes + dn.n * dn.k),
        "quant_ffn": 2 * x_ffn_h.nbytes + Mp_ffn * ffn.k,
        "quant_down": 2 * x_down_h.nbytes + Mp_ffn * down.k,
    }
    hbm = {k: {"algorithmic_bytes": int(b), "tb_per_s": round(b / (ph[k] * 1e-6) / 1e12, 3),
               "frac": round(b / (ph[k] * 1e-6) / 1e12 / HBM_PEAK_TBPS, 4)} for k, b in algo.items()}
    log("phases (us): " + " ".join(f"{k}={v:.1f}" for k, v in ph.items()))
    log("HBM-bound phases: " + " ".join(f"{k}={v['tb_per_s']:.2f}TB/s({v['frac']:.0%})" for k, v in hbm.items()))
    log(f"gate+up GEMM launch {gateup_us:.1f} us = {achieved:.1f} TFLOP/s ({achieved / FP8_PEAK_TFLOPS:.1%} of peak), "
        f"plan BNxBM={plan[0]}x{plan[1]} threads={plan[2]} wgs={plan[3]}")

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "clock_settle": {"seconds": args.clock_settle, "steps": settle_steps},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "config": {
            "workload": ("FFN prefill, M=2048: gate+up K=3584 N=18944 Q4_K sharing one FP8 activation, "
                         "down K=18944 N=3584 Q6_K; step = pack 3 weights + 2 activation quants + 3 GEMMs"),
            "m": M, "gate_up": [gate.n, gate.k], "down": [dn.n, dn.k],
        },
        "roofline": {
            "kernel": (f"gate+up GEMM in one launch, {plan[0]}x{plan[1]} tiles, {plan[3]} persistent workgroups "
                       f"(M=2048, N=2x18944, K=3584)"),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(),
            # GFX clock and board power over the timed steps
            "clock": at_clock(achieved, clock),
            # the counter run (GRBM_GUI_ACTIVE, MFMA busy cycles): its launch
            # ran alone (counter collection serialises dispatches)
            "mfma_counters": measured_clock(),
        },
        "phases_us": {k: round(v, 2) for k, v in ph.items()},
        "hbm_phases": hbm,
        "gemm_tflops": {k: round(v, 2) for k, v in gemm_tflops.items()},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(x_ffn_h, x_down_h, gate_blocks_h, down_blocks_h, gate, dn)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
