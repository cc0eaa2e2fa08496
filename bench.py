#!/usr/bin/env python3
"""Throughput of the gfx950 dense GEMM library on one MI355X.

One step = one GEMM call C = alpha*A*B + beta*C on the headline workload
(BF16 inputs, FP32 accumulate/output, M = N = K = 8192), inputs already
resident in HBM.  Before the W untimed warm-up calls the workload runs
untimed for --settle-ms (default 300 ms): after the GPU has idled (while the
host generates the next inputs) its power-managed clock overshoots and then
settles over some 40-80 calls of the 8192^3 GEMM, and the pages ask for
warm-up before numbers are quoted because the first runs include that ramp
(dilfish.github.io 5.7).  Then K timed calls bracketed by device
synchronisation, timed with HIP events on the stream the kernels run on.
TFLOP/s = 2MNK / time (chongfengling.github.io section 1 counts K multiplies
and K adds per output; 2*2048^3 = 17.18e9 in its section 2.5).

The same JSON line carries, under "also", the small FP32 cases (256^3, and
the ragged 1000^3 with alpha = 1.5, beta = 0.5), the FP32 4096^3 case
(against the fp32 matrix-core peak), the FP16-input 8192^3 case (against the
fp16 peak, equal to bf16's), the skinny decode-shaped case M=8, N=28672,
K=8192 (against HBM bandwidth: its time is the time to stream B once,
dilfish.github.io 5.1 GEMV row), the BF16 square and skinny cases with a
linear layer's operand storage (B stored N x K, A stored K x M; the skinny
one also with FP32 inputs), that
layer's forward with its bias fused, a strided batch of 16 x 2048^3, and the
split-K, stream-K and one-GPU-share shapes, plus:
  * "roofline": the dominant kernel's algorithmic FLOP (or bytes) per launch
    over its measured launch time, against the published MI355X peak, and
    the same against the peak scaled to the engine clock the workload runs
    at ("clock");
  * "clock": the graphics clock (mean over the 8 XCDs) and socket power the
    GPU's own telemetry reports while the workload runs back to back for
    --telemetry-s seconds after its timed calls (amdsmi gpu metrics; the
    firmware refreshes them about once a second, too slowly to sample the
    timed calls themselves);
  * "pcie": one host-to-device copy of A and B and one device-to-host copy
    of C, timed apart from the metric (dilfish.github.io 5.7: transfers are
    part of what a caller pays, but not of the kernel's time);
  * "cpu_baseline": the CPU oracle timed on a bounded row sample of the same
    workload on this host's cores (a reported baseline, not a target), and
    on the two small FP32 cases with one thread and with all of them.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --only bf16_8192 --no-cpu   (one workload, for profiling)
       python bench.py --ladder                    (every rung at FP32 4096^3, BF16 8192^3)
       python bench.py --counter-check             (the naive rung once at FP32 2048^3)
       python bench.py --tile-check                (both DMA tiles against the automatic choice)
       python bench.py --copy-calibration          (copy kernel of known size)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOPS + % of MI355X roofline (FP32 4096^3, BF16 8192^3, skinny GB/s)"

# Published MI355X peaks (dense, no sparsity): matrix cores bf16 and fp16
# 2.5 PFLOP/s, fp32 157.3 TFLOP/s; HBM3E 8 TB/s.
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
HBM_PEAK_GBS = 8000.0

PRIMARY = "bf16_8192"
SECONDARY = ["f32_256", "f32_1000_ragged", "f32_4096", "f16_8192", "bf16_skinny_8x28672x8192",
             "bf16_8192_nt", "bf16_8192_tn", "bf16_skinny_8x28672x8192_nt", "f32_skinny_8x28672x8192_nt",
             "bf16_linear_bias_8192_nt",
             "bf16_bmm_16x2048", "bf16_decode_64x28672x8192_nt", "f32_1000_splitk",
             "bf16_splitk_1024x1024x16384", "bf16_skinny_shard_8x3584x8192",
             "bf16_shard_8192x1024x8192", "bf16_streamk_6144x4096x8192", "f32_streamk_3000"]

# Kernel that dominates each workload's time, for the roofline: a readable
# name, its source file, and a pattern for the name rocprofv3 prints (the
# template arguments: input format, then vector / guard flags where the
# kernel has them, then trans_a, trans_b; the DMA GEMM kernels' end with
# their edge-tile and K-tail flags, false for whole tiles; the skinny DMA
# kernel's are the input format, row-block count, waves, ring stages, bytes
# per row piece of a step and whether A has one register buffer).
DOMINANT = {
    "f32_256": ("mfma_f32_kernel<NN, 64-tiles>", "k_mfma_f32.hip",
                r"mfma_f32_kernel<true, false, false, false, 64>"),
    "f32_1000_ragged": ("mfma_f32_kernel<NN, 64-tiles, guarded>", "k_mfma_f32.hip",
                        r"mfma_f32_kernel<true, true, false, false, 64>"),
    "bf16_8192": ("mfma16_dma_kernel<BF16, NN>", "k_mfma_bf16_dma.hip",
                  r"mfma16_dma_kernel<\(dgt::In\)1, 256, false, false, false, false>"),
    "f16_8192": ("mfma16_dma_kernel<F16, NN>", "k_mfma_bf16_dma.hip",
                 r"mfma16_dma_kernel<\(dgt::In\)2, 256, false, false, false, false>"),
    "f32_4096": ("mfma_f32_dma_kernel<NN, 256-tiles>", "k_mfma_f32_dma.hip",
                 r"mfma_f32_dma_kernel<256, false, false, false, false>"),
    "bf16_skinny_8x28672x8192": ("skinny16_kernel<BF16, NN, 1 row block>", "k_skinny16.hip",
                                 r"skinny16_kernel<\(dgt::In\)1, true, false, false, 1>"),
    "bf16_8192_nt": ("mfma16_dma_kernel<BF16, NT>", "k_mfma_bf16_dma.hip",
                     r"mfma16_dma_kernel<\(dgt::In\)1, 256, false, true, false, false>"),
    "bf16_8192_tn": ("mfma16_dma_kernel<BF16, TN>", "k_mfma_bf16_dma.hip",
                     r"mfma16_dma_kernel<\(dgt::In\)1, 256, true, false, false, false>"),
    "bf16_skinny_8x28672x8192_nt": ("skinny_bt_dma_kernel<BF16, 1 row block, 8 waves>",
                                    "k_skinny_dma.hip",
                                    r"skinny_bt_dma_kernel<\(dgt::In\)1, 1, 8, 2, 256, false>"),
    "bf16_linear_bias_8192_nt": ("mfma16_dma_kernel<BF16, NT> + bias", "k_mfma_bf16_dma.hip",
                                 r"mfma16_dma_kernel<\(dgt::In\)1, 256, false, true, false, false>"),
    "f32_skinny_8x28672x8192_nt": ("skinny_bt_dma_kernel<F32, 1 row block, 8 waves>",
                                   "k_skinny_dma.hip",
                                   r"skinny_bt_dma_kernel<\(dgt::In\)0, 1, 8, 2, 256, false>"),
    "bf16_decode_64x28672x8192_nt": ("skinny_bt_dma_kernel<BF16, 4 row blocks, 8 waves>",
                                     "k_skinny_dma.hip",
                                     r"skinny_bt_dma_kernel<\(dgt::In\)1, 4, 8, 4, 128, true>"),
    "f32_1000_splitk": ("mfma_f32_dma_kernel<NN, 128-tiles, edge> x 4 K slices + reduce (per call)",
                        "k_mfma_f32_dma.hip+k_splitk.hip",
                        r"mfma_f32_dma_kernel<128, false, false, true, (?:false|true)>"),
    "bf16_splitk_1024x1024x16384": ("mfma16_dma_kernel<BF16, NN, 128-tiles> x 8 K slices + "
                                    "reduce (per call)", "k_mfma_bf16_dma.hip+k_splitk.hip",
                                    r"mfma16_dma_kernel<\(dgt::In\)1, 128, false, false, false, false>"),
    "bf16_skinny_shard_8x3584x8192": ("skinny16_kernel<BF16, NN, 1 row block> x 8 K slices + "
                                      "reduce (per call)", "k_skinny16.hip+k_splitk.hip",
                                      r"skinny16_kernel<\(dgt::In\)1, true, false, false, 1>"),
    "bf16_shard_8192x1024x8192": ("mfma16_dma_kernel<BF16, NN, 128-tiles>", "k_mfma_bf16_dma.hip",
                                  r"mfma16_dma_kernel<\(dgt::In\)1, 128, false, false, false, false>"),
    "bf16_bmm_16x2048": ("mfma16_dma_kernel<BF16, NN>, batch 16", "k_mfma_bf16_dma.hip",
                         r"mfma16_dma_kernel<\(dgt::In\)1, 256, false, false, false, false>"),
    "bf16_streamk_6144x4096x8192": ("mfma16_streamk_kernel<BF16, NN> + fix-up (per call)",
                                    "k_mfma_bf16_dma.hip",
                                    r"mfma16_streamk_kernel<\(dgt::In\)1, false, false, false>"),
    "f32_streamk_3000": ("mfma_f32_streamk_kernel<NN, ragged> + fix-up (per call)",
                         "k_mfma_f32_dma.hip",
                         r"mfma_f32_streamk_kernel<false, false, true>"),
}

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ cost model

def gemm_flops(M: int, N: int, K: int) -> int:
    """K multiplies and K adds per output element."""
    return 2 * M * N * K


def algorithmic_bytes(M: int, N: int, K: int, in_bytes: int, beta: float) -> int:
    """Read A and B once, write C once (and read it once when beta != 0)."""
    return (M * K + K * N) * in_bytes + M * N * 4 * (2 if beta != 0 else 1)


def arithmetic_intensity(flops: float, nbytes: float) -> float:
    return flops / nbytes


def naive_lane_view_intensity(K: int, in_bytes: int = 4) -> float:
    """One lane per output reads a row of A and a column of B: 2K FLOP over
    2K loads (dilfish.github.io 5.2; chongfengling.github.io 2.3)."""
    return (2 * K) / (2 * K * in_bytes)


def tile_intensity(T: int, in_bytes: int = 4) -> float:
    """A T x T tile per K-slice of T: 2T^3 FLOP over 2T^2 loaded elements
    (dilfish.github.io 5.3)."""
    return (2 * T ** 3) / (2 * T * T * in_bytes)


def naive_load_requests(M: int, N: int, K: int, wave: int) -> int:
    """Vector load instructions of the one-lane-per-output kernel: each
    wavefront issues one load of A and one of B per k."""
    return 2 * K * (M * N // wave)


# ------------------------------------------------------------ measurement

def source_digest(fname: str) -> str:
    """Digest of the kernel sources a workload runs: one file, or several
    joined by '+', with the headers they include (followed transitively)."""
    csrc = os.path.join(ROOT, "dense_gemm_tuning_amd", "csrc")
    order, todo = [], list(fname.split("+"))
    while todo:
        f = todo.pop(0)
        if f in order:
            continue
        order.append(f)
        with open(os.path.join(csrc, f), "rb") as fh:
            todo += [m.decode() for m in re.findall(rb'^#include "([^"]+)"', fh.read(), re.M)]
    h = hashlib.sha256()
    for f in order:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    absent or taken on a different version of the kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kern, src, _ = DOMINANT[workload]
    want = source_digest(src)
    pat = re.compile(r"^traffic\s+workload=(\S+)\s+kernel=(.+?)\s+src=(\S+)\s+"
                     r"fetch_bytes=(\d+)\s+write_bytes=(\d+)", re.M)
    for m in pat.finditer(open(TRAFFIC_FILE).read()):
        if m.group(1) == workload and m.group(3) == want:
            return int(m.group(4)) + int(m.group(5))
    return None


def to_dev(torch, x, dtype):
    import numpy as np
    if dtype in ("bf16", "f16"):
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
        return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


# ------------------------------------------------------------ GPU telemetry

class Telemetry:
    """The graphics clock, socket power and energy counter the GPU's firmware
    reports (amdsmi gpu metrics), read from a host thread while kernels run,
    so reading them costs the GPU nothing.  The firmware refreshes the table
    about once a second (its system_clock_counter, in ns, says when), so a
    reading describes the second before it: the bench therefore runs each
    workload for a few seconds in a telemetry pass of its own and keeps only
    the tables produced well inside that pass.  ``current_gfxclks`` holds
    one clock per XCD; their mean is the engine clock.  Disabled (error set,
    every reading None) when amdsmi is missing or cannot open the device
    torch uses."""

    # the energy accumulator counts in units of 15.3 uJ (amdsmi's
    # counter_resolution on this part)
    ENERGY_UJ = 15.3

    def __init__(self, torch):
        self.handle, self.error = None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.smi = amdsmi
            props = torch.cuda.get_device_properties(0)
            want = (getattr(props, "pci_domain_id", 0), getattr(props, "pci_bus_id", None),
                    getattr(props, "pci_device_id", 0))
            for h in amdsmi.amdsmi_get_processor_handles():
                dom, bus, rest = amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")  # dddd:bb:dd.f
                got = (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16))
                if want[1] is None or got == want:
                    self.handle = h
                    break
            if self.handle is None:
                self.error = f"no amdsmi device matches torch's device 0 ({want})"
        except Exception as e:  # telemetry is optional; the metric does not depend on it
            self.error = f"{type(e).__name__}: {e}"

    def read(self):
        """(firmware timestamp ns, mean graphics clock over the XCDs in MHz,
        socket power in W, energy counter in J), or None."""
        if self.handle is None:
            return None
        try:
            m = self.smi.amdsmi_get_gpu_metrics_info(self.handle)
        except Exception:
            return None

        def num(x):
            return x if isinstance(x, (int, float)) else None
        clk = m.get("current_gfxclks")
        vals = [c for c in clk if num(c) and c > 0] if isinstance(clk, list) else []
        if not vals and num(m.get("current_gfxclk")):
            vals = [m["current_gfxclk"]]
        en = num(m.get("energy_accumulator"))
        return (num(m.get("system_clock_counter")), sum(vals) / len(vals) if vals else None,
                num(m.get("current_socket_power")),
                en * self.ENERGY_UJ * 1e-6 if en is not None else None)


def telemetry_pass(torch, launch, tel, seconds, ms_call):
    """Run launch(i) back to back for `seconds` while a host thread polls the
    telemetry every 20 ms; summarise the firmware tables first seen at least
    1.2 s into the pass (each describes the second before it, so they cover
    steady running only).  The host queues at most ~20 ms of calls (ms_call
    each) ahead of the GPU, so the pass ends on time however long a call
    takes.  Returns None without telemetry."""
    import threading
    if tel is None or tel.handle is None or seconds <= 0:
        return None
    seen, stop = {}, threading.Event()
    t0 = time.perf_counter()

    def poll():
        while not stop.is_set():
            r = tel.read()
            t = time.perf_counter() - t0
            if r and r[0] is not None and r[0] not in seen:
                seen[r[0]] = (t, r)
            stop.wait(0.02)
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    ahead = max(1, int(20.0 / max(ms_call, 1e-3)))
    n = 0
    while time.perf_counter() - t0 < seconds:
        launch(n)
        n += 1
        if n % ahead == 0:
            torch.cuda.synchronize()  # bound the queue so the pass ends on time
    torch.cuda.synchronize()
    stop.set()
    th.join()
    tables = [r for (t, r) in sorted(seen.values(), key=lambda x: x[1][0]) if t >= 1.2]
    if not tables:
        return {"tables": 0, "calls": n}
    clk = [r[1] for r in tables if r[1] is not None]
    pw = [r[2] for r in tables if r[2] is not None]
    out = {"gfxclk_mhz": round(sum(clk) / len(clk), 1) if clk else None,
           "socket_power_w": round(sum(pw) / len(pw), 1) if pw else None,
           "tables": len(tables), "calls": n, "seconds": seconds,
           "source": "amdsmi gpu metrics (current_gfxclks mean over XCDs, "
                     "current_socket_power, energy_accumulator)"}
    if len(tables) >= 2 and tables[0][3] is not None and tables[-1][3] is not None:
        dt = (tables[-1][0] - tables[0][0]) * 1e-9
        if dt > 0:
            out["energy_power_w"] = round((tables[-1][3] - tables[0][3]) / dt, 1)
    return out


# ------------------------------------------------------------ timing

def make_fn(torch, dgt, w, dbias):
    """The library call the bench times for workload w, as
    fn(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream) -> status,
    and the workspace it holds (allocated here, outside any timing)."""
    code = {"f32": dgt.DTYPE_F32, "bf16": dgt.DTYPE_BF16, "f16": dgt.DTYPE_F16}[w.dtype]
    if w.streamk:
        need = dgt.gemm_streamk_workspace_size(code, w.M, w.N, w.K)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

        def fn(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s):
            return dgt.gemm_streamk(code, w.trans_a, w.trans_b, M, N, K, alpha, A, lda, B, ldb,
                                    beta, C, ldc, ws.data_ptr(), need, s)
        return fn, ws
    if w.splits != 1:
        need = dgt.gemm_splitk_workspace_size(code, w.M, w.N, w.K, w.splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

        def fn(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s):
            return dgt.gemm_splitk(code, w.trans_a, w.trans_b, M, N, K, alpha, A, lda, B, ldb,
                                   beta, C, ldc, w.splits, ws.data_ptr(), need, s)
        return fn, ws
    if w.batch > 1 or dbias is not None:
        def fn(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s):
            return dgt.gemm_strided_batched(
                code, w.trans_a, w.trans_b, dgt.VARIANT_AUTO, M, N, K, alpha,
                A, lda, w.a_shape[0] * lda, B, ldb, w.b_shape[0] * ldb, beta, C, ldc, M * N,
                dbias.data_ptr() if dbias is not None else 0, N, w.batch, s)
        return fn, None
    if w.trans_a or w.trans_b:
        def fn(*args):
            return dgt.gemm_ex(code, w.trans_a, w.trans_b, dgt.VARIANT_AUTO, *args)
        return fn, None
    return {"f32": dgt.gemm_f32, "bf16": dgt.gemm_bf16, "f16": dgt.gemm_f16}[w.dtype], None


def time_calls(torch, launch, steps, warmup, settle_ms):
    """Settle, warm up, then time `steps` back-to-back calls of launch(i)
    between one pair of events on the current stream; a second pass with an
    event after every call gives the per-call spread."""
    stream = torch.cuda.current_stream()
    n_settle = 0
    if settle_ms > 0:
        t_end = time.perf_counter() + settle_ms * 1e-3
        while time.perf_counter() < t_end:
            launch(n_settle)
            n_settle += 1
            if n_settle % 8 == 0:
                torch.cuda.synchronize()  # keep the queue short so the wall clock means GPU time
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    # spread: the markers add a little time of their own, so this pass does
    # not feed the average
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        launch(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return {"ms_avg": total / steps, "ms_median": per[len(per) // 2],
            "ms_min": per[0], "ms_max": per[-1], "settle_calls": n_settle}


def time_workload(torch, dgt, w, steps, warmup, copies=1, settle_ms=300.0, tel=None,
                  pcie=False, telemetry_s=0.0, keep_c=False):
    """Average and spread of one GEMM call's duration (ms) on the current stream."""
    import gemm_inputs as gi
    t0 = time.perf_counter()
    A, B, C0 = gi.make_inputs(w)
    log(f"[{w.name}] inputs generated in {time.perf_counter() - t0:.1f} s")
    bias = gi.make_bias(w)
    pcie_res = measure_pcie(torch, w, A, B) if pcie else None
    dA = [to_dev(torch, A, w.dtype) for _ in range(copies)]
    dB = [to_dev(torch, B, w.dtype) for _ in range(copies)]
    dC = (torch.from_numpy(C0).cuda() if C0 is not None
          else torch.zeros((w.batch, w.M, w.N), dtype=torch.float32, device="cuda"))
    dbias = torch.from_numpy(bias).cuda() if bias is not None else None
    sptr = torch.cuda.current_stream().cuda_stream
    lda, ldb = w.a_shape[1], w.b_shape[1]  # packed stored rows
    fn, ws = make_fn(torch, dgt, w, dbias)

    def launch(i):
        st = fn(w.M, w.N, w.K, w.alpha, dA[i % copies].data_ptr(), lda,
                dB[i % copies].data_ptr(), ldb, w.beta, dC.data_ptr(), w.N, sptr)
        if st != 0:
            raise RuntimeError(dgt.gemm_status_string(st))

    res = time_calls(torch, launch, steps, warmup, settle_ms)
    res["clock"] = telemetry_pass(torch, launch, tel, telemetry_s, res["ms_avg"])
    if pcie_res is not None:
        res["pcie"] = pcie_res
    # the result of the last call (every call writes the same C when beta == 0)
    c_host = dC.cpu().numpy().reshape(w.batch, w.M, w.N)[0] if keep_c and w.beta == 0 else None
    del dA, dB, dC, ws
    torch.cuda.empty_cache()
    return res, (A, B, C0, c_host)


def measure_pcie(torch, w, A, B, reps=3):
    """Host <-> device copies of the workload's operands from and to pinned
    host memory, timed with events (best of `reps`): A and B in, C out."""
    import numpy as np
    stream = torch.cuda.current_stream()
    in_bytes = 4 if w.dtype == "f32" else 2
    hA = torch.from_numpy(np.ascontiguousarray(A).view(np.uint8).reshape(-1)).pin_memory()
    hB = torch.from_numpy(np.ascontiguousarray(B).view(np.uint8).reshape(-1)).pin_memory()
    hC = torch.empty(w.batch * w.M * w.N * 4, dtype=torch.uint8).pin_memory()
    dA, dB = torch.empty_like(hA, device="cuda"), torch.empty_like(hB, device="cuda")
    dC = torch.empty_like(hC, device="cuda")
    best_in, best_out = math.inf, math.inf
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        dA.copy_(hA, non_blocking=True)
        dB.copy_(hB, non_blocking=True)
        e[1].record(stream)
        hC.copy_(dC, non_blocking=True)
        e[2].record(stream)
        torch.cuda.synchronize()
        best_in = min(best_in, e[0].elapsed_time(e[1]))
        best_out = min(best_out, e[1].elapsed_time(e[2]))
    nin = (w.M * w.K + w.K * w.N) * in_bytes * w.batch
    nout = w.batch * w.M * w.N * 4
    del dA, dB, dC
    return {"h2d_ms": round(best_in, 3), "h2d_bytes": nin,
            "h2d_gbs": round(nin / (best_in * 1e-3) / 1e9, 1),
            "d2h_ms": round(best_out, 3), "d2h_bytes": nout,
            "d2h_gbs": round(nout / (best_out * 1e-3) / 1e9, 1),
            "memory": "pinned host buffers (best of %d)" % reps}


def streams_b(w) -> bool:
    """Shapes the skinny path runs (M <= 64): bound by streaming B from HBM
    once, so their roofline is HBM bandwidth."""
    return w.M <= 64


INFINITY_CACHE_BYTES = 256 << 20


def input_copies(w) -> int:
    """Copies of the inputs the bench rotates through: for shapes that stream
    B, enough that the copies together are at least twice the 256 MB
    Infinity Cache, so no launch finds its B there (2 for a 448 MiB B, 10 for
    a 56 MiB one); one otherwise."""
    if not streams_b(w):
        return 1
    b_bytes = w.K * w.N * (4 if w.dtype == "f32" else 2) * w.batch
    return max(2, -(-2 * INFINITY_CACHE_BYTES // b_bytes))


SPEC_CLOCK_MHZ = 2400.0


def roofline(w, ms_avg, clock_mhz=None):
    kern, _, _ = DOMINANT[w.name]
    fl = gemm_flops(w.M, w.N, w.K) * w.batch
    by = algorithmic_bytes(w.M, w.N, w.K, 4 if w.dtype == "f32" else 2, w.beta) * w.batch
    if w.bias:
        by += w.N * 4 * w.batch
    traffic = read_traffic(w.name)
    if streams_b(w):
        ach = by / (ms_avg * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": kern, "algorithmic_bytes": by}
    ach = fl / (ms_avg * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    out = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak,
           "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic,
           "kernel": kern, "algorithmic_flops": fl}
    if clock_mhz:
        # the matrix cores' peak scales with the engine clock: the same
        # kernel against what the chip could issue at the clock it ran at
        p = peak * clock_mhz / SPEC_CLOCK_MHZ
        out["at_measured_clock"] = {"clock_mhz": clock_mhz, "peak": round(p, 1),
                                    "frac": round(ach / p, 4)}
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, A, B, C0, target_s=12.0, c_gpu=None):
    """The oracle as it stands, on a row sample sized for ~target_s seconds.
    With the GPU's C of the timed calls (c_gpu), the same oracle rows also
    give the accuracy of the timed result: normwise and largest elementwise
    error against the oracle's fp64 values, beside the gates the tests
    apply."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    rows = 8
    while True:
        t0 = time.perf_counter()
        R = oracle.gemm(A[:rows], B, None if C0 is None else C0[:rows], w.alpha, w.beta, w.dtype)
        dt = time.perf_counter() - t0
        if dt >= target_s / 3 or rows >= w.M:
            break
        rows = min(w.M, max(rows * 2, int(rows * target_s / max(dt, 1e-3))))
    fl = gemm_flops(rows, w.N, w.K)
    out = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s",
           "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"first {rows} of {w.M} rows of {w.name} "
                     f"({rows}x{w.N}x{w.K}, {dt:.1f} s incl. fp64 widening of B)",
           "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0))}
    if c_gpu is not None:
        d = np.asarray(c_gpu[:rows], np.float64) - R
        nref = float(np.linalg.norm(R))
        out["accuracy"] = {
            "rows": rows, "normwise_rel": float(np.linalg.norm(d)) / nref if nref else None,
            "max_abs": float(np.max(np.abs(d))),
            "gate_normwise": 1e-5,
            "gate_max_abs": 1e-4 * math.sqrt(w.K) * max(1.0, abs(w.alpha)) * w.sigma * w.sigma}
    return out


def cpu_small_cases(names=("f32_256", "f32_1000_ragged")):
    """The oracle on the two small FP32 cases, whole, with one thread and with
    all of them (the pages: below a size of about 128 a CPU can beat the
    GPU once launch and transfer costs count, dilfish.github.io 5.6)."""
    import gemm_inputs as gi
    import oracle
    oracle.build(force=False)
    full = oracle.num_threads()
    out = []
    for name in names:
        w = gi.WORKLOADS[name]
        A, B, C0 = gi.make_inputs(w)
        entry = {"workload": name, "M": w.M, "N": w.N, "K": w.K}
        for threads in (1, full):
            oracle.set_num_threads(threads)
            best = math.inf
            for _ in range(3):
                t0 = time.perf_counter()
                oracle.gemm(A, B, C0, w.alpha, w.beta, w.dtype)
                best = min(best, time.perf_counter() - t0)
            key = "one_thread" if threads == 1 else f"{threads}_threads"
            entry[key] = {"ms": round(best * 1e3, 3),
                          "gflops": round(gemm_flops(w.M, w.N, w.K) / best / 1e9, 2)}
        out.append(entry)
    oracle.set_num_threads(full)
    return out


def copy_calibration(torch, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling HBM byte counters."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes,
                      "copy_calibration_bytes_written": nbytes, "reps": reps}))


# ------------------------------------------------------------ the ladder

# The rungs of the kernel ladder, slowest first (the pages' naive -> shared
# tiles -> register tiles -> matrix units -> deeper pipeline progression,
# qwbw.cn section 三 table; dilfish.github.io 5.2-5.5), by library variant.
LADDER = [("naive", "one lane per output, two global loads per FMA"),
          ("lds", "LDS-staged 128x128 tiles, 8x8 outputs per lane on the vector ALU"),
          ("mfma_regs", "register-staged LDS tiles, MFMA micro-tiles"),
          ("mfma128", "global->LDS DMA pipeline, 128x128 tiles, MFMA"),
          ("mfma256", "global->LDS DMA pipeline, 256x256 tiles, MFMA"),
          ("auto", "what gemm_f32 / gemm_bf16 pick")]
LADDER_WORKLOADS = ("f32_4096", "bf16_8192")


def ladder(torch, dgt, steps, warmup, settle_ms, tel, telemetry_s):
    """Every rung on the FP32 4096^3 and BF16 8192^3 workloads: time per call,
    TFLOP/s and fraction of the matrix-core peak."""
    import gemm_inputs as gi
    out = []
    for name in LADDER_WORKLOADS:
        w = gi.WORKLOADS[name]
        A, B, _ = gi.make_inputs(w)
        dA, dB = to_dev(torch, A, w.dtype), to_dev(torch, B, w.dtype)
        dC = torch.zeros((w.M, w.N), dtype=torch.float32, device="cuda")
        sptr = torch.cuda.current_stream().cuda_stream
        var_fn = {"f32": dgt.gemm_f32_variant, "bf16": dgt.gemm_bf16_variant}[w.dtype]
        for rung, what in LADDER:
            v = dgt.VARIANTS[rung]
            slow = rung in ("naive", "lds")
            n, wu, settle = (max(2, steps // 10), 1, 0.0) if slow else (steps, warmup, settle_ms)

            def launch(i, v=v):
                st = var_fn(v, w.M, w.N, w.K, w.alpha, dA.data_ptr(), w.K, dB.data_ptr(), w.N,
                            w.beta, dC.data_ptr(), w.N, sptr)
                if st != 0:
                    raise RuntimeError(f"{rung}: {dgt.gemm_status_string(st)}")

            log(f"[ladder] {name} {rung}: {n} timed calls")
            r = time_calls(torch, launch, n, wu, settle)
            # the slow rungs' calls are long enough that the pass needs few
            r["clock"] = telemetry_pass(torch, launch, tel, telemetry_s, r["ms_avg"])
            clk = (r["clock"] or {}).get("gfxclk_mhz")
            rf = roofline(w, r["ms_avg"], clk)
            out.append({"workload": name, "rung": rung, "what": what,
                        "ms_per_call": round(r["ms_avg"], 4), "calls": n,
                        "tflops": rf["achieved"], "frac": rf["frac"], "peak": rf["peak"],
                        "clock": r["clock"],
                        "frac_at_measured_clock": rf.get("at_measured_clock", {}).get("frac")})
            log(f"[ladder] {name} {rung}: {r['ms_avg']:.3f} ms, {rf['achieved']} TFLOP/s, "
                f"{rf['frac']:.3f} of peak")
        del dA, dB, dC
        torch.cuda.empty_cache()
    return out


# Shapes on which the automatic choice between the 256 x 256 and 128 x 128
# workgroup tiles of the DMA kernels is checked against timing both.
TILE_CHECK = {"bf16": [(1024, 1024, 1024), (2048, 2048, 2048), (3000, 3000, 3000),
                       (4096, 4096, 4096), (6144, 6144, 6144), (8192, 8192, 8192),
                       (8192, 1024, 8192), (4096, 2048, 4096), (2048, 2048, 8192),
                       (1000, 1000, 1000), (8000, 8000, 8000), (1536, 1536, 4096)],
              "f32": [(1024, 1024, 1024), (2048, 2048, 2048), (3000, 3000, 3000),
                      (4096, 4096, 4096), (6144, 6144, 6144), (1000, 1000, 1000)]}


def tile_check(torch, dgt, steps, warmup):
    """Time the fixed-tile rungs (256 x 256, 128 x 128) and the automatic
    choice on each TILE_CHECK shape, interleaved in one process, and report
    whether the automatic choice is the faster tile (or within 2% of it)."""
    import gemm_inputs as gi
    out = []
    for dtype, shapes in TILE_CHECK.items():
        var_fn = {"f32": dgt.gemm_f32_variant, "bf16": dgt.gemm_bf16_variant}[dtype]
        for (M, N, K) in shapes:
            A = gi.draw(31, M, K, "normal" if dtype == "bf16" else "uniform", dtype=dtype)
            B = gi.draw(32, K, N, "normal" if dtype == "bf16" else "uniform", dtype=dtype)
            dA, dB = to_dev(torch, A, dtype), to_dev(torch, B, dtype)
            dC = torch.zeros((M, N), dtype=torch.float32, device="cuda")
            sptr = torch.cuda.current_stream().cuda_stream
            times = {}
            for rnd in range(3):  # interleaved rounds; the median round counts
                for rung in ("mfma256", "mfma128", "auto"):
                    v = dgt.VARIANTS[rung]

                    def launch(i, v=v):
                        st = var_fn(v, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0,
                                    dC.data_ptr(), N, sptr)
                        if st != 0:
                            raise RuntimeError(dgt.gemm_status_string(st))
                    r = time_calls(torch, launch, steps, warmup if rnd == 0 else 5, 0.0)
                    times.setdefault(rung, []).append(r["ms_avg"])
            med = {k: sorted(v)[1] for k, v in times.items()}
            fastest = min(("mfma256", "mfma128"), key=lambda k: med[k])
            row = {"dtype": dtype, "M": M, "N": N, "K": K,
                   "ms": {k: round(v, 4) for k, v in med.items()},
                   "tflops": {k: round(gemm_flops(M, N, K) / (v * 1e-3) / 1e12, 1)
                              for k, v in med.items()},
                   "faster_tile": fastest,
                   "auto_over_best": round(med["auto"] / med[fastest], 3)}
            out.append(row)
            log(f"[tile-check] {dtype} {M}x{N}x{K}: 256 {med['mfma256']:.4f} ms, "
                f"128 {med['mfma128']:.4f} ms, auto {med['auto']:.4f} ms "
                f"(auto/best {row['auto_over_best']})")
            del dA, dB, dC
            torch.cuda.empty_cache()
    return out


def counter_check(torch, dgt):
    """One call of the naive rung at FP32 2048^3 (chongfengling.github.io
    section 2.3's counter case), for a rocprofv3 counter pass: each wavefront
    of 64 lanes issues one vector load of A and one of B per k, so the
    kernel issues 2 * K * (M*N/64) vector load instructions."""
    import gemm_inputs as gi
    M = N = K = 2048
    A = gi.draw(2048 + 1, M, K, "uniform")
    B = gi.draw(2048 + 2, K, N, "uniform")
    dA, dB = to_dev(torch, A, "f32"), to_dev(torch, B, "f32")
    dC = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    st = dgt.gemm_f32_variant(dgt.VARIANT_NAIVE, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(),
                              N, 0.0, dC.data_ptr(), N, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    if st != 0:
        raise RuntimeError(dgt.gemm_status_string(st))
    print(json.dumps({"counter_check": "naive_kernel<F32>", "M": M, "N": N, "K": K,
                      "wavefronts": M * N // 64,
                      "expected_vector_load_instructions": naive_load_requests(M, N, K, 64),
                      "flops": gemm_flops(M, N, K)}), flush=True)


# ------------------------------------------------------------ main

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    # After an idle period the power-managed clock overshoots and then
    # settles over ~40-80 calls of an 8192^3 GEMM (per-call times 0.82, 1.1,
    # ..., 0.81 ms); each workload first runs untimed for this long.
    ap.add_argument("--settle-ms", type=float, default=300.0)
    # The GPU's telemetry table refreshes about once a second: after the
    # timed calls each workload runs this long again while it is sampled.
    ap.add_argument("--telemetry-s", type=float, default=3.0)
    ap.add_argument("--only", default=None, help="time a single workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--ladder", action="store_true",
                    help="time every rung at FP32 4096^3 and BF16 8192^3")
    ap.add_argument("--counter-check", action="store_true",
                    help="run the naive rung once at FP32 2048^3 (for a counter pass)")
    ap.add_argument("--tile-check", action="store_true",
                    help="time both DMA workgroup tiles and the automatic choice on a set of shapes")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the GEMM "
              "shards by rows or columns with no exchange, so N GPUs run N "
              "independent copies of the single-GPU kernel.", file=sys.stderr)
        return 2

    import torch
    import dense_gemm_tuning_amd as dgt
    import gemm_inputs as gi

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    dgt.library()  # fail loudly if the HIP library is missing

    if args.copy_calibration:
        copy_calibration(torch)
        return 0
    if args.counter_check:
        counter_check(torch, dgt)
        return 0

    tel = Telemetry(torch)
    if tel.error:
        log(f"[telemetry] unavailable: {tel.error}")
    if args.tile_check:
        print(json.dumps({"tile_check": tile_check(torch, dgt, args.steps, args.warmup)}),
              flush=True)
        return 0
    if args.ladder:
        rows = ladder(torch, dgt, args.steps, args.warmup, args.settle_ms, tel, args.telemetry_s)
        print(json.dumps({"ladder": rows, "telemetry_error": tel.error}), flush=True)
        return 0

    names = [args.only] if args.only else [PRIMARY] + SECONDARY
    results = {}
    for name in names:
        w = gi.WORKLOADS[name]
        copies = input_copies(w)
        log(f"[{name}] {w.M}x{w.N}x{w.K} {w.dtype}: settle {args.settle_ms:.0f} ms, "
            f"warmup {args.warmup}, steps {args.steps}")
        res, inputs = time_workload(torch, dgt, w, args.steps, args.warmup, copies,
                                    args.settle_ms, tel, pcie=(name == names[0]),
                                    telemetry_s=args.telemetry_s,
                                    keep_c=(name == names[0] and not args.no_cpu))
        clk = (res.get("clock") or {}).get("gfxclk_mhz")
        res["roofline"] = roofline(w, res["ms_avg"], clk)
        res["tflops"] = gemm_flops(w.M, w.N, w.K) * w.batch / (res["ms_avg"] * 1e-3) / 1e12
        log(f"[{name}] {res['ms_avg']:.4f} ms  {res['tflops']:.1f} TFLOP/s  "
            f"roofline frac {res['roofline']['frac']:.3f}  clock {clk} MHz")
        results[name] = (w, res, inputs if name == names[0] else None)

    head = names[0]
    w, res, (A, B, C0, c_gpu) = results[head]
    cpu = None
    if not args.no_cpu:
        log("[cpu] timing the oracle on a row sample ...")
        cpu = cpu_baseline(w, A, B, C0, c_gpu=c_gpu)
        log(f"[cpu] {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")
        cpu["small_cases"] = cpu_small_cases()

    also = []
    for name in names[1:]:
        w2, r2, _ = results[name]
        entry = {"workload": name, "M": w2.M, "N": w2.N, "K": w2.K, "dtype": w2.dtype,
                 "trans_a": w2.trans_a, "trans_b": w2.trans_b, "batch": w2.batch,
                 "bias": w2.bias, "alpha": w2.alpha, "beta": w2.beta,
                 "ms_per_step": round(r2["ms_avg"], 5),
                 "tflops": round(r2["tflops"], 2), "roofline": r2["roofline"],
                 "clock": r2.get("clock"), "settle_calls": r2["settle_calls"]}
        if streams_b(w2):
            entry["gbs"] = r2["roofline"]["achieved"]
        also.append(entry)

    line = {
        "metric": METRIC,
        "value": round(res["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_avg"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded SplitMix64; bf16/fp16 N(0,1) / fp32 uniform[-1,1))",
        "config": {"workload": head, "M": w.M, "N": w.N, "K": w.K,
                   "alpha": w.alpha, "beta": w.beta,
                   "inputs": w.dtype, "accumulate": "f32", "output": "f32"},
        "settle_ms": args.settle_ms,
        "settle_calls": res["settle_calls"],
        "launch_ms": {k: round(res[k], 5) for k in ("ms_median", "ms_min", "ms_max")},
        "clock": res.get("clock"),
        "telemetry_error": tel.error,
        "pcie": res.get("pcie"),
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
