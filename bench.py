#!/usr/bin/env python3
"""Throughput of the gfx950 dense GEMM library on one MI355X.

One step = one GEMM call C = alpha*A*B + beta*C on the headline workload
(BF16 inputs, FP32 accumulate/output, M = N = K = 8192), inputs already
resident in HBM.  W untimed warm-up calls (the pages ask for warm-up before
quoting numbers: dilfish.github.io 5.7; here they also let the power-managed
clock settle, which takes some 40-80 calls of the 8192^3 GEMM after the GPU
has idled while the next inputs were generated), then K timed calls
bracketed by device synchronisation, timed with HIP events on the stream the
kernels run on.  TFLOP/s = 2MNK / time (chongfengling.github.io section 1 counts K
multiplies and K adds per output; 2*2048^3 = 17.18e9 in its section 2.5).

The same JSON line carries, under "also", the FP32 4096^3 case (against the
fp32 matrix-core peak), the FP16-input 8192^3 case (against the fp16 peak,
equal to bf16's), the skinny decode-shaped case M=8, N=28672,
K=8192 (against HBM bandwidth: its time is the time to stream B once,
dilfish.github.io 5.1 GEMV row), the BF16 square and skinny cases with a
linear layer's operand storage (B stored N x K, A stored K x M), that
layer's forward with its bias fused, and a strided batch of 16 x 2048^3,
plus:
  * "roofline": the dominant kernel's algorithmic FLOP per launch over its
    measured launch time, against the published MI355X peak;
  * "cpu_baseline": the CPU oracle timed on a bounded row sample of the same
    workload on this host's cores (a reported baseline, not a target).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --only bf16_8192 --no-cpu   (one workload, for profiling)
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
SECONDARY = ["f32_4096", "f16_8192", "bf16_skinny_8x28672x8192", "bf16_8192_nt",
             "bf16_8192_tn", "bf16_skinny_8x28672x8192_nt", "bf16_linear_bias_8192_nt",
             "bf16_bmm_16x2048", "bf16_decode_64x28672x8192_nt", "f32_1000_splitk",
             "bf16_splitk_1024x1024x16384", "bf16_skinny_shard_8x3584x8192",
             "bf16_shard_8192x1024x8192"]

# Kernel that dominates each workload's time, for the roofline: a readable
# name, its source file, and a pattern for the name rocprofv3 prints (the
# template arguments: input format, then vector / guard flags where the
# kernel has them, then trans_a, trans_b; the DMA GEMM kernels' end with
# their edge-tile and K-tail flags, false for whole tiles; the skinny DMA
# kernel's are the row-block count, waves, ring stages, step depth and
# whether A has one register buffer).
DOMINANT = {
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
    "bf16_skinny_8x28672x8192_nt": ("skinny16_bt_dma_kernel<BF16, 1 row block, 8 waves>",
                                    "k_skinny16_dma.hip",
                                    r"skinny16_bt_dma_kernel<\(dgt::In\)1, 1, 8, 2, 128, false>"),
    "bf16_linear_bias_8192_nt": ("mfma16_dma_kernel<BF16, NT> + bias", "k_mfma_bf16_dma.hip",
                                 r"mfma16_dma_kernel<\(dgt::In\)1, 256, false, true, false, false>"),
    "bf16_decode_64x28672x8192_nt": ("skinny16_bt_dma_kernel<BF16, 4 row blocks, 8 waves>",
                                     "k_skinny16_dma.hip",
                                     r"skinny16_bt_dma_kernel<\(dgt::In\)1, 4, 8, 4, 64, true>"),
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
    joined by '+', with the headers they include."""
    h = hashlib.sha256()
    files = fname.split("+")
    extra = (("skinny_common.hpp",) if any(f.startswith("k_skinny") for f in files) else ()) + \
        (("dma_common.hpp",) if any(f.endswith("_dma.hip") for f in files) else ())
    for f in (*files, "gemm_common.hpp", *extra):
        with open(os.path.join(ROOT, "dense_gemm_tuning_amd", "csrc", f), "rb") as fh:
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


def time_workload(torch, dgt, w, steps, warmup, copies=1):
    """Average and spread of one GEMM call's duration (ms) on the current stream."""
    import gemm_inputs as gi
    t0 = time.perf_counter()
    A, B, C0 = gi.make_inputs(w)
    log(f"[{w.name}] inputs generated in {time.perf_counter() - t0:.1f} s")
    bias = gi.make_bias(w)
    dA = [to_dev(torch, A, w.dtype) for _ in range(copies)]
    dB = [to_dev(torch, B, w.dtype) for _ in range(copies)]
    dC = (torch.from_numpy(C0).cuda() if C0 is not None
          else torch.zeros((w.batch, w.M, w.N), dtype=torch.float32, device="cuda"))
    dbias = torch.from_numpy(bias).cuda() if bias is not None else None
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    lda, ldb = w.a_shape[1], w.b_shape[1]  # packed stored rows
    code = {"f32": dgt.DTYPE_F32, "bf16": dgt.DTYPE_BF16, "f16": dgt.DTYPE_F16}[w.dtype]
    if w.splits != 1:
        need = dgt.gemm_splitk_workspace_size(code, w.M, w.N, w.K, w.splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")  # outside the timing

        def fn(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s):
            return dgt.gemm_splitk(code, w.trans_a, w.trans_b, M, N, K, alpha, A, lda, B, ldb,
                                   beta, C, ldc, w.splits, ws.data_ptr(), need, s)
    elif w.batch > 1 or bias is not None:
        def fn(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s):
            return dgt.gemm_strided_batched(
                code, w.trans_a, w.trans_b, dgt.VARIANT_AUTO, M, N, K, alpha,
                A, lda, w.a_shape[0] * lda, B, ldb, w.b_shape[0] * ldb, beta, C, ldc, M * N,
                dbias.data_ptr() if dbias is not None else 0, N, w.batch, s)
    elif w.trans_a or w.trans_b:
        def fn(*args):
            return dgt.gemm_ex(code, w.trans_a, w.trans_b, dgt.VARIANT_AUTO, *args)
    else:
        fn = {"f32": dgt.gemm_f32, "bf16": dgt.gemm_bf16, "f16": dgt.gemm_f16}[w.dtype]

    def launch(i):
        st = fn(w.M, w.N, w.K, w.alpha, dA[i % copies].data_ptr(), lda,
                dB[i % copies].data_ptr(), ldb, w.beta, dC.data_ptr(), w.N, sptr)
        if st != 0:
            raise RuntimeError(dgt.gemm_status_string(st))

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    # timed region: K back-to-back launches between one pair of events
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    # spread: a second pass with an event after every launch (the markers add
    # a little time of their own, so this pass does not feed the average)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        launch(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    res = {"ms_avg": total / steps, "ms_median": per[len(per) // 2],
           "ms_min": per[0], "ms_max": per[-1]}
    del dA, dB, dC
    torch.cuda.empty_cache()
    return res, (A, B, C0)


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


def roofline(w, ms_avg):
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
    return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic,
            "kernel": kern, "algorithmic_flops": fl}


def cpu_baseline(w, A, B, C0, target_s=12.0):
    """The oracle as it stands, on a row sample sized for ~target_s seconds."""
    import oracle
    oracle.build(force=False)
    rows = 8
    while True:
        t0 = time.perf_counter()
        oracle.gemm(A[:rows], B, None if C0 is None else C0[:rows], w.alpha, w.beta, w.dtype)
        dt = time.perf_counter() - t0
        if dt >= target_s / 3 or rows >= w.M:
            break
        rows = min(w.M, max(rows * 2, int(rows * target_s / max(dt, 1e-3))))
    fl = gemm_flops(rows, w.N, w.K)
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {rows} of {w.M} rows of {w.name} "
                      f"({rows}x{w.N}x{w.K}, {dt:.1f} s incl. fp64 widening of B)"}


def copy_calibration(torch, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling HBM byte counters."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes,
                      "copy_calibration_bytes_written": nbytes, "reps": reps}))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The power-managed clock overshoots and then settles over the first
    # ~40-80 launches of an 8192^3 GEMM after the GPU has idled (per-launch
    # times 0.82, 1.1, ..., 0.81 ms); 100 untimed launches reach steady state.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--only", default=None, help="time a single workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
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

    names = [args.only] if args.only else [PRIMARY] + SECONDARY
    results = {}
    for name in names:
        w = gi.WORKLOADS[name]
        copies = input_copies(w)
        log(f"[{name}] {w.M}x{w.N}x{w.K} {w.dtype}: warmup {args.warmup}, steps {args.steps}")
        res, inputs = time_workload(torch, dgt, w, args.steps, args.warmup, copies)
        res["roofline"] = roofline(w, res["ms_avg"])
        res["tflops"] = gemm_flops(w.M, w.N, w.K) * w.batch / (res["ms_avg"] * 1e-3) / 1e12
        log(f"[{name}] {res['ms_avg']:.4f} ms  {res['tflops']:.1f} TFLOP/s  "
            f"roofline frac {res['roofline']['frac']:.3f}")
        results[name] = (w, res, inputs)

    head = names[0]
    w, res, (A, B, C0) = results[head]
    cpu = None
    if not args.no_cpu:
        log("[cpu] timing the oracle on a row sample ...")
        cpu = cpu_baseline(w, A, B, C0)
        log(f"[cpu] {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")

    also = []
    for name in names[1:]:
        w2, r2, _ = results[name]
        entry = {"workload": name, "M": w2.M, "N": w2.N, "K": w2.K, "dtype": w2.dtype,
                 "trans_a": w2.trans_a, "trans_b": w2.trans_b, "batch": w2.batch,
                 "bias": w2.bias, "ms_per_step": round(r2["ms_avg"], 5),
                 "tflops": round(r2["tflops"], 2), "roofline": r2["roofline"]}
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
        "launch_ms": {k: round(res[k], 5) for k in ("ms_median", "ms_min", "ms_max")},
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
