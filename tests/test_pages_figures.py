"""The FLOP and byte model the bench reports against, pinned to numbers the
pages print (tests/golden/pages_figures.json, each with its passage)."""

import json
import os

import pytest

import bench

HERE = os.path.dirname(os.path.abspath(__file__))
FIG = {f["id"]: f for f in json.load(open(os.path.join(HERE, "golden", "pages_figures.json")))["figures"]}


def close(x, fig):
    want, tol = fig["value"], fig["rel_tol"]
    return abs(x - want) <= tol * abs(want) if tol else x == want


def test_flop_count():
    assert close(bench.gemm_flops(2048, 2048, 2048), FIG["flops_2048"])
    assert bench.gemm_flops(2048, 2048, 2048) == 2 * 2048 ** 3


def test_naive_and_tile_intensity():
    assert close(bench.naive_lane_view_intensity(4096), FIG["naive_intensity"])
    assert close(bench.tile_intensity(32), FIG["tile_intensity_T32"])
    assert close(bench.tile_intensity(128), FIG["tile_intensity_T128"])


def test_square_and_gemv_intensity():
    n = 1024
    ai = bench.arithmetic_intensity(bench.gemm_flops(n, n, n),
                                    bench.algorithmic_bytes(n, n, n, 4, 0.0))
    assert close(ai, FIG["square_1024_intensity"])
    # matrix-vector product y = A x with A (M x K) fp32: one output column
    M = K = 1 << 14
    ai = bench.arithmetic_intensity(bench.gemm_flops(M, 1, K),
                                    bench.algorithmic_bytes(M, 1, K, 4, 0.0))
    assert close(ai, FIG["gemv_intensity"])


def test_naive_counter_closed_form():
    # two loads per k per warp of 32 lanes; each 32-lane request touches two
    # 32-byte sectors in the 16 x 16 launch the page profiles
    req = bench.naive_load_requests(2048, 2048, 2048, 32)
    assert close(req, FIG["naive_requests_2048"])
    assert close(2 * req, FIG["naive_sectors_2048"])


def test_skinny_bytes_and_bf16_model():
    # bytes the skinny workload must move: B dominates
    by = bench.algorithmic_bytes(8, 28672, 8192, 2, 0.0)
    assert by == 469762048 + 131072 + 917504


@pytest.mark.parametrize("gpus", [2, 8])
def test_bench_refuses_more_than_one_gpu(gpus, capsys):
    assert bench.main(["--gpus", str(gpus)]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_traffic_lines_parse_kernel_names_with_spaces(tmp_path, monkeypatch):
    """The committed counter summary names kernels such as
    'mfma16_dma_kernel<BF16, NN>'; a line is used only when its source digest
    matches the current kernel source."""
    w = "bf16_8192"
    kern, src, _ = bench.DOMINANT[w]
    assert " " in kern
    dig = bench.source_digest(src)
    f = tmp_path / "hbm.md"
    f.write_text(f"traffic workload={w} kernel={kern} src={dig} fetch_bytes=1000 write_bytes=24\n"
                 f"traffic workload=f32_4096 kernel=x src=0000 fetch_bytes=5 write_bytes=5\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic(w) == 1024
    assert bench.read_traffic("f32_4096") is None  # stale digest
    f.write_text(f"traffic workload={w} kernel={kern} src=ffff fetch_bytes=1000 write_bytes=24\n")
    assert bench.read_traffic(w) is None


def test_cpu_baseline_reports_accuracy_of_a_result():
    """The CPU-baseline leg times the oracle on a row sample and, given the
    GPU's C, reports its error on those rows: zero-ish for the oracle's own
    result rounded to fp32, and a planted error shows up in max_abs."""
    import numpy as np

    import gemm_inputs as gi
    import oracle
    w = gi.WORKLOADS["f32_256"].scaled(M=64, N=96, K=80)
    A, B, C0 = gi.make_inputs(w)
    exact = oracle.round_f32(oracle.gemm(A, B, C0, w.alpha, w.beta, w.dtype))
    r = bench.cpu_baseline(w, A, B, C0, target_s=0.0, c_gpu=exact)
    acc = r["accuracy"]
    assert acc["rows"] >= 8 and acc["normwise_rel"] < 1e-7 and acc["max_abs"] < 1e-6
    bad = exact.copy()
    bad[3, 5] += 0.5
    acc = bench.cpu_baseline(w, A, B, C0, target_s=0.0, c_gpu=bad)["accuracy"]
    assert abs(acc["max_abs"] - 0.5) < 1e-3
    assert acc["gate_max_abs"] == pytest.approx(1e-4 * np.sqrt(80))


def _template_params(src, name):
    """Template parameter count of __global__ kernel `name` in source text."""
    import re
    m = re.search(r"template\s*<([^>]*)>\s*__global__[^;{]*?\b" + name + r"\s*\(", src)
    assert m, f"kernel {name} not found"
    return len([p for p in m.group(1).split(",") if p.strip()])


def test_dominant_kernels_exist_with_their_template_arity():
    """Every bench workload names a dominant kernel whose rocprofv3 pattern
    matches a kernel defined in the named source file, with as many template
    arguments as the definition has (a renamed kernel or a changed template
    would otherwise leave the bench's profile lookups silently empty)."""
    import re
    csrc = os.path.join(os.path.dirname(HERE), "dense_gemm_tuning_amd", "csrc")
    for w in [bench.PRIMARY] + bench.SECONDARY:
        assert w in bench.DOMINANT, w
        _, srcs, pat = bench.DOMINANT[w]
        text = "".join(open(os.path.join(csrc, f)).read() for f in srcs.split("+"))
        m = re.match(r"(\w+)<(.*)>$", pat)
        assert m, (w, pat)
        name, args = m.group(1), m.group(2)
        nargs = len(re.split(r",\s*", args.replace(r"\(dgt::In\)", "")))
        assert _template_params(text, name) == nargs, (w, name, nargs)
