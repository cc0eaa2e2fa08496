"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Gates (tests/gates.py): bit-exact on integer-valued inputs; otherwise
normwise relative error <= 1e-5 and max elementwise error
<= 1e-4 * sqrt(K) * max(1,|alpha|) * sigma_A * sigma_B.

Coverage: every rung (naive, LDS, MFMA, skinny) at sizes spanning several
tiles plus a ragged tail, for fp32, bf16 and fp16 inputs; the workload
shapes in the configuration the
bench times (AUTO), every one checked over the whole of C at its full size
(and the square FP32 4096^3 / BF16 8192^3 ones again on integer inputs, bit
for bit over all of C); ragged and degenerate shapes; padded leading dimensions and
misaligned base pointers; beta == 0 with NaN in C; alpha == 0 and K == 0;
guard bands around C; run-to-run determinism; a non-default stream;
permutation and rank-1 inputs that expose swapped fragment layouts
(dilfish.github.io 5.5 warns these "look right").
"""

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from gates import assert_bit_exact, assert_close
from gpu_util import TORCH_DTYPE, bits16, run_gemm, say, to_dev

torch = pytest.importorskip("torch")
import dense_gemm_tuning_amd as dgt  # noqa: E402

pytestmark = pytest.mark.gpu

RUNGS = ["naive", "lds", "mfma", "mfma_regs", "skinny", "auto"]
DTYPES = ["f32", "bf16", "f16"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    dgt.library()  # raises if the HIP library is missing: no fallback
    oracle.build(force=False)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def supports(variant, M):
    return not (variant == "skinny" and M > 64)


def ints(seed, r, c, dtype):
    return gi.draw(seed, r, c, "int", dtype=dtype)


# ------------------------------------------------------------ exact cases

SHAPES = [
    (1, 1, 1), (2, 3, 5), (15, 17, 16), (16, 64, 63), (17, 65, 65),
    (8, 200, 300), (64, 128, 64), (65, 129, 127), (127, 255, 129),
    (128, 256, 256), (255, 257, 100), (256, 256, 256), (300, 260, 520),
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("variant", RUNGS)
def test_integer_inputs_bit_exact(variant, dtype):
    for idx, (M, N, K) in enumerate(SHAPES):
        if not supports(variant, M):
            continue
        say(f"int parity {variant} {dtype} M={M} N={N} K={K}")
        A, B = ints(100 + idx, M, K, dtype), ints(200 + idx, K, N, dtype)
        C0 = gi.draw(300 + idx, M, N, "int")
        for alpha, beta in [(1.0, 0.0), (1.5, 0.5), (-2.0, 1.0)]:
            st, C = run_gemm(variant, dtype, A, B, C0 if beta else None, alpha, beta)
            assert st == 0, dgt.gemm_status_string(st)
            R = oracle.round_f32(oracle.gemm(A, B, C0 if beta else None, alpha, beta, dtype))
            assert_bit_exact(C, R, f"{variant}/{dtype} {M}x{N}x{K} a={alpha} b={beta}")


# Skinny rung, B stored K x N with a ragged N: the last strip's lanes that
# run past N read the row's last whole piece and repeat a neighbour's
# columns; N = 128 + 3 leaves a last strip narrower than one piece.  Packed
# and padded (odd) pitches of B.
SKINNY_RAGGED = [(8, 131, 256), (16, 1027, 512), (33, 255, 96), (64, 1000, 520), (8, 28671, 64)]


@pytest.mark.parametrize("dtype", DTYPES)
def test_skinny_ragged_columns_bit_exact(dtype):
    for idx, (M, N, K) in enumerate(SKINNY_RAGGED):
        for pad in (0, 1, 8):
            say(f"skinny ragged {dtype} M={M} N={N} K={K} ldb=N+{pad}")
            A = ints(700 + idx, M, K, dtype)
            Bw = ints(710 + idx, K, N + pad, dtype)
            C0 = gi.draw(720 + idx, M, N, "int")
            dA = to_dev(A, dtype)
            dB = to_dev(Bw, dtype)[:, :N]
            dC = torch.from_numpy(C0).cuda()
            st = dgt.gemm(dA, dB, dC, 1.5, 0.5, variant="skinny")
            torch.cuda.synchronize()
            assert st == 0, dgt.gemm_status_string(st)
            R = oracle.round_f32(oracle.gemm(A, np.ascontiguousarray(Bw[:, :N]), C0, 1.5, 0.5,
                                             dtype))
            assert_bit_exact(dC.cpu().numpy(), R, f"skinny ragged {dtype} {M}x{N}x{K} +{pad}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("variant", ["mfma", "lds", "skinny"])
def test_permutation_and_rank1(variant, dtype):
    """Swapped rows/columns or transposed fragments cannot pass these."""
    rng = np.random.default_rng(7)
    one = 1.0 if dtype == "f32" else bits16([1.0], dtype)[0]
    for (M, N, K) in [(16, 300, 272), (256, 256, 256), (130, 70, 130), (48, 300, 272)]:
        if not supports(variant, M):
            continue
        say(f"perm/rank1 {variant} {dtype} {M}x{N}x{K}")
        # A = selection matrix picking row p[i] of B
        p = rng.integers(0, K, M)
        A = np.zeros((M, K), np.float32 if dtype == "f32" else np.uint16)
        A[np.arange(M), p] = one
        B = gi.draw(11, K, N, "uniform" if dtype == "f32" else "normal", dtype=dtype)
        st, C = run_gemm(variant, dtype, A, B, None, 1.0, 0.0)
        assert st == 0
        want = gi.as_fp32(B, dtype)[p]
        assert_bit_exact(C, want, f"row selection {variant}/{dtype}")
        # rank-1 integer outer products: exact closed form
        u, v = rng.integers(-3, 4, M), rng.integers(-3, 4, K)
        w, z = rng.integers(-3, 4, K), rng.integers(-3, 4, N)
        A = np.outer(u, v).astype(np.float32)
        B = np.outer(w, z).astype(np.float32)
        if dtype != "f32":
            A, B = bits16(A, dtype), bits16(B, dtype)
        st, C = run_gemm(variant, dtype, A, B, None, 1.0, 0.0)
        # + 0.0: an exact zero sum of products starting from +0 is +0, while
        # the closed form's 0 * (negative) is -0
        want = (float(np.dot(v, w)) * np.outer(u, z) + 0.0).astype(np.float32)
        assert_bit_exact(C, want, f"rank-1 {variant}/{dtype}")


# ------------------------------------------------------ real-valued gates

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("variant", RUNGS)
def test_real_inputs_within_tolerance(variant, dtype):
    dist = "uniform" if dtype == "f32" else "normal"
    for (M, N, K, alpha, beta) in [(300, 520, 777, 1.0, 0.0), (16, 1000, 1000, 1.5, 0.5),
                                   (513, 257, 1030, -0.5, 2.0), (40, 700, 1000, -1.0, 1.0),
                                   (64, 384, 2048, 1.0, 0.0)]:
        if not supports(variant, M):
            continue
        say(f"real parity {variant} {dtype} {M}x{N}x{K}")
        A = gi.draw(31, M, K, dist, dtype=dtype)
        B = gi.draw(32, K, N, dist, dtype=dtype)
        C0 = gi.draw(33, M, N, "uniform")
        st, C = run_gemm(variant, dtype, A, B, C0, alpha, beta)
        assert st == 0
        R = oracle.gemm(A, B, C0, alpha, beta, dtype)
        assert_close(C, R, K, alpha, what=f"{variant}/{dtype} {M}x{N}x{K}")


# ------------------------------------------------------- workload configs

@pytest.mark.parametrize("name", list(gi.WORKLOADS))
def test_workload_configs(name):
    """Every workload in the launch configuration the bench times, at its full
    size, against the oracle over the whole of C (every problem of a batch)."""
    w = gi.WORKLOADS[name]
    say(f"workload {name}: generating inputs")
    A, B, C0 = gi.make_inputs(w)
    bias = gi.make_bias(w)
    say(f"workload {name}: running AUTO on the GPU")
    if w.streamk:
        # stream-K, as the bench times it
        code = {"f32": dgt.DTYPE_F32, "bf16": dgt.DTYPE_BF16, "f16": dgt.DTYPE_F16}[w.dtype]
        dA, dB = to_dev(A, w.dtype), to_dev(B, w.dtype)
        dC = (torch.from_numpy(np.ascontiguousarray(C0, np.float32)).cuda() if C0 is not None
              else torch.zeros((w.M, w.N), device="cuda"))
        need = dgt.gemm_streamk_workspace_size(code, w.M, w.N, w.K)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        st = dgt.gemm_streamk(code, w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, dA.data_ptr(),
                              A.shape[1], dB.data_ptr(), B.shape[1], w.beta, dC.data_ptr(), w.N,
                              ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        A3, B3, C3 = A[None], B[None], dC.cpu().numpy()[None]
        del dA, dB, dC, ws
    elif w.splits != 1:
        # split-K, as the bench times it
        dC = (torch.from_numpy(np.ascontiguousarray(C0, np.float32)).cuda() if C0 is not None
              else torch.zeros((w.M, w.N), device="cuda"))
        st = dgt.gemm_split(to_dev(A, w.dtype), to_dev(B, w.dtype), dC, w.alpha, w.beta,
                            splits=w.splits, trans_a=w.trans_a, trans_b=w.trans_b)
        torch.cuda.synchronize()
        A3, B3, C3 = A[None], B[None], dC.cpu().numpy()[None]
        del dC
    elif w.batch > 1 or bias is not None:
        # the strided-batch entry point, as the bench times it
        A3 = A if w.batch > 1 else A[None]
        B3 = B if w.batch > 1 else B[None]
        dC = (torch.from_numpy(np.ascontiguousarray(C0, np.float32).reshape(w.batch, w.M, w.N))
              .cuda() if C0 is not None else torch.zeros((w.batch, w.M, w.N), device="cuda"))
        dbias = None if bias is None else torch.from_numpy(bias).cuda()
        st = dgt.gemm_batched(to_dev(A3, w.dtype), to_dev(B3, w.dtype), dC, w.alpha, w.beta,
                              bias=dbias, trans_a=w.trans_a, trans_b=w.trans_b)
        torch.cuda.synchronize()
        C3 = dC.cpu().numpy()
        del dC
    else:
        st, C = run_gemm("auto", w.dtype, A, B, C0, w.alpha, w.beta, trans_a=w.trans_a,
                         trans_b=w.trans_b)
        A3, B3, C3 = A[None], B[None], C[None]
    torch.cuda.empty_cache()
    assert st == 0
    C0s = None if C0 is None else np.asarray(C0, np.float32).reshape(w.batch, w.M, w.N)
    for z in range(w.batch):
        say(f"workload {name}: oracle on all {w.M} rows of problem {z}")
        R = oracle.gemm(A3[z], B3[z], None if C0s is None else C0s[z], w.alpha, w.beta, w.dtype,
                        trans_a=w.trans_a, trans_b=w.trans_b,
                        bias=None if bias is None else bias[z])
        rel, mx = assert_close(C3[z], R, w.K, w.alpha, w.sigma, w.sigma, what=f"{name}[{z}]")
        say(f"workload {name}[{z}]: normwise {rel:.3e}, max abs {mx:.3e} over {C3[z].size} "
            "elements")
        del R


# Integer-valued variants (entries in {-3..3}): every partial sum is exact,
# so the device result must equal the oracle's bit for bit over all of C, at
# the full sizes of the small, ragged, square and skinny workloads.
@pytest.mark.parametrize("name", ["f32_256", "f32_1000_ragged", "f32_4096", "bf16_8192",
                                  "bf16_skinny_8x28672x8192", "bf16_skinny_8x28672x8192_nt",
                                  "f32_skinny_8x28672x8192_nt"])
def test_workload_integer_variants(name):
    w = gi.WORKLOADS[name].with_ints()
    A, B, C0 = gi.make_inputs(w)
    say(f"integer workload {w.name} {w.M}x{w.N}x{w.K}")
    st, C = run_gemm("auto", w.dtype, A, B, C0, w.alpha, w.beta, trans_a=w.trans_a,
                     trans_b=w.trans_b)
    torch.cuda.empty_cache()
    assert st == 0
    R = oracle.round_f32(oracle.gemm(A, B, C0, w.alpha, w.beta, w.dtype,
                                     trans_a=w.trans_a, trans_b=w.trans_b))
    assert_bit_exact(C, R, w.name)
    say(f"integer workload {w.name}: {C.size} elements bit-exact")


# -------------------------------------------------------------- semantics

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("variant", RUNGS)
def test_alpha_zero_and_k_zero(variant, dtype):
    M, N = (16 if variant == "skinny" else 70), 90
    C0 = gi.draw(41, M, N, "uniform")
    A, B = ints(42, M, 33, dtype), ints(43, 33, N, dtype)
    st, C = run_gemm(variant, dtype, A, B, C0, 0.0, -1.5)
    assert st == 0
    assert_bit_exact(C, (-1.5 * C0.astype(np.float64)).astype(np.float32), "alpha=0")
    A0 = np.zeros((M, 0), A.dtype)
    B0 = np.zeros((0, N), B.dtype)
    st, C = run_gemm(variant, dtype, A0, B0, C0, 1.0, 0.5)
    assert st == 0
    assert_bit_exact(C, (0.5 * C0.astype(np.float64)).astype(np.float32), "K=0")
    st, C = run_gemm(variant, dtype, A0, B0, C0, 1.0, 0.0)
    assert st == 0 and np.all(C == 0.0)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("variant", RUNGS)
def test_beta_zero_ignores_nan_in_c(variant, dtype):
    M, N, K = (8 if variant == "skinny" else 200), 300, 64
    A, B = ints(51, M, K, dtype), ints(52, K, N, dtype)
    st, C = run_gemm(variant, dtype, A, B, None, 1.0, 0.0)  # C prefilled with NaN
    assert st == 0
    assert np.all(np.isfinite(C))
    assert_bit_exact(C, oracle.round_f32(oracle.gemm(A, B, None, 1.0, 0.0, dtype)), "beta=0")


def _strided(shape, ld, dtype, offset_elems, fill):
    """A device tensor view with row pitch ld and a base offset in elements."""
    rows, cols = shape
    tdt = torch.float32 if dtype == "f32" else getattr(torch, TORCH_DTYPE[dtype])
    base = torch.full((rows * ld + offset_elems + 8,), fill, dtype=tdt, device="cuda")
    return base, base[offset_elems:offset_elems + rows * ld].view(rows, ld)[:, :cols]


# (row pitch padding, base offset in elements): padded rows that keep every
# row 16-byte aligned (vector path), odd padding, and a misaligned base.
LAYOUTS = {"aligned_pad": (8, 0), "odd_pad": (3, 0), "misaligned": (8, 1)}


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("variant", RUNGS)
@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_leading_dims_alignment_and_guard_band(variant, dtype, layout):
    """Padded lda/ldb/ldc, optionally misaligned bases; the padding of C and the
    elements past its end must stay untouched (canaries)."""
    pad, offset = LAYOUTS[layout]
    M, N, K = (13 if variant == "skinny" else 150), 200, 192
    lda, ldb, ldc = K + pad, N + pad, N + pad + 1
    A, B = ints(61, M, K, dtype), ints(62, K, N, dtype)
    C0 = gi.draw(63, M, N, "int")
    say(f"ld/alignment {variant} {dtype} {layout}")
    _, dA = _strided((M, K), lda, dtype, offset, 0.0)
    _, dB = _strided((K, N), ldb, dtype, offset, 0.0)
    canary = -12345.0
    cbase, dC = _strided((M, N), ldc, "f32", offset, canary)
    dA.copy_(to_dev(A, dtype))
    dB.copy_(to_dev(B, dtype))
    dC.copy_(torch.from_numpy(C0).cuda())
    st = dgt.gemm(dA, dB, dC, 1.5, 0.5, variant=variant)
    torch.cuda.synchronize()
    assert st == 0
    R = oracle.round_f32(oracle.gemm(A, B, C0, 1.5, 0.5, dtype))
    assert_bit_exact(dC.cpu().numpy(), R, "strided C")
    full = cbase.cpu().numpy()
    mask = np.ones(full.shape, bool)
    body = np.arange(offset, offset + M * ldc).reshape(M, ldc)[:, :N]
    mask[body.ravel()] = False
    assert np.all(full[mask] == canary), "kernel wrote outside C"


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("variant", ["mfma", "lds", "skinny"])
def test_deterministic_and_stream(variant, dtype):
    M, N, K = (16 if variant == "skinny" else 384), 640, 1000
    dist = "uniform" if dtype == "f32" else "normal"
    A = to_dev(gi.draw(71, M, K, dist, dtype=dtype), dtype)
    B = to_dev(gi.draw(72, K, N, dist, dtype=dtype), dtype)
    s = torch.cuda.Stream()
    outs = []
    for _ in range(2):
        C = torch.zeros((M, N), device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            assert dgt.gemm(A, B, C, 1.0, 0.0, variant=variant, stream=s) == 0
        s.synchronize()
        outs.append(C.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), \
        "two runs differ: a race in the LDS pipeline?"


def test_status_codes_on_gpu():
    A = torch.zeros((4, 4), device="cuda")
    C = torch.zeros((4, 4), device="cuda")
    assert dgt.gemm(A, A, C, variant="skinny") == 0
    big = torch.zeros((65, 4), device="cuda")
    assert dgt.gemm(big, A, torch.zeros((65, 4), device="cuda"), variant="skinny") == dgt.GEMM_ERR_VARIANT
    assert dgt.gemm(A, A, A) == dgt.GEMM_ERR_OVERLAP
