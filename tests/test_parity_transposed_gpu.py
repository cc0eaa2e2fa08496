"""GPU parity for transposed operand storage (gemm_ex with trans_a / trans_b)
against the CPU oracle, through the C ABI.

op(A) = A^T with A stored K x M, op(B) = B^T with B stored N x K: the storage
of a linear layer's products (elainafan.one "全连接层": X W^T for the forward
pass, G^T X for the weight gradient).  Every rung takes every layout; the
untransposed layout is covered by test_parity_gpu.py.

Gates as there: bit-exact on integer-valued inputs, the normwise /
elementwise tolerance otherwise.  Coverage per layout (NT, TN, TT) x rung x
input type: integer inputs at shapes spanning several tiles, ragged tails and
whole-tile shapes that take the global->LDS DMA kernel (M, N multiples of
256, K of 128); real inputs; row and column selection matrices (a swapped
or mis-transposed fragment cannot pass them); padded and misaligned storage
with a guard band around C; run-to-run determinism on the DMA kernel.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from gates import assert_bit_exact, assert_close
from gpu_util import TORCH_DTYPE, as_input, run_gemm, say, to_dev

torch = pytest.importorskip("torch")
import dense_gemm_tuning_amd as dgt  # noqa: E402

pytestmark = pytest.mark.gpu

RUNGS = ["naive", "lds", "mfma", "mfma_regs", "skinny", "auto"]
DTYPES = ["f32", "bf16", "f16"]
LAYOUTS = {"nt": (False, True), "tn": (True, False), "tt": (True, True)}

SHAPES = [(1, 1, 1), (15, 17, 16), (17, 65, 65), (65, 129, 127), (128, 256, 256),
          (300, 260, 520), (256, 512, 384), (512, 256, 256)]
# Skinny shapes with B stored N x K and several row blocks: a last column
# strip with 44 rows (N = 300) or one (N = 129), and K = 128, a single K step,
# which leaves all but one wave of the workgroup without a step.
SKINNY_SHAPES = [(1, 1, 1), (15, 17, 16), (8, 200, 300), (16, 384, 256), (5, 1000, 129),
                 (17, 130, 96), (33, 384, 256), (48, 257, 300), (64, 512, 512),
                 (40, 300, 512), (20, 1000, 128), (64, 129, 256)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    dgt.library()  # raises if the HIP library is missing: no fallback
    oracle.build(force=False)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def stored(M, N, K, ta, tb):
    """Stored shapes of A and B."""
    return ((K, M) if ta else (M, K)), ((N, K) if tb else (K, N))


def shapes_for(variant):
    return SKINNY_SHAPES if variant == "skinny" else SHAPES


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("variant", RUNGS)
def test_integer_inputs_bit_exact(variant, dtype, layout):
    ta, tb = LAYOUTS[layout]
    for idx, (M, N, K) in enumerate(shapes_for(variant)):
        say(f"int parity {variant} {dtype} {layout} M={M} N={N} K={K}")
        sa, sb = stored(M, N, K, ta, tb)
        A = gi.draw(400 + idx, *sa, "int", dtype=dtype)
        B = gi.draw(500 + idx, *sb, "int", dtype=dtype)
        C0 = gi.draw(600 + idx, M, N, "int")
        for alpha, beta in [(1.0, 0.0), (1.5, 0.5)]:
            c0 = C0 if beta else None
            st, C = run_gemm(variant, dtype, A, B, c0, alpha, beta, trans_a=ta, trans_b=tb)
            assert st == 0, dgt.gemm_status_string(st)
            R = oracle.round_f32(oracle.gemm(A, B, c0, alpha, beta, dtype,
                                             trans_a=ta, trans_b=tb))
            assert_bit_exact(C, R, f"{variant}/{dtype}/{layout} {M}x{N}x{K} a={alpha} b={beta}")


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("variant", RUNGS)
def test_real_inputs_within_tolerance(variant, dtype, layout):
    ta, tb = LAYOUTS[layout]
    dist = "uniform" if dtype == "f32" else "normal"
    cases = ([(16, 1000, 1000, 1.5, 0.5), (50, 640, 1024, 1.0, 0.0)] if variant == "skinny"
             else [(300, 520, 777, 1.0, 0.0), (512, 512, 1024, -0.5, 2.0)])
    for (M, N, K, alpha, beta) in cases:
        say(f"real parity {variant} {dtype} {layout} {M}x{N}x{K}")
        sa, sb = stored(M, N, K, ta, tb)
        A = gi.draw(41, *sa, dist, dtype=dtype)
        B = gi.draw(42, *sb, dist, dtype=dtype)
        C0 = gi.draw(43, M, N, "uniform")
        st, C = run_gemm(variant, dtype, A, B, C0, alpha, beta, trans_a=ta, trans_b=tb)
        assert st == 0
        R = oracle.gemm(A, B, C0, alpha, beta, dtype, trans_a=ta, trans_b=tb)
        assert_close(C, R, K, alpha, what=f"{variant}/{dtype}/{layout} {M}x{N}x{K}")


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("variant", ["mfma", "lds", "skinny"])
def test_selection_matrices(variant, dtype, layout):
    """op(A) = row selection S (S[i, p[i]] = 1): C = rows p of op(B).
    op(B) = column selection T (T[q[j], j] = 1): C = columns q of op(A)."""
    ta, tb = LAYOUTS[layout]
    rng = np.random.default_rng(17)
    shapes = ([(16, 300, 272), (64, 256, 384)] if variant == "skinny"
              else [(256, 256, 256), (130, 70, 130), (512, 256, 384)])
    dist = "uniform" if dtype == "f32" else "normal"
    for (M, N, K) in shapes:
        say(f"selection {variant} {dtype} {layout} {M}x{N}x{K}")
        p = rng.integers(0, K, M)
        S = np.zeros((M, K), np.float32)
        S[np.arange(M), p] = 1.0
        A = as_input(S.T if ta else S, dtype)
        sb = (N, K) if tb else (K, N)
        B = gi.draw(51, *sb, dist, dtype=dtype)
        st, C = run_gemm(variant, dtype, A, B, None, 1.0, 0.0, trans_a=ta, trans_b=tb)
        assert st == 0
        opB = gi.as_fp32(B, dtype)
        opB = opB.T if tb else opB
        assert_bit_exact(C, np.ascontiguousarray(opB[p]), f"row selection {variant}/{dtype}/{layout}")

        q = rng.integers(0, K, N)
        T = np.zeros((K, N), np.float32)
        T[q, np.arange(N)] = 1.0
        B = as_input(T.T if tb else T, dtype)
        sa = (K, M) if ta else (M, K)
        A = gi.draw(52, *sa, dist, dtype=dtype)
        st, C = run_gemm(variant, dtype, A, B, None, 1.0, 0.0, trans_a=ta, trans_b=tb)
        assert st == 0
        opA = gi.as_fp32(A, dtype)
        opA = opA.T if ta else opA
        assert_bit_exact(C, np.ascontiguousarray(opA[:, q]),
                         f"column selection {variant}/{dtype}/{layout}")


def _strided(rows, cols, ld, dtype, offset, fill):
    tdt = getattr(torch, TORCH_DTYPE[dtype])
    base = torch.full((rows * ld + offset + 8,), fill, dtype=tdt, device="cuda")
    return base, base[offset:offset + rows * ld].view(rows, ld)[:, :cols]


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("variant", RUNGS)
@pytest.mark.parametrize("pad,offset", [(8, 0), (3, 0), (8, 1)],
                         ids=["aligned_pad", "odd_pad", "misaligned"])
def test_padded_and_misaligned_storage(variant, dtype, layout, pad, offset):
    """Padded pitches of the stored operands, optionally misaligned bases; C's
    padding and the elements past its end must stay untouched.  The skinny
    rung runs with one row block (8 waves, M = 13) and with three (4 waves,
    M = 40); the other rungs at M = 256."""
    ta, tb = LAYOUTS[layout]
    for M in ([13, 40] if variant == "skinny" else [256]):
        _padded_case(variant, dtype, layout, pad, offset, ta, tb, M)


def _padded_case(variant, dtype, layout, pad, offset, ta, tb, M):
    N, K = 256, 256
    sa, sb = stored(M, N, K, ta, tb)
    A = gi.draw(61, *sa, "int", dtype=dtype)
    B = gi.draw(62, *sb, "int", dtype=dtype)
    C0 = gi.draw(63, M, N, "int")
    say(f"storage {variant} {dtype} {layout} M={M} pad={pad} offset={offset}")
    _, dA = _strided(*sa, sa[1] + pad, dtype, offset, 0.0)
    _, dB = _strided(*sb, sb[1] + pad, dtype, offset, 0.0)
    canary = -12345.0
    ldc = N + pad + 1
    cbase, dC = _strided(M, N, ldc, "f32", offset, canary)
    dA.copy_(to_dev(A, dtype))
    dB.copy_(to_dev(B, dtype))
    dC.copy_(torch.from_numpy(C0).cuda())
    st = dgt.gemm(dA, dB, dC, 1.5, 0.5, variant=variant, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    assert st == 0
    R = oracle.round_f32(oracle.gemm(A, B, C0, 1.5, 0.5, dtype, trans_a=ta, trans_b=tb))
    assert_bit_exact(dC.cpu().numpy(), R, f"strided C, M={M}")
    full = cbase.cpu().numpy()
    mask = np.ones(full.shape, bool)
    body = np.arange(offset, offset + M * ldc).reshape(M, ldc)[:, :N]
    mask[body.ravel()] = False
    assert np.all(full[mask] == canary), f"kernel wrote outside C (M={M})"


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_dma_kernel_deterministic(dtype, layout):
    """Whole tiles take the global->LDS DMA kernel; two runs agree bit for bit
    and match the oracle on real inputs."""
    ta, tb = LAYOUTS[layout]
    M, N, K = 512, 768, 1024
    sa, sb = stored(M, N, K, ta, tb)
    A = gi.draw(71, *sa, "normal", dtype=dtype)
    B = gi.draw(72, *sb, "normal", dtype=dtype)
    outs = []
    for _ in range(2):
        st, C = run_gemm("mfma", dtype, A, B, None, 1.0, 0.0, trans_a=ta, trans_b=tb)
        assert st == 0
        outs.append(C)
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    R = oracle.gemm(A, B, None, 1.0, 0.0, dtype, trans_a=ta, trans_b=tb)
    assert_close(outs[0], R, K, 1.0, what=f"dma {dtype}/{layout}")
