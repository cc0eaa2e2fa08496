"""GPU parity for the whole-tile BF16/FP16 path on shapes that are not whole
tiles, against the CPU oracle, through the C ABI.

M and N that are not multiples of the workgroup tile (256 or 128; the
fixed-tile rungs run each) run the global->LDS DMA kernel with edge tiles: the copy descriptors' ranges stop at each operand's last
element and the epilogue stores only rows < M and columns < N.  Any K runs
there too: when K is not a multiple of 128 the last group of 1 to 4 slices
runs after the main loop, and in a partial last slice the k-contiguous
fragments are masked past K element by element while m/n-contiguous rows
past K read as zeros through the copy range.  Covered, for every stored
layout: integer inputs bit-exact (K = 5 .. 1096, with and without a partial
slice, with half a k-contiguous pair, and with K not a multiple of 8 on
padded storage), a guard band around a padded C (nothing outside C is
written), the bias added once, beta = 0 never reading a NaN-filled C, real
inputs within the gates, a large ragged shape on sampled rows, and
run-to-run determinism.  Shapes whose stored rows are not 16-byte aligned
take the register-staged kernel.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from gates import assert_bit_exact, assert_close
from gpu_util import TORCH_DTYPE, run_gemm, say, to_dev

torch = pytest.importorskip("torch")
import dense_gemm_tuning_amd as dgt  # noqa: E402

pytestmark = pytest.mark.gpu

LAYOUTS = {"nn": (False, False), "nt": (False, True), "tn": (True, False), "tt": (True, True)}

# (M, N, K): edge tiles with K a multiple of 128, including eight rows and
# eight columns; K a multiple of 32 only (32, 96 and 224: one, three and
# seven slices, ending in half a k-contiguous pair when odd); K with a
# partial last slice (200, 1000, 136, 1096: 8 of 32 k valid).  Stored row
# lengths are multiples of 8 elements (16-byte rows, which the DMA kernel
# needs); (300, 260, 520) is not, and takes the register-staged kernel.
EDGE = [(296, 264, 512), (264, 1000, 256), (1000, 296, 384), (8, 704, 128), (520, 8, 256)]
RAGGED_K = [(256, 256, 32), (512, 512, 96), (296, 264, 224), (512, 512, 200),
            (296, 264, 1000), (256, 384, 136), (72, 4096, 1096), (300, 260, 520)]


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
    return ((K, M) if ta else (M, K)), ((N, K) if tb else (K, N))


@pytest.mark.parametrize("tile", ["mfma256", "mfma128"])
@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_edge_and_ragged_k_integer_bit_exact(dtype, layout, tile):
    """Every shape with both workgroup tiles (the fixed-tile rungs), except
    the one whose rows are not 16-byte aligned, which runs the automatic
    choice (the register-staged kernel)."""
    ta, tb = LAYOUTS[layout]
    for idx, (M, N, K) in enumerate(EDGE + RAGGED_K):
        sa, sb = stored(M, N, K, ta, tb)
        aligned = sa[1] % 8 == 0 and sb[1] % 8 == 0
        A = gi.draw(1600 + idx, *sa, "int", dtype=dtype)
        B = gi.draw(1700 + idx, *sb, "int", dtype=dtype)
        C0 = gi.draw(1800 + idx, M, N, "int")
        for alpha, beta in [(1.0, 0.0), (1.5, 0.5)]:
            c0 = C0 if beta else None  # beta = 0: C starts NaN and must not be read
            say(f"edge {dtype} {layout} {tile} {M}x{N}x{K} a={alpha} b={beta}")
            st, C = run_gemm(tile if aligned else "mfma", dtype, A, B, c0, alpha, beta,
                             trans_a=ta, trans_b=tb)
            assert st == 0, dgt.gemm_status_string(st)
            R = oracle.round_f32(oracle.gemm(A, B, c0, alpha, beta, dtype, trans_a=ta,
                                             trans_b=tb))
            assert_bit_exact(C, R, f"{dtype}/{layout} {M}x{N}x{K} a={alpha} b={beta}")


@pytest.mark.parametrize("tile", ["mfma256", "mfma128"])
@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_k_not_multiple_of_8_on_padded_storage(layout, tile):
    """Pitches padded to multiples of 8 elements keep 16-byte rows, so K that
    is not a multiple of 8 still runs the DMA kernel: the last slice's
    fragments are masked element by element (K = 5 and 77 fit in one or
    three slices)."""
    ta, tb = LAYOUTS[layout]
    for idx, (M, N, K) in enumerate([(296, 264, 1001), (264, 520, 999), (300, 256, 77),
                                     (256, 300, 5)]):
        sa, sb = stored(M, N, K, ta, tb)
        A = gi.draw(2300 + idx, *sa, "int", dtype="bf16")
        B = gi.draw(2400 + idx, *sb, "int", dtype="bf16")
        C0 = gi.draw(2500 + idx, M, N, "int")

        def padded(X):
            rows, cols = X.shape
            ld = (cols + 7) // 8 * 8 + 8
            t = torch.zeros((rows, ld), dtype=torch.bfloat16, device="cuda")
            t[:, :cols] = to_dev(X, "bf16")
            return t[:, :cols]

        dA, dB = padded(A), padded(B)
        dC = torch.from_numpy(C0).cuda()
        say(f"padded K {layout} {tile} {M}x{N}x{K}")
        st = dgt.gemm(dA, dB, dC, 1.5, 0.5, variant=tile, trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        assert st == 0, dgt.gemm_status_string(st)
        R = oracle.round_f32(oracle.gemm(A, B, C0, 1.5, 0.5, "bf16", trans_a=ta, trans_b=tb))
        assert_bit_exact(dC.cpu().numpy(), R, f"padded K {layout} {M}x{N}x{K}")


@pytest.mark.parametrize("tile", ["mfma256", "mfma128"])
@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_edge_guard_band(layout, tile):
    """C padded (ldc > N) inside a canary-filled buffer: an edge tile stores
    only its valid part, so the padding and the elements after C keep the
    canary; the same with a K remainder (two passes over C)."""
    ta, tb = LAYOUTS[layout]
    for (M, N, K) in [(296, 264, 512), (296, 264, 520)]:
        sa, sb = stored(M, N, K, ta, tb)
        A = gi.draw(1900, *sa, "int", dtype="bf16")
        B = gi.draw(1901, *sb, "int", dtype="bf16")
        C0 = gi.draw(1902, M, N, "int")
        ldc, canary = N + 13, -4242.0
        base = torch.full((M * ldc + 300,), canary, device="cuda")
        dC = base[:M * ldc].view(M, ldc)[:, :N]
        dC.copy_(torch.from_numpy(C0).cuda())
        say(f"edge guard band {layout} {tile} {M}x{N}x{K}")
        st = dgt.gemm(to_dev(A, "bf16"), to_dev(B, "bf16"), dC, 1.5, 0.5, variant=tile,
                      trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        assert st == 0
        full = base.cpu().numpy()
        mask = np.ones(full.shape, bool)
        mask[np.arange(M * ldc).reshape(M, ldc)[:, :N].ravel()] = False
        assert np.all(full[mask] == canary), "an edge tile wrote outside C"
        R = oracle.round_f32(oracle.gemm(A, B, C0, 1.5, 0.5, "bf16", trans_a=ta, trans_b=tb))
        assert_bit_exact(dC.cpu().numpy(), R, f"guard band {layout} {M}x{N}x{K}")


@pytest.mark.parametrize("layout", ["nn", "nt"])
def test_ragged_k_bias_added_once(layout):
    """With a partial last slice the bias is still added once, by the
    epilogue, for every problem of a strided batch."""
    ta, tb = LAYOUTS[layout]
    M, N, K, batch = 296, 264, 1000, 3
    sa, sb = stored(M, N, K, ta, tb)
    A = gi.draw(2000, batch * sa[0], sa[1], "int", dtype="bf16").reshape(batch, *sa)
    B = gi.draw(2001, batch * sb[0], sb[1], "int", dtype="bf16").reshape(batch, *sb)
    C0 = gi.draw(2002, batch * M, N, "int").reshape(batch, M, N)
    bias = gi.draw(2003, batch, N, "int")
    dC = torch.from_numpy(np.ascontiguousarray(C0)).cuda()
    say(f"ragged K with bias {layout} batch {batch}")
    st = dgt.gemm_batched(to_dev(A, "bf16"), to_dev(B, "bf16"), dC, 1.5, 0.5,
                          bias=torch.from_numpy(bias).cuda(), trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    assert st == 0
    R = oracle.gemm_batched(A, B, C0, 1.5, 0.5, "bf16", trans_a=ta, trans_b=tb, biases=bias)
    assert_bit_exact(dC.cpu().numpy(), oracle.round_f32(R), f"bias {layout}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_edge_real_inputs(dtype):
    for (M, N, K, alpha, beta) in [(2000, 1504, 1024, 1.0, 0.0), (1496, 2000, 1000, -0.5, 2.0)]:
        say(f"edge real {dtype} {M}x{N}x{K}")
        A = gi.draw(2100, M, K, "normal", dtype=dtype)
        B = gi.draw(2101, K, N, "normal", dtype=dtype)
        C0 = gi.draw(2102, M, N, "uniform")
        st, C = run_gemm("auto", dtype, A, B, C0, alpha, beta)
        assert st == 0
        R = oracle.gemm(A, B, C0, alpha, beta, dtype)
        assert_close(C, R, K, alpha, what=f"edge real {dtype} {M}x{N}x{K}")


def test_large_ragged_sampled_rows_and_determinism():
    """8000^3: edge tiles in M and N and 250 slices of 32 (the last group
    runs after the loop); sampled rows against the oracle, and two runs bit
    for bit."""
    M = N = K = 8000
    A = gi.draw(2200, M, K, "normal", dtype="bf16")
    B = gi.draw(2201, K, N, "normal", dtype="bf16")
    dA, dB = to_dev(A, "bf16"), to_dev(B, "bf16")
    outs = []
    for _ in range(2):
        dC = torch.full((M, N), float("nan"), device="cuda")
        assert dgt.gemm(dA, dB, dC, 1.0, 0.0) == 0
        torch.cuda.synchronize()
        outs.append(dC.cpu().numpy())
        del dC
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    rows = [0, 1, 255, 256, 4000, 7679, 7680, 7998, 7999]
    say(f"large ragged: oracle on {len(rows)} rows")
    R = oracle.gemm(A[rows], B, None, 1.0, 0.0, "bf16")
    assert_close(outs[0][rows], R, K, 1.0, what="8000^3 sampled rows")
    assert np.all(np.isfinite(outs[0]))
