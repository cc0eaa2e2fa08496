"""GPU parity for the FP32 whole-tile DMA kernel (256 x 256 tiles, one
wavefront per SIMD) against the CPU oracle, through the C ABI.

The automatic choice takes that kernel for 16-byte aligned rows when a
model of both kernels' waves of tiles says it finishes first (a strided
batch counts every problem's tiles: 256 tiles of 256 x 256 against at least
513 of 128 x 128 qualifies); the cases below meet that with one 4096 x 4096
or 4000 x 4000 problem, or with batches of small ones.  Covered, for every
stored layout: integer inputs bit-exact on whole tiles (K = 64, 128 and 192:
one to three groups of four 16-deep slices), on edge tiles, and with K not
a multiple of 64 (a last group of 1 to 4 slices) or of 16 (a partial last
slice, masked) or of 4 (on padded storage); alpha / beta, the bias, a C
pitch padded inside a canary-filled buffer, real inputs within the gates,
and run-to-run determinism.  The smaller shapes of the other FP32 tests take
the 128 x 128 register-staged kernel.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from gates import assert_bit_exact, assert_close
from gpu_util import say, to_dev

torch = pytest.importorskip("torch")
import dense_gemm_tuning_amd as dgt  # noqa: E402

pytestmark = pytest.mark.gpu

LAYOUTS = {"nn": (False, False), "nt": (False, True), "tn": (True, False), "tt": (True, True)}


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


@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_one_problem_integer_bit_exact(layout):
    """4096 x 4096 (256 tiles) with K = 64 and 192."""
    ta, tb = LAYOUTS[layout]
    M = N = 4096
    for idx, K in enumerate([64, 192]):
        sa, sb = stored(M, N, K, ta, tb)
        A = gi.draw(3100 + idx, *sa, "int")
        B = gi.draw(3200 + idx, *sb, "int")
        C0 = gi.draw(3300 + idx, M, N, "int")
        dA, dB = to_dev(A, "f32"), to_dev(B, "f32")
        for alpha, beta in [(1.0, 0.0), (1.5, 0.5)]:
            say(f"f32 dma {layout} {M}x{N}x{K} a={alpha} b={beta}")
            dC = (torch.from_numpy(C0).cuda() if beta else
                  torch.full((M, N), float("nan"), device="cuda"))
            st = dgt.gemm(dA, dB, dC, alpha, beta, trans_a=ta, trans_b=tb)
            torch.cuda.synchronize()
            assert st == 0, dgt.gemm_status_string(st)
            R = oracle.round_f32(oracle.gemm(A, B, C0 if beta else None, alpha, beta, "f32",
                                             trans_a=ta, trans_b=tb))
            assert_bit_exact(dC.cpu().numpy(), R, f"f32 dma {layout} {M}x{N}x{K}")
            del dC


@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_batch_of_small_problems_with_bias(layout):
    """256 problems of 256 x 256 x 128 (one tile each), bias per problem."""
    ta, tb = LAYOUTS[layout]
    M = N = 256
    K, batch = 128, 256
    sa, sb = stored(M, N, K, ta, tb)
    A = gi.draw(3400, batch * sa[0], sa[1], "int").reshape(batch, *sa)
    B = gi.draw(3401, batch * sb[0], sb[1], "int").reshape(batch, *sb)
    C0 = gi.draw(3402, batch * M, N, "int").reshape(batch, M, N)
    bias = gi.draw(3403, batch, N, "int")
    dC = torch.from_numpy(np.ascontiguousarray(C0)).cuda()
    say(f"f32 dma batch {layout} {batch} x {M}x{N}x{K} with bias")
    st = dgt.gemm_batched(to_dev(A, "f32"), to_dev(B, "f32"), dC, 1.5, 0.5,
                          bias=torch.from_numpy(bias).cuda(), trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    assert st == 0, dgt.gemm_status_string(st)
    R = oracle.gemm_batched(A, B, C0, 1.5, 0.5, "f32", trans_a=ta, trans_b=tb, biases=bias)
    assert_bit_exact(dC.cpu().numpy(), oracle.round_f32(R), f"f32 dma batch {layout}")


@pytest.mark.parametrize("layout", ["nn", "tt"])
def test_padded_pitches_and_guard_band(layout):
    """Operand pitches padded by 16 floats, C by 40 inside a canary-filled
    buffer: only C's elements change."""
    ta, tb = LAYOUTS[layout]
    M = N = 4096
    K = 128
    sa, sb = stored(M, N, K, ta, tb)
    A = gi.draw(3500, *sa, "int")
    B = gi.draw(3501, *sb, "int")
    C0 = gi.draw(3502, M, N, "int")

    def padded(X, pad):
        t = torch.zeros((X.shape[0], X.shape[1] + pad), device="cuda")
        t[:, :X.shape[1]] = torch.from_numpy(X).cuda()
        return t[:, :X.shape[1]]

    ldc, canary = N + 40, -4242.0
    base = torch.full((M * ldc + 500,), canary, device="cuda")
    dC = base[:M * ldc].view(M, ldc)[:, :N]
    dC.copy_(torch.from_numpy(C0).cuda())
    say(f"f32 dma padded {layout}")
    st = dgt.gemm(padded(A, 16), padded(B, 16), dC, 1.5, 0.5, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    assert st == 0, dgt.gemm_status_string(st)
    full = base.cpu().numpy()
    mask = np.ones(full.shape, bool)
    mask[np.arange(M * ldc).reshape(M, ldc)[:, :N].ravel()] = False
    assert np.all(full[mask] == canary), "the kernel wrote outside C"
    R = oracle.round_f32(oracle.gemm(A, B, C0, 1.5, 0.5, "f32", trans_a=ta, trans_b=tb))
    assert_bit_exact(dC.cpu().numpy(), R, f"f32 dma padded {layout}")


@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_real_inputs_and_determinism(layout):
    """Uniform inputs, 4096 x 4096 x 1024 against the oracle; two runs bit
    for bit."""
    ta, tb = LAYOUTS[layout]
    M = N = 4096
    K = 1024
    sa, sb = stored(M, N, K, ta, tb)
    A = gi.draw(3600, *sa, "uniform")
    B = gi.draw(3601, *sb, "uniform")
    dA, dB = to_dev(A, "f32"), to_dev(B, "f32")
    outs = []
    for _ in range(2):
        dC = torch.full((M, N), float("nan"), device="cuda")
        assert dgt.gemm(dA, dB, dC, -0.5, 0.0, trans_a=ta, trans_b=tb) == 0
        torch.cuda.synchronize()
        outs.append(dC.cpu().numpy())
        del dC
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    say(f"f32 dma real {layout}: oracle")
    R = oracle.gemm(A, B, None, -0.5, 0.0, "f32", trans_a=ta, trans_b=tb)
    assert_close(outs[0], R, K, -0.5, what=f"f32 dma real {layout}")


# (M, N, K, batch): edge tiles with K a multiple of 64; K a multiple of 16
# only (32, 96: one slice pair, six slices); a partial last slice (1000,
# 136, 520: 8 of 16 k valid).  Each batch makes 256 tiles of 256 x 256.
EDGE_BATCHED = [(296, 264, 512, 64), (264, 1000, 256, 32), (1000, 296, 384, 32),
                (256, 256, 32, 256), (512, 512, 96, 64), (296, 264, 1000, 64),
                (256, 384, 136, 128), (300, 260, 520, 64)]


@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_edge_tiles_and_ragged_k_integer_bit_exact(layout):
    ta, tb = LAYOUTS[layout]
    for idx, (M, N, K, batch) in enumerate(EDGE_BATCHED):
        sa, sb = stored(M, N, K, ta, tb)
        A = gi.draw(3700 + idx, batch * sa[0], sa[1], "int").reshape(batch, *sa)
        B = gi.draw(3720 + idx, batch * sb[0], sb[1], "int").reshape(batch, *sb)
        C0 = gi.draw(3740 + idx, batch * M, N, "int").reshape(batch, M, N)
        for alpha, beta in [(1.0, 0.0), (1.5, 0.5)]:
            say(f"f32 dma edge {layout} {batch} x {M}x{N}x{K} a={alpha} b={beta}")
            dC = (torch.from_numpy(np.ascontiguousarray(C0)).cuda() if beta else
                  torch.full((batch, M, N), float("nan"), device="cuda"))
            st = dgt.gemm_batched(to_dev(A, "f32"), to_dev(B, "f32"), dC, alpha, beta,
                                  trans_a=ta, trans_b=tb)
            torch.cuda.synchronize()
            assert st == 0, dgt.gemm_status_string(st)
            R = oracle.gemm_batched(A, B, C0 if beta else None, alpha, beta, "f32",
                                    trans_a=ta, trans_b=tb)
            assert_bit_exact(dC.cpu().numpy(), oracle.round_f32(R),
                             f"f32 dma edge {layout} {M}x{N}x{K}")
            del dC


@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_k_not_multiple_of_4_on_padded_storage(layout):
    """Pitches padded to multiples of 4 floats keep 16-byte rows, so K = 1001
    and 77 still run the DMA kernel, the last slice masked element by
    element."""
    ta, tb = LAYOUTS[layout]
    for idx, (M, N, K, batch) in enumerate([(296, 264, 1001, 64), (264, 300, 77, 64)]):
        sa, sb = stored(M, N, K, ta, tb)
        A = gi.draw(3800 + idx, batch * sa[0], sa[1], "int").reshape(batch, *sa)
        B = gi.draw(3810 + idx, batch * sb[0], sb[1], "int").reshape(batch, *sb)
        C0 = gi.draw(3820 + idx, batch * M, N, "int").reshape(batch, M, N)

        def padded(X):
            b, rows, cols = X.shape
            ld = (cols + 3) // 4 * 4 + 4
            t = torch.zeros((b, rows, ld), device="cuda")
            t[:, :, :cols] = torch.from_numpy(np.ascontiguousarray(X)).cuda()
            return t[:, :, :cols]

        dC = torch.from_numpy(np.ascontiguousarray(C0)).cuda()
        say(f"f32 dma padded K {layout} {batch} x {M}x{N}x{K}")
        st = dgt.gemm_batched(padded(A), padded(B), dC, 1.5, 0.5, trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        assert st == 0, dgt.gemm_status_string(st)
        R = oracle.gemm_batched(A, B, C0, 1.5, 0.5, "f32", trans_a=ta, trans_b=tb)
        assert_bit_exact(dC.cpu().numpy(), oracle.round_f32(R), f"f32 dma padded K {layout}")


@pytest.mark.parametrize("layout", ["nn", "nt"])
def test_large_ragged_real_inputs(layout):
    """4000 x 4000 x 1000 (256 edge-clipped tiles, a partial last slice)
    against the oracle, and the same call twice bit for bit."""
    ta, tb = LAYOUTS[layout]
    M = N = 4000
    K = 1000
    sa, sb = stored(M, N, K, ta, tb)
    A = gi.draw(3900, *sa, "uniform")
    B = gi.draw(3901, *sb, "uniform")
    C0 = gi.draw(3902, M, N, "uniform")
    dA, dB = to_dev(A, "f32"), to_dev(B, "f32")
    outs = []
    for _ in range(2):
        dC = torch.from_numpy(C0).cuda()
        assert dgt.gemm(dA, dB, dC, 0.75, -1.25, trans_a=ta, trans_b=tb) == 0
        torch.cuda.synchronize()
        outs.append(dC.cpu().numpy())
        del dC
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    say(f"f32 dma large ragged {layout}: oracle")
    R = oracle.gemm(A, B, C0, 0.75, -1.25, "f32", trans_a=ta, trans_b=tb)
    assert_close(outs[0], R, K, 0.75, what=f"f32 dma large ragged {layout}")
