"""GPU parity for the FP32 DMA kernel against the CPU oracle, through the
C ABI.

The automatic choice takes that kernel for 16-byte aligned rows, with
256 x 256 tiles (one workgroup per CU) unless 128 x 128 tiles (two per CU)
take fewer waves (a strided batch counts every problem's tiles): one
4096 x 4096, 4000 x 4000 or 4000 x 3968 problem and a batch of 256
one-tile 256 x 256 problems run 256-tiles; batches of smaller ragged
problems and the single small problems run 128-tiles.  Covered, for every
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
from gpu_util import run_gemm, say, to_dev

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


# The same edge and ragged-K shapes as one problem each: too few tiles for
# 256 x 256, so the launch takes 128 x 128 tiles, two workgroups per CU.
@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_128_tiles_edge_and_ragged_k_integer_bit_exact(layout):
    ta, tb = LAYOUTS[layout]
    shapes = [(M, N, K) for (M, N, K, _) in EDGE_BATCHED] + [(512, 384, 256), (128, 128, 64),
                                                            (2048, 2048, 192)]
    for idx, (M, N, K) in enumerate(shapes):
        sa, sb = stored(M, N, K, ta, tb)
        A = gi.draw(4000 + idx, *sa, "int")
        B = gi.draw(4020 + idx, *sb, "int")
        C0 = gi.draw(4040 + idx, M, N, "int")
        for alpha, beta in [(1.0, 0.0), (1.5, 0.5)]:
            say(f"f32 dma128 {layout} {M}x{N}x{K} a={alpha} b={beta}")
            st, C = run_gemm("auto", "f32", A, B, C0 if beta else None, alpha, beta,
                             trans_a=ta, trans_b=tb)
            assert st == 0, dgt.gemm_status_string(st)
            R = oracle.round_f32(oracle.gemm(A, B, C0 if beta else None, alpha, beta, "f32",
                                             trans_a=ta, trans_b=tb))
            assert_bit_exact(C, R, f"f32 dma128 {layout} {M}x{N}x{K}")


@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_128_tiles_real_inputs(layout):
    """2048^3 (256 tiles of 128 x 128) and 1000^3 with alpha / beta, real
    inputs, against the oracle."""
    ta, tb = LAYOUTS[layout]
    for idx, (M, N, K, alpha, beta) in enumerate([(2048, 2048, 2048, 1.0, 0.0),
                                                  (1000, 1000, 1000, 1.5, 0.5)]):
        sa, sb = stored(M, N, K, ta, tb)
        A = gi.draw(4100 + idx, *sa, "uniform")
        B = gi.draw(4110 + idx, *sb, "uniform")
        C0 = gi.draw(4120 + idx, M, N, "uniform")
        say(f"f32 dma128 real {layout} {M}x{N}x{K}")
        st, C = run_gemm("auto", "f32", A, B, C0, alpha, beta, trans_a=ta, trans_b=tb)
        assert st == 0
        R = oracle.gemm(A, B, C0, alpha, beta, "f32", trans_a=ta, trans_b=tb)
        assert_close(C, R, K, alpha, what=f"f32 dma128 real {layout} {M}x{N}x{K}")


@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_256_tiles_edge_and_ragged_k_integer_bit_exact(layout):
    """Edge tiles in both dimensions with K = 136 (a partial last slice) and
    K = 1000 (a partial last slice after 15 whole groups), 256-tiles."""
    ta, tb = LAYOUTS[layout]
    for idx, (M, N, K) in enumerate([(4000, 3968, 136), (3968, 4000, 1000)]):
        sa, sb = stored(M, N, K, ta, tb)
        A = gi.draw(4200 + idx, *sa, "int")
        B = gi.draw(4210 + idx, *sb, "int")
        C0 = gi.draw(4220 + idx, M, N, "int")
        dA, dB = to_dev(A, "f32"), to_dev(B, "f32")
        say(f"f32 dma256 edge {layout} {M}x{N}x{K}")
        dC = torch.from_numpy(C0).cuda()
        st = dgt.gemm(dA, dB, dC, 1.5, 0.5, trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        assert st == 0, dgt.gemm_status_string(st)
        R = oracle.round_f32(oracle.gemm(A, B, C0, 1.5, 0.5, "f32", trans_a=ta, trans_b=tb))
        assert_bit_exact(dC.cpu().numpy(), R, f"f32 dma256 edge {layout} {M}x{N}x{K}")
        del dC
