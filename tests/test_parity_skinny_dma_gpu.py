"""GPU parity for the skinny kernel that streams B through LDS by copies
(A stored M x K, B stored N x K: a linear layer's weight; 16-bit and fp32
inputs), against the CPU oracle, through the C ABI.

The skinny rung takes that kernel when K is a multiple of the elements in
16 bytes (8 for 16-bit inputs, 4 for fp32) and every row is 16-byte
aligned; each wave takes one K-range of a 128-column strip, eight waves per
workgroup: 256-byte row pieces per step (128 k of 16-bit inputs, 64 of
fp32), a two-stage ring per wave and two A buffers for M <= 32; 128-byte
pieces, four stages and one A buffer above.
Covered: every row-block count (M = 1 .. 64, both configurations), ragged
column strips (N not a multiple of 128, fewer
columns than one group), K tails (K not a multiple of the 128-deep step,
down to K = 8, where most waves have no step), integer inputs bit-exact
for every input type (fp32 also with K a multiple of 4 but not of 8);
alpha / beta and the bias through the strided batch; row pitches padded
with NaN (no k >= K may reach a product) and canaries around C; K not a
multiple of 8 (16-bit) or 4 (fp32), which the register-staged kernels take;
real inputs within the gates at a decode-like size; run-to-run determinism.
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


def ints(seed, r, c, dtype):
    return gi.draw(seed, r, c, "int", dtype=dtype)


# (M, N, K): row blocks 1..4 across both configurations, ragged
# strips, K tails (of both step depths) and a K shorter than one step.
SHAPES = [
    (1, 128, 128), (5, 3, 16), (8, 1000, 1032), (16, 4097, 8), (17, 130, 136),
    (24, 256, 2048), (32, 129, 4104), (33, 777, 520), (40, 128, 1000), (48, 1, 264),
    (57, 385, 392), (63, 640, 4096), (64, 4096 + 96, 1024), (64, 31, 8),
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_integer_inputs_bit_exact(shape, dtype):
    M, N, K = shape
    A, B = ints(5100 + M, M, K, dtype), ints(5200 + N, N, K, dtype)
    say(f"skinny dma {dtype} {M}x{N}x{K}")
    st, C = run_gemm("skinny", dtype, A, B, None, 1.0, 0.0, trans_b=True)
    assert st == 0, dgt.gemm_status_string(st)
    R = oracle.round_f32(oracle.gemm(A, B, None, 1.0, 0.0, dtype, trans_b=True))
    assert_bit_exact(C, R, f"skinny dma {dtype} {M}x{N}x{K}")


# fp32 only: K a multiple of 4 but not of 8 (a 16-byte piece is 4 floats),
# in both configurations, down to a single piece.
F32_SHAPES = [(9, 200, 1004), (33, 333, 12), (50, 129, 260), (64, 100, 4), (2, 4099, 8196)]


@pytest.mark.parametrize("shape", F32_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_k_multiple_of_4_bit_exact(shape):
    M, N, K = shape
    A, B = ints(6600 + M, M, K, "f32"), ints(6700 + N, N, K, "f32")
    say(f"skinny dma f32 {M}x{N}x{K}")
    st, C = run_gemm("skinny", "f32", A, B, None, 1.0, 0.0, trans_b=True)
    assert st == 0, dgt.gemm_status_string(st)
    R = oracle.round_f32(oracle.gemm(A, B, None, 1.0, 0.0, "f32", trans_b=True))
    assert_bit_exact(C, R, f"skinny dma f32 {M}x{N}x{K}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_alpha_beta_bias_batch(dtype):
    """Three problems, per-problem bias, alpha / beta, one with a shared A."""
    nb, M, N, K = 3, 40, 300, 648
    A = np.stack([ints(5300 + z, M, K, dtype) for z in range(nb)])
    B = np.stack([ints(5400 + z, N, K, dtype) for z in range(nb)])
    C0 = np.stack([gi.draw(5500 + z, M, N, "int") for z in range(nb)])
    bias = np.stack([gi.draw(5600 + z, 1, N, "int")[0] for z in range(nb)])
    say(f"skinny dma batch {dtype} {nb}x{M}x{N}x{K}")
    dC = torch.from_numpy(C0.astype(np.float32)).cuda()
    st = dgt.gemm_batched(to_dev(A, dtype), to_dev(B, dtype), dC, 1.5, 0.5,
                          bias=torch.from_numpy(bias.astype(np.float32)).cuda(),
                          variant="skinny", trans_b=True)
    torch.cuda.synchronize()
    assert st == 0, dgt.gemm_status_string(st)
    C = dC.cpu().numpy()
    for z in range(nb):
        R = oracle.round_f32(oracle.gemm(A[z], B[z], C0[z], 1.5, 0.5, dtype, trans_b=True,
                                         bias=bias[z]))
        assert_bit_exact(C[z], R, f"batch problem {z}")


def _strided(shape, ld, dtype, fill):
    rows, cols = shape
    tdt = torch.float32 if dtype == "f32" else getattr(torch, TORCH_DTYPE[dtype])
    base = torch.full((rows * ld + 64,), fill, dtype=tdt, device="cuda")
    return base, base[:rows * ld].view(rows, ld)[:, :cols]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M", [12, 29, 64])
def test_nan_padded_pitches_and_canaries(M, dtype):
    """Row pitches K + 24 (still 16-byte aligned) whose padding holds NaN, a
    K tail inside a step, and a C pitch padded with canaries: no element at
    k >= K may reach a product, and nothing outside C may be written."""
    N, K = 300, 392
    lda, ldb, ldc = K + 24, K + 24, N + 5
    A, B = ints(5700 + M, M, K, dtype), ints(5800 + M, N, K, dtype)
    C0 = gi.draw(5900 + M, M, N, "int")
    _, dA = _strided((M, K), lda, dtype, float("nan"))
    _, dB = _strided((N, K), ldb, dtype, float("nan"))
    canary = -12345.0
    cbase, dC = _strided((M, N), ldc, "f32", canary)
    dA.copy_(to_dev(A, dtype))
    dB.copy_(to_dev(B, dtype))
    dC.copy_(torch.from_numpy(C0).cuda())
    say(f"skinny dma padded {dtype} M={M}")
    st = dgt.gemm(dA, dB, dC, 1.0, 0.5, variant="skinny", trans_b=True)
    torch.cuda.synchronize()
    assert st == 0, dgt.gemm_status_string(st)
    R = oracle.round_f32(oracle.gemm(A, B, C0, 1.0, 0.5, dtype, trans_b=True))
    assert_bit_exact(dC.cpu().numpy(), R, "padded pitches")
    full = cbase.cpu().numpy()
    mask = np.ones(full.shape, bool)
    mask[np.arange(M * ldc).reshape(M, ldc)[:, :N].ravel()] = False
    assert np.all(full[mask] == canary), "kernel wrote outside C"


@pytest.mark.parametrize("dtype,K", [("bf16", 1001), ("bf16", 1004), ("f32", 1001), ("f32", 1002)])
def test_k_not_multiple_of_piece_takes_register_kernel(dtype, K):
    M, N = 40, 200
    A, B = ints(6000 + K, M, K, dtype), ints(6100 + K, N, K, dtype)
    st, C = run_gemm("skinny", dtype, A, B, None, 1.0, 0.0, trans_b=True)
    assert st == 0
    R = oracle.round_f32(oracle.gemm(A, B, None, 1.0, 0.0, dtype, trans_b=True))
    assert_bit_exact(C, R, f"{dtype} K={K}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [8, 32, 64])
def test_real_inputs_decode_like(M, dtype):
    """Normal inputs (sigma 0.02, as a weight) at K = 8192, ragged N."""
    N, K = 2048 + 72, 8192
    A = gi.draw(6200 + M, M, K, "normal", sigma=0.02, dtype=dtype)
    B = gi.draw(6300 + M, N, K, "normal", sigma=0.02, dtype=dtype)
    say(f"skinny dma real {dtype} M={M}")
    st, C = run_gemm("auto", dtype, A, B, None, 1.0, 0.0, trans_b=True)
    assert st == 0
    R = oracle.gemm(A, B, None, 1.0, 0.0, dtype, trans_b=True)
    assert_close(C, R, K, 1.0, 0.02, 0.02, what=f"decode-like {dtype} M={M}")
    assert np.all(np.isfinite(C))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [16, 40, 64])
def test_deterministic(M, dtype):
    N, K = 1000, 4096
    dA = to_dev(gi.draw(6400, M, K, "normal", dtype=dtype), dtype)
    dB = to_dev(gi.draw(6500, N, K, "normal", dtype=dtype), dtype)
    outs = []
    for _ in range(2):
        C = torch.zeros((M, N), device="cuda")
        assert dgt.gemm(dA, dB, C, 1.0, 0.0, variant="skinny", trans_b=True) == 0
        torch.cuda.synchronize()
        outs.append(C.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), \
        "two runs differ"
