"""GPU parity for stream-K (gemm_streamk) against the CPU oracle, through
the C ABI.

The K iterations (128 k each for 16-bit inputs, 64 k for FP32) of all
256 x 256 tiles are dealt out in equal contiguous ranges to one workgroup per
CU; a tile covered by one workgroup is written directly, the parts of a split
tile go to the workspace and a second kernel sums them in k order.  Covered,
for FP32, BF16 and FP16: integer inputs bit-exact for every stored layout on
shapes where every tile is split into many parts (fewer iterations than
workgroups), where ranges span one and a half tiles, with edge tiles and a
partial last slice, and with alpha / beta; real inputs within the gates;
run-to-run determinism; beta == 0 never reading a NaN-filled C; a padded C
inside a canary band (the fix-up kernel writes only C); the calls stream-K
does not cover (M <= 64, unaligned rows), which run as gemm_ex; a short
workspace refused; the torch-facing gemm_stream, with its own workspace and
with one it allocates, on stored-transposed operands.
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

CODE = {"f32": dgt.DTYPE_F32, "bf16": dgt.DTYPE_BF16, "f16": dgt.DTYPE_F16}
LAYOUTS = {"nn": (False, False), "nt": (False, True), "tn": (True, False), "tt": (True, True)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    dgt.library()
    oracle.build(force=False)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def stored(M, N, K, ta, tb):
    return ((K, M) if ta else (M, K)), ((N, K) if tb else (K, N))


def run_streamk(dtype, A, B, C0, M, N, K, alpha, beta, ta=False, tb=False, ws_bytes=None):
    code = CODE[dtype]
    dA, dB = to_dev(A, dtype), to_dev(B, dtype)
    dC = (torch.from_numpy(np.ascontiguousarray(C0, np.float32)).cuda() if C0 is not None
          else torch.full((M, N), float("nan"), device="cuda"))
    need = dgt.gemm_streamk_workspace_size(code, M, N, K)
    assert need >= 0
    nbytes = need if ws_bytes is None else ws_bytes
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    st = dgt.gemm_streamk(code, ta, tb, M, N, K, alpha, dA.data_ptr(), A.shape[1], dB.data_ptr(),
                          B.shape[1], beta, dC.data_ptr(), N, ws.data_ptr() if nbytes else 0,
                          nbytes, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st, dC.cpu().numpy(), need


# (M, N, K), with 16-bit / FP32 iterations: 6 tiles x 8 / 16 iterations <
# 256 workgroups (every tile in several parts); 25 tiles x 16 / 32 (1.6 / 3.1
# iterations a workgroup); 384 tiles x 8 / 16 (one and a half tiles a
# workgroup); edge tiles with K = 1000 (a partial last slice); edge tiles with
# K = 1120, a multiple of the slice but not of the iteration
SHAPES = [(512, 768, 1024), (1280, 1280, 2048), (6144, 4096, 1024), (1000, 1000, 1000),
          (776, 1288, 1120)]


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_streamk_integer_bit_exact(dtype, layout):
    ta, tb = LAYOUTS[layout]
    for idx, (M, N, K) in enumerate(SHAPES):
        sa, sb = stored(M, N, K, ta, tb)
        A = gi.draw(2400 + idx, *sa, "int", dtype=dtype)
        B = gi.draw(2410 + idx, *sb, "int", dtype=dtype)
        C0 = gi.draw(2420 + idx, M, N, "int")
        for alpha, beta in [(1.0, 0.0), (1.5, 0.5)]:
            say(f"stream-K {dtype} {layout} {M}x{N}x{K} a={alpha} b={beta}")
            st, C, need = run_streamk(dtype, A, B, C0 if beta else None, M, N, K, alpha, beta,
                                      ta, tb)
            assert st == 0, dgt.gemm_status_string(st)
            assert need > 0
            R = oracle.round_f32(oracle.gemm(A, B, C0 if beta else None, alpha, beta, dtype,
                                             trans_a=ta, trans_b=tb))
            assert_bit_exact(C, R, f"stream-K {dtype}/{layout} {M}x{N}x{K} a={alpha} b={beta}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_streamk_real_inputs_and_determinism(dtype):
    M, N, K = 3072, 2560, 4096
    A = gi.draw(2430, M, K, "normal", dtype=dtype)
    B = gi.draw(2431, K, N, "normal", dtype=dtype)
    say(f"stream-K real {dtype} {M}x{N}x{K}")
    st, C1, _ = run_streamk(dtype, A, B, None, M, N, K, 1.0, 0.0)
    assert st == 0
    st, C2, _ = run_streamk(dtype, A, B, None, M, N, K, 1.0, 0.0)
    assert st == 0
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32)), "two runs differ"
    R = oracle.gemm(A, B, None, 1.0, 0.0, dtype)
    assert_close(C1, R, K, 1.0, what=f"stream-K real {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_streamk_padded_c_guard_band(dtype):
    M, N, K, pad = 600, 520, 768, 24
    A = gi.draw(2440, M, K, "int", dtype=dtype)
    B = gi.draw(2441, K, N, "int", dtype=dtype)
    C0 = gi.draw(2442, M, N, "int")
    ldc = N + pad
    canary = -777.0
    cbuf = torch.full((M * ldc + 64,), canary, device="cuda")
    dC = cbuf[:M * ldc].view(M, ldc)[:, :N]
    dC.copy_(torch.from_numpy(C0).cuda())
    need = dgt.gemm_streamk_workspace_size(CODE[dtype], M, N, K)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dA, dB = to_dev(A, dtype), to_dev(B, dtype)
    st = dgt.gemm_streamk(CODE[dtype], 0, 0, M, N, K, -2.0, dA.data_ptr(), K, dB.data_ptr(), N,
                          1.0, dC.data_ptr(), ldc, ws.data_ptr(), need,
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0, dgt.gemm_status_string(st)
    R = oracle.round_f32(oracle.gemm(A, B, C0, -2.0, 1.0, dtype))
    assert_bit_exact(dC.cpu().numpy(), R, f"stream-K padded C {dtype}")
    full = cbuf.cpu().numpy()
    mask = np.ones(full.shape, bool)
    mask[np.arange(M * ldc).reshape(M, ldc)[:, :N].ravel()] = False
    assert np.all(full[mask] == canary), "stream-K wrote outside C"


def test_streamk_uncovered_calls_run_as_gemm_ex():
    """M <= 64 needs no workspace; rows that are not 16-byte aligned (B's
    260 bf16 = 520 bytes, or 259 floats) leave the DMA kernels.  These run as
    gemm_ex and give the oracle's result."""
    cases = [("bf16", 64, 512, 1024), ("f32", 48, 512, 1024), ("bf16", 300, 260, 520),
             ("f32", 300, 259, 512)]
    for dtype, M, N, K in cases:
        need = dgt.gemm_streamk_workspace_size(CODE[dtype], M, N, K)
        assert (need == 0) == (M <= 64)
        A = gi.draw(2450, M, K, "int", dtype=dtype)
        B = gi.draw(2451, K, N, "int", dtype=dtype)
        say(f"stream-K fallback {dtype} {M}x{N}x{K}")
        st, C, _ = run_streamk(dtype, A, B, None, M, N, K, 1.0, 0.0)
        assert st == 0, dgt.gemm_status_string(st)
        R = oracle.round_f32(oracle.gemm(A, B, None, 1.0, 0.0, dtype))
        assert_bit_exact(C, R, f"stream-K fallback {dtype} {M}x{N}x{K}")


def test_streamk_short_workspace_refused():
    M, N, K = 1024, 1024, 1024
    A = gi.draw(2460, M, K, "int", dtype="bf16")
    B = gi.draw(2461, K, N, "int", dtype="bf16")
    need = dgt.gemm_streamk_workspace_size(CODE["bf16"], M, N, K)
    st, C, _ = run_streamk("bf16", A, B, None, M, N, K, 1.0, 0.0, ws_bytes=need - 1024)
    assert st == dgt.GEMM_ERR_WORKSPACE
    assert np.all(np.isnan(C)), "a refused call wrote C"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gemm_stream_tensor_call(dtype):
    """The torch-facing form: integer inputs bit-exact, A stored K x M and B
    stored N x K, once with a caller's workspace and once with the one it
    allocates."""
    M, N, K = 1000, 1288, 1120
    ta, tb = True, True
    sa, sb = stored(M, N, K, ta, tb)
    A = gi.draw(2450, *sa, "int", dtype=dtype)
    B = gi.draw(2451, *sb, "int", dtype=dtype)
    C0 = gi.draw(2452, M, N, "int")
    R = oracle.round_f32(oracle.gemm(A, B, C0, 1.5, 0.5, dtype, trans_a=ta, trans_b=tb))
    need = dgt.gemm_streamk_workspace_size(CODE[dtype], M, N, K)
    assert need > 0
    for ws in (torch.empty(need, dtype=torch.uint8, device="cuda"), None):
        say(f"gemm_stream {dtype} {M}x{N}x{K} workspace {'given' if ws is not None else 'allocated'}")
        dC = torch.from_numpy(C0.astype(np.float32)).cuda()
        st = dgt.gemm_stream(to_dev(A, dtype), to_dev(B, dtype), dC, 1.5, 0.5, workspace=ws,
                             trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        assert st == 0, dgt.gemm_status_string(st)
        assert_bit_exact(dC.cpu().numpy(), R, f"gemm_stream {dtype}")
