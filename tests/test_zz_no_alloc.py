"""gemm_splitk_noalloc -- split-K into the library's fixed scratch, for
callers that cannot allocate -- through the C ABI, against gemm_splitk with a
caller-provided workspace (the same kernels, so bit-identical results) and
against the oracle (bit-exact on integer inputs, the tolerance gates on real
ones).  Two calls in a row, the second smaller, so the second reads a scratch
that still holds the first call's partials; a shape whose partials exceed the
scratch is refused before anything is queued; no call changes the device's
free memory once the library is loaded.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    dgt.library()
    oracle.build(force=False)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _both(dtype, A, B, C0, M, N, K, alpha, beta, splits, ta=False, tb=False):
    """Run gemm_splitk (torch workspace) and gemm_splitk_noalloc on the same
    inputs; return both C's as numpy."""
    dA, dB = to_dev(A, dtype), to_dev(B, dtype)
    lda, ldb = A.shape[1], B.shape[1]
    c0 = torch.from_numpy(np.ascontiguousarray(C0, np.float32)).cuda()
    code = CODE[dtype]
    need = dgt.gemm_splitk_workspace_size(code, M, N, K, splits)
    assert 0 < need <= dgt.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    c_ws, c_na = c0.clone(), c0.clone()
    torch.cuda.synchronize()
    st = dgt.gemm_splitk(code, ta, tb, M, N, K, alpha, dA.data_ptr(), lda, dB.data_ptr(), ldb,
                         beta, c_ws.data_ptr(), N, splits, ws.data_ptr(), need, s)
    assert st == 0, dgt.gemm_status_string(st)
    st = dgt.gemm_splitk_noalloc(code, ta, tb, M, N, K, alpha, dA.data_ptr(), lda, dB.data_ptr(),
                                 ldb, beta, c_na.data_ptr(), N, splits, s)
    assert st == 0, dgt.gemm_status_string(st)
    torch.cuda.synchronize()
    return c_ws.cpu().numpy(), c_na.cpu().numpy(), need


def test_noalloc_matches_workspace_entry_point_two_calls():
    # call 1: the larger split (BF16 1024 x 1024 x 16384, automatic slices:
    # 32 MiB of partials), real inputs; call 2: the ragged FP32 1000^3 with
    # beta (16 MB), which finds call 1's partials still in the scratch
    cases = [("bf16", 1024, 1024, 16384, 1.0, 0.0, "normal", 0),
             ("f32", 1000, 1000, 1000, 1.5, 0.5, "uniform", 0)]
    for idx, (dtype, M, N, K, alpha, beta, dist, splits) in enumerate(cases):
        say(f"noalloc call {idx + 1}: {dtype} {M}x{N}x{K} splits={splits}")
        A = gi.draw(1700 + idx, M, K, dist, dtype=dtype)
        B = gi.draw(1710 + idx, K, N, dist, dtype=dtype)
        C0 = gi.draw(1720 + idx, M, N, "uniform")
        c_ws, c_na, need = _both(dtype, A, B, C0, M, N, K, alpha, beta, splits)
        say(f"noalloc call {idx + 1}: {need} bytes of partials")
        assert_bit_exact(c_na, c_ws, f"noalloc vs workspace, call {idx + 1}")
        R = oracle.gemm(A, B, C0 if beta else None, alpha, beta, dtype)
        assert_close(c_na, R, K, alpha, what=f"noalloc vs oracle, call {idx + 1}")


def test_noalloc_integer_inputs_bit_exact_two_calls():
    # integer inputs: exact in any order, so equal to the oracle bit for bit;
    # the second call is smaller and stored transposed
    cases = [("f16", 512, 768, 8192, 1.0, 0.0, 0, False, False),
             ("bf16", 200, 136, 3000, -2.0, 0.5, 5, True, True)]
    for idx, (dtype, M, N, K, alpha, beta, splits, ta, tb) in enumerate(cases):
        say(f"noalloc integer call {idx + 1}: {dtype} {M}x{N}x{K} ta={ta} tb={tb}")
        A = gi.draw(1800 + idx, *((K, M) if ta else (M, K)), "int", dtype=dtype)
        B = gi.draw(1810 + idx, *((N, K) if tb else (K, N)), "int", dtype=dtype)
        C0 = gi.draw(1820 + idx, M, N, "int")
        c_ws, c_na, _ = _both(dtype, A, B, C0, M, N, K, alpha, beta, splits, ta, tb)
        assert_bit_exact(c_na, c_ws, f"noalloc vs workspace, integer call {idx + 1}")
        R = oracle.round_f32(oracle.gemm(A, B, C0 if beta else None, alpha, beta, dtype,
                                         trans_a=ta, trans_b=tb))
        assert_bit_exact(c_na, R, f"noalloc vs oracle, integer call {idx + 1}")


def test_noalloc_refuses_partials_beyond_the_scratch():
    M, N, K, splits = 2048, 2048, 16384, 8          # 8 x 2048^2 x 4 B = 128 MiB
    code = dgt.DTYPE_F32
    assert dgt.gemm_splitk_workspace_size(code, M, N, K, splits) > dgt.NOALLOC_SCRATCH_BYTES
    dA = torch.zeros((M, K), device="cuda")
    dB = torch.zeros((K, N), device="cuda")
    dC = torch.full((M, N), float("nan"), device="cuda")
    st = dgt.gemm_splitk_noalloc(code, 0, 0, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N,
                                 0.0, dC.data_ptr(), N, splits,
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == dgt.GEMM_ERR_SCRATCH
    assert torch.isnan(dC).all().item(), "a refused call wrote C"


def test_noalloc_leaves_free_memory_unchanged():
    M, N, K = 256, 384, 8192
    A = to_dev(gi.draw(1900, M, K, "int", dtype="bf16"), "bf16")
    B = to_dev(gi.draw(1901, K, N, "int", dtype="bf16"), "bf16")
    C = torch.zeros((M, N), device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def call():
        st = dgt.gemm_splitk_noalloc(dgt.DTYPE_BF16, 0, 0, M, N, K, 1.0, A.data_ptr(), K,
                                     B.data_ptr(), N, 0.0, C.data_ptr(), N, 0, s)
        assert st == 0, dgt.gemm_status_string(st)
    call()  # first call on this GPU: the library's code is loaded
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
