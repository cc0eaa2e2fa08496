"""GPU parity for split-K (gemm_splitk) against the CPU oracle, through the
C ABI.

The K range is cut into slices whose fp32 partial products go to a
caller-provided workspace and are summed in a fixed order; the result is
the same operation as gemm_ex.  Covered: fp32 / bf16 / fp16, stored layouts
NN / NT / TN, automatic and requested slice counts, K not a multiple of the
slice length (the shorter last slice runs in the same launch), slices that
take the skinny path (M <= 64) and the whole-tile DMA kernel, integer inputs bit-exact, real inputs within the gates, beta on
and off, a guard band after the workspace and around C, a workspace that
starts right after A when the last slice is shorter, and run-to-run
determinism.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from gates import assert_bit_exact, assert_close
from gpu_util import TORCH_DTYPE, say, to_dev

torch = pytest.importorskip("torch")
import dense_gemm_tuning_amd as dgt  # noqa: E402

pytestmark = pytest.mark.gpu

LAYOUTS = {"nn": (False, False), "nt": (False, True), "tn": (True, False)}
CODE = {"f32": 0, "bf16": 1, "f16": 2}
# (M, N, K, splits): automatic (the 1000^3 shape gets 4 fp32 or 8 16-bit
# slices), requests, K not a multiple of the slice (the shorter last slice is
# the last problem of the same launch), slices on the skinny paths (the one
# for B stored N x K included, K a multiple of 8) and on whole tiles, and one
# GPU's share of the skinny shape under an 8-way column split (8 x 3584 x
# 8192, 8 automatic slices)
CASES = [(1000, 1000, 1000, 0), (300, 260, 1000, 3), (64, 64, 4096, 4), (1, 1, 300, 2),
         (256, 256, 2048, 0), (130, 70, 700, 5), (8, 3584, 8192, 0), (40, 500, 1000, 3)]


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


def run_split(dtype, A, B, C0, alpha, beta, splits, ta, tb, M, N, K, canary=-777.0):
    """One gemm_splitk call with a guard band after the workspace; returns
    (status, C, slices)."""
    code = CODE[dtype]
    need = dgt.gemm_splitk_workspace_size(code, M, N, K, splits)
    slices = dgt.gemm_splitk_slices(code, M, N, K, splits)
    assert need >= 0 and slices >= 1
    ws = torch.full((need // 4 + 1024,), canary, device="cuda")
    dA, dB = to_dev(A, dtype), to_dev(B, dtype)
    dC = (torch.from_numpy(np.ascontiguousarray(C0, np.float32)).cuda() if C0 is not None
          else torch.full((M, N), float("nan"), device="cuda"))
    st = dgt.gemm_split(dA, dB, dC, alpha, beta, splits=splits, workspace=ws[:need // 4] if need
                        else None, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    tail = ws[need // 4:].cpu().numpy()
    assert np.all(tail == canary), "split-K wrote past its workspace"
    return st, dC.cpu().numpy(), slices


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_splitk_integer_bit_exact(dtype, layout):
    ta, tb = LAYOUTS[layout]
    for idx, (M, N, K, splits) in enumerate(CASES):
        sa, sb = stored(M, N, K, ta, tb)
        A = gi.draw(1100 + idx, *sa, "int", dtype=dtype)
        B = gi.draw(1200 + idx, *sb, "int", dtype=dtype)
        C0 = gi.draw(1300 + idx, M, N, "int")
        for alpha, beta in [(1.0, 0.0), (1.5, 0.5)]:
            c0 = C0 if beta else None
            st, C, slices = run_split(dtype, A, B, c0, alpha, beta, splits, ta, tb, M, N, K)
            say(f"split-K {dtype} {layout} {M}x{N}x{K} splits={splits} -> {slices} slices")
            assert st == 0, dgt.gemm_status_string(st)
            R = oracle.round_f32(oracle.gemm(A, B, c0, alpha, beta, dtype, trans_a=ta,
                                             trans_b=tb))
            assert_bit_exact(C, R, f"split-K {dtype}/{layout} {M}x{N}x{K} s={splits}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_splitk_real_inputs(dtype):
    dist = "uniform" if dtype == "f32" else "normal"
    for (M, N, K, splits, alpha, beta) in [(1000, 1000, 1000, 0, 1.5, 0.5),
                                           (512, 384, 8192, 0, 1.0, 0.0),
                                           (48, 200, 3000, 6, -1.0, 2.0)]:
        say(f"split-K real {dtype} {M}x{N}x{K}")
        A = gi.draw(1400, M, K, dist, dtype=dtype)
        B = gi.draw(1401, K, N, dist, dtype=dtype)
        C0 = gi.draw(1402, M, N, "uniform")
        st, C, slices = run_split(dtype, A, B, C0, alpha, beta, splits, False, False, M, N, K)
        assert st == 0 and slices > 1
        R = oracle.gemm(A, B, C0, alpha, beta, dtype)
        assert_close(C, R, K, alpha, what=f"split-K {dtype} {M}x{N}x{K}")


def test_splitk_padded_c_guard_band_and_determinism():
    M, N, K, ldc = 200, 300, 2000, 307
    A = gi.draw(1500, M, K, "uniform")
    B = gi.draw(1501, K, N, "uniform")
    C0 = gi.draw(1502, M, N, "uniform")
    canary = -4321.0
    outs = []
    for _ in range(2):
        base = torch.full((M * ldc + 64,), canary, device="cuda")
        dC = base[:M * ldc].view(M, ldc)[:, :N]
        dC.copy_(torch.from_numpy(C0).cuda())
        st = dgt.gemm_split(to_dev(A, "f32"), to_dev(B, "f32"), dC, 0.75, -0.25, splits=5)
        torch.cuda.synchronize()
        assert st == 0
        full = base.cpu().numpy()
        mask = np.ones(full.shape, bool)
        mask[np.arange(M * ldc).reshape(M, ldc)[:, :N].ravel()] = False
        assert np.all(full[mask] == canary), "split-K wrote outside C"
        outs.append(dC.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    R = oracle.gemm(A, B, C0, 0.75, -0.25, "f32")
    assert_close(outs[0], R, K, 0.75, what="padded C")


def test_splitk_workspace_errors_on_gpu():
    A = torch.zeros((64, 4096), device="cuda")
    B = torch.zeros((4096, 64), device="cuda")
    C = torch.zeros((64, 64), device="cuda")
    small = torch.zeros(16, dtype=torch.uint8, device="cuda")
    assert dgt.gemm_split(A, B, C, splits=4, workspace=small) == dgt.GEMM_ERR_WORKSPACE
    # one slice needs no workspace at all
    assert dgt.gemm_split(A, B, C, splits=1) == 0
    torch.cuda.synchronize()
    # a host workspace would hand a host pointer to the kernels: refused
    # by the binding before anything is queued
    with pytest.raises(ValueError, match="workspace"):
        dgt.gemm_split(A, B, C, splits=4, workspace=torch.zeros(1 << 20, dtype=torch.uint8))


@pytest.mark.parametrize("ta", [False, True])
def test_splitk_workspace_right_after_a(ta):
    """The workspace starts at the byte after A's last element while the last
    slice is shorter than the others: the overlap check must measure that
    slice's operand span with its own K (not the full slice length), so the
    call runs, and the result is exact."""
    M, N, K, splits = 100, 64, 1000, 3      # slices of 384, 384, 232
    code = CODE["f32"]
    assert dgt.gemm_splitk_slices(code, M, N, K, splits) == 3
    need = dgt.gemm_splitk_workspace_size(code, M, N, K, splits)
    sa = (K, M) if ta else (M, K)
    A = gi.draw(1600, *sa, "int")
    B = gi.draw(1601, K, N, "int")
    n_a = sa[0] * sa[1]                       # A's elements, packed (lda = its row length)
    buf = torch.zeros((n_a + need // 4 + 64,), device="cuda")
    dA = buf[:n_a].view(*sa)
    dA.copy_(torch.from_numpy(A).cuda())
    ws_ptr = buf.data_ptr() + n_a * 4         # 16-byte aligned: n_a * 4 = 400000
    dB = to_dev(B, "f32")
    dC = torch.full((M, N), float("nan"), device="cuda")
    say(f"split-K workspace after A, ta={ta}")
    st = dgt.gemm_splitk(code, ta, False, M, N, K, 1.0, dA.data_ptr(), sa[1], dB.data_ptr(), N,
                         0.0, dC.data_ptr(), N, splits, ws_ptr, need,
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0, dgt.gemm_status_string(st)
    R = oracle.round_f32(oracle.gemm(A, B, None, 1.0, 0.0, "f32", trans_a=ta))
    assert_bit_exact(dC.cpu().numpy(), R, f"split-K, workspace after A, ta={ta}")
    assert np.array_equal(dA.cpu().numpy(), A), "A was written"
