"""GPU parity for strided batches and the bias epilogue
(gemm_strided_batched) against the CPU oracle, through the C ABI.

C_z <- alpha*op(A_z)*op(B_z) + beta*C_z + bias_z for z < batch: the batched
form of a linear layer (elainafan.one "全连接层": X W^T + b, with a batch
dimension kept).  Covered: every rung and layout family on integer inputs
(bit-exact) with no bias, a shared bias and a per-problem bias; a shared
operand (stride 0); padded batch strides with a guard band between the
problems' C; alpha == 0 and K == 0 with a bias; a batch longer than one
launch takes (65535 problems) with the seams checked; real inputs at a
whole-tile size that takes the DMA kernel.
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

RUNGS = ["naive", "lds", "mfma", "skinny", "auto"]
LAYOUTS = {"nn": (False, False), "nt": (False, True), "tn": (True, False)}


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


def draw3(seed, n, shape, dist, dtype):
    return np.stack([gi.draw(seed + z, *shape, dist, dtype=dtype) for z in range(n)])


def dev3(x, dtype):
    return to_dev(np.ascontiguousarray(x), dtype)


@pytest.mark.parametrize("bias_mode", ["none", "shared", "shared_row", "per_problem"])
@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", RUNGS)
def test_batched_integer_bit_exact(variant, dtype, layout, bias_mode):
    ta, tb = LAYOUTS[layout]
    nb = 3
    shapes = ([(8, 300, 256), (13, 128, 64), (36, 256, 256)] if variant == "skinny"
              else [(65, 129, 127), (256, 256, 256)])
    for idx, (M, N, K) in enumerate(shapes):
        say(f"batched {variant} {dtype} {layout} bias={bias_mode} {nb}x{M}x{N}x{K}")
        sa, sb = stored(M, N, K, ta, tb)
        A = draw3(700 + 10 * idx, nb, sa, "int", dtype)
        shared_b = idx == 0  # first shape: one B for every problem (stride 0)
        B = (gi.draw(750 + idx, *sb, "int", dtype=dtype)[None] if shared_b
             else draw3(760 + 10 * idx, nb, sb, "int", dtype))
        C0 = draw3(780 + 10 * idx, nb, (M, N), "int", "f32")
        if bias_mode == "none":
            bias = None
        elif bias_mode == "shared":
            bias = gi.draw(790 + idx, 1, N, "int")[0]
        elif bias_mode == "shared_row":  # a [1, N] tensor: one row for every problem
            bias = gi.draw(790 + idx, 1, N, "int")
        else:
            bias = draw3(795 + 10 * idx, nb, (1, N), "int", "f32")[:, 0, :]
        dA = dev3(A, dtype)
        dB = dev3(B, dtype)
        dB = dB.expand(nb, *dB.shape[1:]) if shared_b else dB
        dC = torch.from_numpy(C0.copy()).cuda()
        dbias = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias)).cuda()
        st = dgt.gemm_batched(dA, dB, dC, 1.5, 0.5, bias=dbias, variant=variant,
                              trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        assert st == 0, dgt.gemm_status_string(st)
        Bs = [B[0]] * nb if shared_b else list(B)
        biases = (None if bias is None else [bias] * nb if bias_mode == "shared"
                  else [bias[0]] * nb if bias_mode == "shared_row" else list(bias))
        R = oracle.gemm_batched(list(A), Bs, list(C0), 1.5, 0.5, dtype, trans_a=ta,
                                trans_b=tb, biases=biases)
        assert_bit_exact(dC.cpu().numpy(), oracle.round_f32(R),
                         f"{variant}/{dtype}/{layout}/{bias_mode} {M}x{N}x{K}")


@pytest.mark.parametrize("extra", [40, 41], ids=["aligned_strides", "odd_strides"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("variant", ["mfma", "skinny", "naive"])
def test_padded_batch_strides_and_guard_band(variant, dtype, extra):
    """Problems spaced further apart than their size: the gaps between the
    problems' C (and past the last one) must stay untouched.  Odd strides
    leave later problems' rows unaligned, which the vector paths must see."""
    nb = 4
    M, N, K = (12 if variant == "skinny" else 256), 256, 128
    lda, ldb, ldc = K + 8, N + 8, N + 3
    sa_el, sb_el, sc_el = M * lda + extra, K * ldb + extra - 16, M * ldc + 77
    A = draw3(810, nb, (M, K), "int", dtype)
    B = draw3(820, nb, (K, N), "int", dtype)
    C0 = draw3(830, nb, (M, N), "int", "f32")
    bias = draw3(840, nb, (1, N), "int", "f32")[:, 0, :]
    say(f"padded strides {variant} {dtype}")
    tdt = torch.float32 if dtype == "f32" else getattr(torch, {"bf16": "bfloat16",
                                                                 "f16": "float16"}[dtype])
    bufA = torch.zeros(nb * sa_el + 16, dtype=tdt, device="cuda")
    bufB = torch.zeros(nb * sb_el + 16, dtype=tdt, device="cuda")
    canary = -4242.0
    bufC = torch.full((nb * sc_el + 64,), canary, device="cuda")
    bufbias = torch.zeros(nb * (N + 5), device="cuda")
    for z in range(nb):
        bufA[z * sa_el:z * sa_el + M * lda].view(M, lda)[:, :K].copy_(to_dev(A[z], dtype))
        bufB[z * sb_el:z * sb_el + K * ldb].view(K, ldb)[:, :N].copy_(to_dev(B[z], dtype))
        bufC[z * sc_el:z * sc_el + M * ldc].view(M, ldc)[:, :N].copy_(torch.from_numpy(C0[z]))
        bufbias[z * (N + 5):z * (N + 5) + N].copy_(torch.from_numpy(bias[z]))
    code = {"f32": dgt.DTYPE_F32, "bf16": dgt.DTYPE_BF16, "f16": dgt.DTYPE_F16}[dtype]
    st = dgt.gemm_strided_batched(code, 0, 0, dgt.VARIANTS[variant], M, N, K, -0.5,
                                  bufA.data_ptr(), lda, sa_el, bufB.data_ptr(), ldb, sb_el,
                                  2.0, bufC.data_ptr(), ldc, sc_el, bufbias.data_ptr(), N + 5,
                                  nb, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0, dgt.gemm_status_string(st)
    R = oracle.round_f32(oracle.gemm_batched(list(A), list(B), list(C0), -0.5, 2.0, dtype,
                                             biases=list(bias)))
    full = bufC.cpu().numpy()
    mask = np.ones(full.shape, bool)
    for z in range(nb):
        body = z * sc_el + np.arange(M * ldc).reshape(M, ldc)[:, :N]
        assert_bit_exact(full[body], R[z], f"problem {z}")
        mask[body.ravel()] = False
    assert np.all(full[mask] == canary), "kernel wrote outside the problems' C"


@pytest.mark.parametrize("variant", RUNGS)
def test_bias_with_alpha_zero_and_k_zero(variant):
    nb, M, N, K = 2, (16 if variant == "skinny" else 70), 90, 33
    C0 = draw3(850, nb, (M, N), "int", "f32")
    bias = draw3(860, nb, (1, N), "int", "f32")[:, 0, :]
    A = draw3(870, nb, (M, K), "int", "bf16")
    B = draw3(880, nb, (K, N), "int", "bf16")
    dbias = torch.from_numpy(bias.copy()).cuda()
    for alpha, k in [(0.0, K), (1.0, 0)]:
        dA = dev3(A[:, :, :k], "bf16")
        dB = dev3(B[:, :k, :], "bf16")
        dC = torch.from_numpy(C0.copy()).cuda()
        st = dgt.gemm_batched(dA, dB, dC, alpha, -1.5, bias=dbias, variant=variant)
        torch.cuda.synchronize()
        assert st == 0
        want = (-1.5 * C0.astype(np.float64) + bias[:, None, :]).astype(np.float32)
        assert_bit_exact(dC.cpu().numpy(), want, f"alpha={alpha} K={k}")


def test_batch_longer_than_one_launch():
    """65537 + 3 problems take two launches; the problems around the seam
    and at both ends match the oracle."""
    nb, M, N, K = 65540, 3, 5, 4
    rng = np.random.default_rng(21)
    A = rng.integers(-3, 4, (nb, M, K)).astype(np.float32)
    B = rng.integers(-3, 4, (nb, K, N)).astype(np.float32)
    bias = rng.integers(-3, 4, (nb, N)).astype(np.float32)
    dC = torch.zeros((nb, M, N), device="cuda")
    say(f"long batch {nb}")
    st = dgt.gemm_batched(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), dC, 1.0, 0.0,
                          bias=torch.from_numpy(bias).cuda(), variant="mfma")
    torch.cuda.synchronize()
    assert st == 0
    C = dC.cpu().numpy()
    for z in [0, 1, 65533, 65534, 65535, 65536, nb - 1]:
        R = oracle.round_f32(oracle.gemm(A[z], B[z], None, 1.0, 0.0, "f32", bias=bias[z]))
        assert_bit_exact(C[z], R, f"problem {z}")


@pytest.mark.parametrize("layout", ["nn", "nt"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_batched_real_inputs_dma(dtype, layout):
    """Whole tiles (DMA kernel), real inputs, per-problem bias."""
    ta, tb = LAYOUTS[layout]
    nb, M, N, K = 3, 512, 256, 384
    sa, sb = stored(M, N, K, ta, tb)
    A = draw3(900, nb, sa, "normal", dtype)
    B = draw3(910, nb, sb, "normal", dtype)
    bias = draw3(920, nb, (1, N), "uniform", "f32")[:, 0, :]
    dC = torch.zeros((nb, M, N), device="cuda")
    st = dgt.gemm_batched(dev3(A, dtype), dev3(B, dtype), dC, 1.0, 0.0,
                          bias=torch.from_numpy(bias.copy()).cuda(), trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    assert st == 0
    R = oracle.gemm_batched(list(A), list(B), None, 1.0, 0.0, dtype, trans_a=ta, trans_b=tb,
                            biases=list(bias))
    C = dC.cpu().numpy()
    for z in range(nb):
        assert_close(C[z], R[z], K, 1.0, what=f"problem {z}")
