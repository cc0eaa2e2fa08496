"""Seeded random shapes through the tiled MFMA paths, bit-exact against the
CPU oracle on small-integer inputs (exact in any summation order).

Each case draws M, N, K (1 .. 700, with a bias towards a few rows or columns
past a multiple of 128 or 256 and towards K just past a multiple of 16 or
32), a stored layout, alpha and beta from {0.5, 1, 1.5} x {0, 0.5}, and
a pitch for A and B (packed, rounded up to 16 bytes plus one more chunk,
or packed plus 3 elements).  Every case runs the automatic choice; aligned cases
also run both fixed-tile DMA rungs (256 x 256 and 128 x 128 workgroup tiles).
The draw is a function of the case number only, so a failure names a case
that reproduces on its own.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from gates import assert_bit_exact
from gpu_util import TORCH_DTYPE, say, to_dev

torch = pytest.importorskip("torch")
import dense_gemm_tuning_amd as dgt  # noqa: E402

pytestmark = pytest.mark.gpu

N_CASES = 64
ELEMS_PER_CHUNK = {"f32": 4, "bf16": 8, "f16": 8}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    dgt.library()  # raises if the HIP library is missing: no fallback
    oracle.build(force=False)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def draw_case(case):
    rng = np.random.default_rng(7000 + case)

    def dim(lo, hi, steps):
        if rng.random() < 0.5:  # at, or just past, a tile or slice multiple
            base = steps[rng.integers(len(steps))] * int(rng.integers(1, 4))
            return int(max(lo, min(hi, base + int(rng.choice([0, 0, 1, -1, 3, 8])))))
        return int(rng.integers(lo, hi + 1))

    M = dim(65, 700, [128, 256])       # above the skinny path
    N = dim(1, 700, [128, 256])
    K = dim(1, 600, [16, 32, 64, 128])
    ta, tb = bool(rng.integers(2)), bool(rng.integers(2))
    alpha = float(rng.choice([0.5, 1.0, 1.5]))
    beta = float(rng.choice([0.0, 0.5]))
    pad = [int(rng.choice([0, 1, 3])) for _ in range(2)]  # packed / aligned + chunk / +3
    return M, N, K, ta, tb, alpha, beta, pad


def padded_dev(X, dtype, pad_code):
    rows, cols = X.shape
    step = ELEMS_PER_CHUNK[dtype]
    extra = {0: 0, 1: (-cols) % step + step, 3: 3}[pad_code]
    t = torch.zeros((rows, cols + extra), dtype=getattr(torch, TORCH_DTYPE[dtype]), device="cuda")
    t[:, :cols] = to_dev(X, dtype)
    return t[:, :cols]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("case", range(N_CASES))
def test_random_shape_bit_exact(case, dtype):
    M, N, K, ta, tb, alpha, beta, pad = draw_case(case)
    sa = (K, M) if ta else (M, K)
    sb = (N, K) if tb else (K, N)
    A = gi.draw(7100 + case, *sa, "int", dtype=dtype)
    B = gi.draw(7200 + case, *sb, "int", dtype=dtype)
    C0 = gi.draw(7300 + case, M, N, "int")
    dA, dB = padded_dev(A, dtype, pad[0]), padded_dev(B, dtype, pad[1])
    step = ELEMS_PER_CHUNK[dtype]
    aligned = dA.stride(0) % step == 0 and dB.stride(0) % step == 0
    R = oracle.round_f32(oracle.gemm(A, B, C0 if beta else None, alpha, beta, dtype,
                                     trans_a=ta, trans_b=tb))
    for variant in ["auto"] + (["mfma256", "mfma128"] if aligned else []):
        say(f"random case {case} {dtype} {variant}: {M}x{N}x{K} ta={ta} tb={tb} "
            f"a={alpha} b={beta} pad={pad}")
        dC = (torch.from_numpy(C0).cuda() if beta else
              torch.full((M, N), float("nan"), device="cuda"))
        st = dgt.gemm(dA, dB, dC, alpha, beta, variant=variant, trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        assert st == 0, dgt.gemm_status_string(st)
        assert_bit_exact(dC.cpu().numpy(), R, f"case {case} {dtype} {variant}")
        del dC


def test_cases_cover_the_paths():
    """The draw reaches aligned and unaligned pitches, every layout, K past a
    slice boundary and both beta branches."""
    cases = [draw_case(c) for c in range(N_CASES)]
    assert {(c[3], c[4]) for c in cases} == {(False, False), (False, True), (True, False),
                                              (True, True)}
    assert any(3 in c[7] for c in cases) and any(c[7] == [0, 0] for c in cases)
    assert any(c[2] % 16 != 0 for c in cases) and any(c[2] % 64 == 0 for c in cases)
    assert {c[6] for c in cases} == {0.0, 0.5}
