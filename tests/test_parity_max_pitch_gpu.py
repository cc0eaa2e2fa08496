"""GPU parity at the largest row pitches, through the C ABI.

The global->LDS DMA kernels address a wave's rows through 32-bit buffer
offsets, so they take stored row pitches below 2^24 elements for 16-bit
inputs and 2^23 for fp32 (host check `mfma16_dma_eligible` /
`mfma_f32_dma_eligible`); larger pitches run the register-staged kernel.  At
the boundary -- the largest 16-byte-aligned pitch below the limit, and the
limit itself -- both paths must give the oracle's result bit for bit on
integer inputs, for operands stored with k contiguous (A as M x K, B as
N x K) and with m / n contiguous (B as K x N).  The fixed-tile rung
GEMM_VARIANT_MFMA_T256 pins which side of the boundary a pitch is on: it
runs the DMA kernel below the limit and is refused (GEMM_ERR_VARIANT, on the
host) at it.  Each case allocates up to 8 GiB of device memory per operand
(256 rows at a 2^24-element pitch) and writes only the used elements.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from gates import assert_bit_exact
from gpu_util import TORCH_DTYPE, say

torch = pytest.importorskip("torch")
import dense_gemm_tuning_amd as dgt  # noqa: E402

pytestmark = pytest.mark.gpu

LIMIT = {"bf16": 1 << 24, "f16": 1 << 24, "f32": 1 << 23}
STEP = {"bf16": 8, "f16": 8, "f32": 4}   # 16 bytes of elements
CODE = {"f32": 0, "bf16": 1, "f16": 2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    dgt.library()
    oracle.build(force=False)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _pitched(host, pitch, dtype):
    """A device view of `host` (rows x cols) with row pitch `pitch` elements,
    inside a buffer of exactly rows x pitch elements (the rest unwritten)."""
    rows, cols = host.shape
    tdt = getattr(torch, TORCH_DTYPE[dtype])
    buf = torch.empty(rows * pitch, dtype=tdt, device="cuda")
    view = buf.view(rows, pitch)[:, :cols]
    src = torch.from_numpy(np.ascontiguousarray(host).view(np.int16 if dtype != "f32" else np.float32))
    view.copy_(src.cuda().view(tdt))
    return buf, view


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("trans_b", [False, True], ids=["nn", "nt"])
def test_largest_pitches(dtype, trans_b):
    M, N, K = 256, 256, 128
    A = gi.draw(2301, M, K, "int", dtype=dtype)
    B = gi.draw(2302, *((N, K) if trans_b else (K, N)), "int", dtype=dtype)
    R = oracle.round_f32(oracle.gemm(A, B, None, 1.0, 0.0, dtype, trans_b=trans_b))
    s = torch.cuda.current_stream().cuda_stream
    for pitch, dma in [(LIMIT[dtype] - STEP[dtype], True), (LIMIT[dtype], False)]:
        say(f"max pitch {dtype} trans_b={trans_b} pitch={pitch} ({'DMA' if dma else 'registers'})")
        bufa, dA = _pitched(A, pitch, dtype)
        bufb, dB = _pitched(B, pitch, dtype)
        for variant in ([dgt.VARIANT_MFMA_T256, dgt.VARIANT_AUTO] if dma
                        else [dgt.VARIANT_AUTO, dgt.VARIANT_MFMA_REGS]):
            C = torch.full((M, N), float("nan"), device="cuda")
            st = dgt.gemm_ex(CODE[dtype], 0, int(trans_b), variant, M, N, K, 1.0, dA.data_ptr(),
                             pitch, dB.data_ptr(), pitch, 0.0, C.data_ptr(), N, s)
            torch.cuda.synchronize()
            assert st == 0, dgt.gemm_status_string(st)
            assert_bit_exact(C.cpu().numpy(), R, f"{dtype} pitch {pitch} variant {variant}")
        if not dma:
            # the DMA rung refuses the pitch on the host, before any launch
            C = torch.zeros((M, N), device="cuda")
            st = dgt.gemm_ex(CODE[dtype], 0, int(trans_b), dgt.VARIANT_MFMA_T256, M, N, K, 1.0,
                             dA.data_ptr(), pitch, dB.data_ptr(), pitch, 0.0, C.data_ptr(), N, s)
            assert st == dgt.GEMM_ERR_VARIANT
        del bufa, bufb, dA, dB
        torch.cuda.empty_cache()
