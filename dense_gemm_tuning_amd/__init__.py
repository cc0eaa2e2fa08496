"""Python binding of the gfx950 dense GEMM library (``libdgt_gemm.so``).

Argument marshalling only: every function forwards to the C entry point of
the same name in ``include/dgt_gemm.h``; all arithmetic happens in the HIP
kernels behind it.  Pointers are device addresses passed as Python ints,
``stream`` is a ``hipStream_t`` as an int (0 = null stream).  Each function
returns the library's status code (0 = GEMM_OK); ``check`` turns a non-zero
status into an exception.

``gemm(A, B, C, alpha, beta, variant, trans_a=..., trans_b=...)`` is a
convenience for torch tensors on the GPU: it reads shapes, leading dimensions
(``stride(0)``) and ``torch.cuda.current_stream()`` and calls ``gemm_f32`` /
``gemm_bf16`` / ``gemm_f16`` (or ``gemm_ex`` for transposed or explicit-rung
calls).  Torch is used for memory and streams only.

There is no fallback: if the library has not been built, every call raises.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib",
                        "libdgt_gemm.so")

GEMM_OK = 0
GEMM_ERR_DIM = -1
GEMM_ERR_LD = -2
GEMM_ERR_NULL = -3
GEMM_ERR_OVERLAP = -4
GEMM_ERR_VARIANT = -5
GEMM_ERR_LAUNCH = -6
GEMM_ERR_ARG = -7
GEMM_ERR_WORKSPACE = -8

VARIANT_AUTO = 0
VARIANT_NAIVE = 1
VARIANT_LDS = 2
VARIANT_MFMA = 3
VARIANT_SKINNY = 4
VARIANT_MFMA_T256 = 5
VARIANT_MFMA_T128 = 6
VARIANTS = {"auto": VARIANT_AUTO, "naive": VARIANT_NAIVE, "lds": VARIANT_LDS,
            "mfma": VARIANT_MFMA, "skinny": VARIANT_SKINNY, "mfma256": VARIANT_MFMA_T256,
            "mfma128": VARIANT_MFMA_T128}

# Every symbol the header declares (the tests check the library exports them).
EXPORTS = ("gemm_f32", "gemm_bf16", "gemm_f16", "gemm_f32_variant", "gemm_bf16_variant",
           "gemm_f16_variant", "gemm_ex", "gemm_strided_batched", "gemm_splitk",
           "gemm_splitk_slices", "gemm_splitk_workspace_size", "gemm_select_variant",
           "gemm_status_string", "gemm_abi_version")

DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_F16 = 2

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(gemm_status_string(status))
        self.status = status


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP GEMM library not built ({LIB_PATH} missing); run "
                "`python -m dense_gemm_tuning_amd.build` or "
                "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        i, f, p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
        core = [i, i, i, f, p, i, p, i, f, p, i, p]
        for name in ("gemm_f32", "gemm_bf16", "gemm_f16"):
            fn = getattr(lib, name)
            fn.restype = i
            fn.argtypes = core
        for name in ("gemm_f32_variant", "gemm_bf16_variant", "gemm_f16_variant"):
            fn = getattr(lib, name)
            fn.restype = i
            fn.argtypes = [i, *core]
        lib.gemm_ex.restype = i
        lib.gemm_ex.argtypes = [i, i, i, i, *core]
        i64 = ctypes.c_int64
        lib.gemm_splitk.restype = i
        lib.gemm_splitk.argtypes = [i, i, i, *core[:11], i, p, i64, p]
        lib.gemm_splitk_slices.restype = i
        lib.gemm_splitk_slices.argtypes = [i, i, i, i, i]
        lib.gemm_splitk_workspace_size.restype = i64
        lib.gemm_splitk_workspace_size.argtypes = [i, i, i, i, i]
        lib.gemm_strided_batched.restype = i
        lib.gemm_strided_batched.argtypes = [i, i, i, i, i, i, i, f, p, i, i64, p, i, i64, f,
                                             p, i, i64, p, i64, i, p]
        lib.gemm_select_variant.restype = i
        lib.gemm_select_variant.argtypes = [i] * 9
        lib.gemm_status_string.restype = ctypes.c_char_p
        lib.gemm_status_string.argtypes = [i]
        lib.gemm_abi_version.restype = i
        lib.gemm_abi_version.argtypes = []
        _lib = lib
    return _lib


def library() -> ctypes.CDLL:
    """The loaded ctypes handle (raises if the library is not built)."""
    return _load()


def gemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return _load().gemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_bf16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return _load().gemm_bf16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_f16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return _load().gemm_f16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_f32_variant(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                     stream=0) -> int:
    return _load().gemm_f32_variant(variant, M, N, K, alpha, A, lda, B, ldb, beta,
                                    C, ldc, stream)


def gemm_bf16_variant(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                      stream=0) -> int:
    return _load().gemm_bf16_variant(variant, M, N, K, alpha, A, lda, B, ldb, beta,
                                     C, ldc, stream)


def gemm_f16_variant(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                     stream=0) -> int:
    return _load().gemm_f16_variant(variant, M, N, K, alpha, A, lda, B, ldb, beta,
                                    C, ldc, stream)


def gemm_ex(dtype, trans_a, trans_b, variant, M, N, K, alpha, A, lda, B, ldb, beta, C,
            ldc, stream=0) -> int:
    return _load().gemm_ex(int(dtype), int(trans_a), int(trans_b), int(variant), M, N, K,
                           alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_strided_batched(dtype, trans_a, trans_b, variant, M, N, K, alpha, A, lda, stride_a,
                         B, ldb, stride_b, beta, C, ldc, stride_c, bias, stride_bias, batch,
                         stream=0) -> int:
    return _load().gemm_strided_batched(int(dtype), int(trans_a), int(trans_b), int(variant),
                                        M, N, K, alpha, A, lda, stride_a, B, ldb, stride_b,
                                        beta, C, ldc, stride_c, bias, stride_bias, batch,
                                        stream)


def gemm_splitk(dtype, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                workspace, workspace_bytes, stream=0) -> int:
    return _load().gemm_splitk(int(dtype), int(trans_a), int(trans_b), M, N, K, alpha, A, lda,
                               B, ldb, beta, C, ldc, int(splits), workspace,
                               int(workspace_bytes), stream)


def gemm_splitk_slices(dtype, M, N, K, splits) -> int:
    return _load().gemm_splitk_slices(int(dtype), M, N, K, int(splits))


def gemm_splitk_workspace_size(dtype, M, N, K, splits) -> int:
    return _load().gemm_splitk_workspace_size(int(dtype), M, N, K, int(splits))


def gemm_select_variant(dtype, trans_a, trans_b, M, N, K, lda, ldb, ldc) -> int:
    """dtype: DTYPE_F32, DTYPE_BF16 or DTYPE_F16; trans_a, trans_b: 0 or 1."""
    return _load().gemm_select_variant(int(dtype), int(trans_a), int(trans_b), M, N, K,
                                       lda, ldb, ldc)


def gemm_status_string(status: int) -> str:
    return _load().gemm_status_string(status).decode()


def gemm_abi_version() -> int:
    return _load().gemm_abi_version()


def check(status: int) -> None:
    if status != GEMM_OK:
        raise GemmError(status)


def _ld(t) -> int:
    """Row pitch of a 2-D tensor; for an empty or single-row operand the pitch
    is never used (torch may report 0), so report a legal one."""
    rows, cols = t.shape
    if rows <= 1 or t.numel() == 0:
        return max(t.stride(0), cols, 1)
    return t.stride(0)


def gemm(A, B, C, alpha: float = 1.0, beta: float = 0.0, variant=VARIANT_AUTO,
         stream=None, trans_a: bool = False, trans_b: bool = False) -> int:
    """C <- alpha*op(A)*op(B) + beta*C on torch tensors (row-major, unit column
    stride).  op(X) is X, or X transposed when trans_x: then A is the stored
    K x M tensor, B the stored N x K tensor.

    A and B are float32, bfloat16 or float16 (16-bit bits are passed as-is),
    C float32.  ``variant`` is a ladder rung (enum gemm_variant) or its name
    in VARIANTS: "auto", "naive", "lds", "mfma", "skinny", or "mfma256" /
    "mfma128" for the DMA kernels with a fixed workgroup tile.
    Returns the status code; the work is queued on ``stream`` (default: torch's
    current stream) and not waited for.
    """
    import torch

    if isinstance(variant, str):
        variant = VARIANTS[variant]
    if A.dtype != B.dtype or A.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise TypeError("A and B must both be float32, both bfloat16 or both float16")
    if C.dtype != torch.float32:
        raise TypeError("C must be float32")
    for t in (A, B, C):
        if t.dim() != 2 or (t.numel() > 0 and t.stride(1) != 1):
            raise ValueError("operands must be 2-D row-major with unit column stride")
        if t.numel() > 0 and not t.is_cuda:
            raise ValueError("operands must be GPU tensors")
    M, K = A.shape[::-1] if trans_a else A.shape
    K2, N = B.shape[::-1] if trans_b else B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, "
                         f"C {tuple(C.shape)}")
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    lda, ldb, ldc = _ld(A), _ld(B), _ld(C)
    args = (M, N, K, float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb,
            float(beta), C.data_ptr(), ldc, stream)
    dtype = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16,
             torch.float16: DTYPE_F16}[A.dtype]
    if trans_a or trans_b:
        return gemm_ex(dtype, trans_a, trans_b, variant, *args)
    auto_fn, var_fn = {DTYPE_F32: (gemm_f32, gemm_f32_variant),
                       DTYPE_BF16: (gemm_bf16, gemm_bf16_variant),
                       DTYPE_F16: (gemm_f16, gemm_f16_variant)}[dtype]
    if variant == VARIANT_AUTO:
        return auto_fn(*args)
    return var_fn(variant, *args)


def gemm_batched(A, B, C, alpha: float = 1.0, beta: float = 0.0, bias=None,
                 variant=VARIANT_AUTO, stream=None, trans_a: bool = False,
                 trans_b: bool = False) -> int:
    """C[z] <- alpha*op(A[z])*op(B[z]) + beta*C[z] + bias[z] on torch tensors.

    A, B and C are 3-D (batch first; a batch stride of 0, e.g. from
    ``expand``, shares one matrix) or 2-D for an operand shared by every
    problem; each matrix is row-major with unit column stride.  bias is None,
    a 1-D tensor of N floats (shared) or a 2-D [batch, N] tensor.  Returns
    the status code of gemm_strided_batched.
    """
    import torch

    if isinstance(variant, str):
        variant = VARIANTS[variant]
    if A.dtype != B.dtype or A.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise TypeError("A and B must both be float32, both bfloat16 or both float16")
    if C.dtype != torch.float32 or C.dim() != 3:
        raise TypeError("C must be a 3-D float32 tensor")
    batch = C.shape[0]

    def mat(t, name):
        if t.dim() == 2:
            return t, 0
        if t.dim() != 3 or t.shape[0] not in (batch, 1):
            raise ValueError(f"{name} must be 2-D or [batch, rows, cols]")
        return t[0] if t.shape[0] == 1 else t, (0 if t.shape[0] == 1 else t.stride(0))

    def pitch(t):
        m = t if t.dim() == 2 else t[0]
        if m.numel() > 0 and m.stride(1) != 1:
            raise ValueError("matrices must be row-major with unit column stride")
        return _ld(m)

    A2, sa = mat(A, "A")
    B2, sb = mat(B, "B")
    a_rows, a_cols = A2.shape[-2:]
    b_rows, b_cols = B2.shape[-2:]
    M, K = (a_cols, a_rows) if trans_a else (a_rows, a_cols)
    K2, N = (b_cols, b_rows) if trans_b else (b_rows, b_cols)
    if K2 != K or tuple(C.shape[1:]) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, "
                         f"C {tuple(C.shape)}")
    bias_ptr, sbias = 0, 0
    if bias is not None:
        if bias.dtype != torch.float32 or bias.shape[-1] != N or bias.stride(-1) != 1:
            raise ValueError("bias must be float32 [N] or [batch, N] with unit stride")
        bias_ptr = bias.data_ptr()
        sbias = bias.stride(0) if bias.dim() == 2 else 0
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    dtype = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16,
             torch.float16: DTYPE_F16}[A.dtype]
    return gemm_strided_batched(dtype, trans_a, trans_b, variant, M, N, K, float(alpha),
                                A2.data_ptr(), pitch(A2), sa, B2.data_ptr(), pitch(B2), sb,
                                float(beta), C.data_ptr(), pitch(C), C.stride(0),
                                bias_ptr, sbias, batch, stream)


def gemm_split(A, B, C, alpha: float = 1.0, beta: float = 0.0, splits: int = 0,
               workspace=None, stream=None, trans_a: bool = False,
               trans_b: bool = False) -> int:
    """Split-K form of ``gemm`` on torch tensors (gemm_splitk).  ``workspace``
    is a device tensor of at least gemm_splitk_workspace_size bytes; when None
    one is allocated here with torch (the library itself allocates nothing).
    Returns the status code."""
    import torch

    if A.dtype != B.dtype or A.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise TypeError("A and B must both be float32, both bfloat16 or both float16")
    if C.dtype != torch.float32:
        raise TypeError("C must be float32")
    M, K = A.shape[::-1] if trans_a else A.shape
    K2, N = B.shape[::-1] if trans_b else B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, "
                         f"C {tuple(C.shape)}")
    dtype = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16,
             torch.float16: DTYPE_F16}[A.dtype]
    need = gemm_splitk_workspace_size(dtype, M, N, K, splits)
    if need < 0:
        return need
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=C.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    return gemm_splitk(dtype, trans_a, trans_b, M, N, K, float(alpha), A.data_ptr(), _ld(A),
                       B.data_ptr(), _ld(B), float(beta), C.data_ptr(), _ld(C), splits,
                       ws_ptr, ws_bytes, stream)
