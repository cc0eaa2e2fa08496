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
GEMM_ERR_SCRATCH = -9
NOALLOC_SCRATCH_BYTES = 64 << 20  # DGT_GEMM_NOALLOC_SCRATCH_BYTES

VARIANT_AUTO = 0
VARIANT_NAIVE = 1
VARIANT_LDS = 2
VARIANT_MFMA = 3
VARIANT_SKINNY = 4
VARIANT_MFMA_T256 = 5
VARIANT_MFMA_T128 = 6
VARIANT_MFMA_REGS = 7
VARIANTS = {"auto": VARIANT_AUTO, "naive": VARIANT_NAIVE, "lds": VARIANT_LDS,
            "mfma": VARIANT_MFMA, "skinny": VARIANT_SKINNY, "mfma256": VARIANT_MFMA_T256,
            "mfma128": VARIANT_MFMA_T128, "mfma_regs": VARIANT_MFMA_REGS}

# Every symbol the header declares (the tests check the library exports them).
EXPORTS = ("gemm_f32", "gemm_bf16", "gemm_f16", "gemm_f32_variant", "gemm_bf16_variant",
           "gemm_f16_variant", "gemm_ex", "gemm_strided_batched", "gemm_splitk",
           "gemm_splitk_noalloc", "gemm_splitk_slices", "gemm_splitk_workspace_size",
           "gemm_streamk", "gemm_streamk_workspace_size", "gemm_select_variant",
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
        lib.gemm_splitk_noalloc.restype = i
        lib.gemm_splitk_noalloc.argtypes = [i, i, i, *core[:11], i, p]
        lib.gemm_streamk.restype = i
        lib.gemm_streamk.argtypes = [i, i, i, *core[:11], p, i64, p]
        lib.gemm_streamk_workspace_size.restype = i64
        lib.gemm_streamk_workspace_size.argtypes = [i, i, i, i]
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


def gemm_splitk_noalloc(dtype, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                        splits, stream=0) -> int:
    return _load().gemm_splitk_noalloc(int(dtype), int(trans_a), int(trans_b), M, N, K, alpha, A,
                                       lda, B, ldb, beta, C, ldc, int(splits), stream)


def gemm_streamk(dtype, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                 workspace, workspace_bytes, stream=0) -> int:
    return _load().gemm_streamk(int(dtype), int(trans_a), int(trans_b), M, N, K, alpha, A, lda,
                                B, ldb, beta, C, ldc, workspace, int(workspace_bytes), stream)


def gemm_streamk_workspace_size(dtype, M, N, K) -> int:
    return _load().gemm_streamk_workspace_size(int(dtype), M, N, K)


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


def _check_layout(named, dims=(2,)):
    """Structure checks of the torch-facing calls, run before anything reaches
    the library: each (name, tensor) has a dimension count in ``dims`` and,
    unless it is empty, unit stride along its last axis (row-major rows).  A
    column-strided view would otherwise pass the leading-dimension check and
    read the wrong elements."""
    for name, t in named:
        if t.dim() not in dims:
            raise ValueError(f"{name} must have {' or '.join(map(str, dims))} dimensions, "
                             f"got {t.dim()}")
        if t.numel() > 0 and t.stride(-1) != 1:
            raise ValueError(f"{name} must be row-major with unit column stride")


def _check_device(named, device):
    """Every non-empty (name, tensor) must live on the GPU ``device``: a host
    tensor would hand a host pointer to a kernel."""
    for name, t in named:
        if t.numel() > 0 and (not t.is_cuda or t.device != device):
            raise ValueError(f"{name} must be a GPU tensor on {device}, got {t.device}")


def _dtype_code(A, B, C):
    import torch
    if A.dtype != B.dtype or A.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise TypeError("A and B must both be float32, both bfloat16 or both float16")
    if C.dtype != torch.float32:
        raise TypeError("C must be float32")
    return {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16,
            torch.float16: DTYPE_F16}[A.dtype]


def _stream_handle(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return stream


def gemm(A, B, C, alpha: float = 1.0, beta: float = 0.0, variant=VARIANT_AUTO,
         stream=None, trans_a: bool = False, trans_b: bool = False) -> int:
    """C <- alpha*op(A)*op(B) + beta*C on torch tensors (row-major, unit column
    stride).  op(X) is X, or X transposed when trans_x: then A is the stored
    K x M tensor, B the stored N x K tensor.

    A and B are float32, bfloat16 or float16 (16-bit bits are passed as-is),
    C float32.  ``variant`` is a ladder rung (enum gemm_variant) or its name
    in VARIANTS: "auto", "naive", "lds", "mfma", "skinny", "mfma256" /
    "mfma128" for the DMA kernels with a fixed workgroup tile, or
    "mfma_regs" for the register-staged MFMA kernel.
    Returns the status code; the work is queued on ``stream`` (default: torch's
    current stream) and not waited for.
    """
    if isinstance(variant, str):
        variant = VARIANTS[variant]
    dtype = _dtype_code(A, B, C)
    named = (("A", A), ("B", B), ("C", C))
    _check_layout(named)
    M, K = A.shape[::-1] if trans_a else A.shape
    K2, N = B.shape[::-1] if trans_b else B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, "
                         f"C {tuple(C.shape)}")
    _check_device(named, C.device)
    stream = _stream_handle(stream)
    lda, ldb, ldc = _ld(A), _ld(B), _ld(C)
    args = (M, N, K, float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb,
            float(beta), C.data_ptr(), ldc, stream)
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
    a 1-D tensor of N floats or a [1, N] tensor (shared by every problem), or
    a [batch, N] tensor (one row per problem).  Every tensor must be on C's
    GPU.  Returns the status code of gemm_strided_batched.
    """
    import torch

    if isinstance(variant, str):
        variant = VARIANTS[variant]
    dtype = _dtype_code(A, B, C)
    if C.dim() != 3:
        raise TypeError("C must be a 3-D float32 tensor")
    _check_layout((("A", A), ("B", B)), dims=(2, 3))
    _check_layout((("C", C),), dims=(3,))
    batch = C.shape[0]

    def mat(t, name):
        if t.dim() == 2:
            return t, 0
        if t.shape[0] not in (batch, 1):
            raise ValueError(f"{name} must be 2-D or [batch, rows, cols]")
        return t[0] if t.shape[0] == 1 else t, (0 if t.shape[0] == 1 else t.stride(0))

    def pitch(t):
        return _ld(t if t.dim() == 2 else t[0])

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
        if bias.dtype != torch.float32 or bias.dim() not in (1, 2) or bias.shape[-1] != N:
            raise ValueError("bias must be float32 [N], [1, N] or [batch, N]")
        if bias.dim() == 2 and bias.shape[0] not in (1, batch):
            raise ValueError(f"a 2-D bias must have 1 or batch = {batch} rows, "
                             f"got {bias.shape[0]}")
        _check_layout((("bias", bias),), dims=(1, 2))
        bias_ptr = bias.data_ptr()
        # one row shared by every problem reads with stride 0; otherwise row z
        # starts bias.stride(0) floats after row z - 1
        sbias = bias.stride(0) if bias.dim() == 2 and bias.shape[0] > 1 else 0
    _check_device((("A", A), ("B", B), ("C", C)) + ((("bias", bias),) if bias is not None
                                                     else ()), C.device)
    return gemm_strided_batched(dtype, trans_a, trans_b, variant, M, N, K, float(alpha),
                                A2.data_ptr(), pitch(A2), sa, B2.data_ptr(), pitch(B2), sb,
                                float(beta), C.data_ptr(), pitch(C), C.stride(0),
                                bias_ptr, sbias, batch, _stream_handle(stream))


def gemm_split(A, B, C, alpha: float = 1.0, beta: float = 0.0, splits: int = 0,
               workspace=None, stream=None, trans_a: bool = False,
               trans_b: bool = False) -> int:
    """Split-K form of ``gemm`` on torch tensors (gemm_splitk).  ``workspace``
    is a device tensor of at least gemm_splitk_workspace_size bytes; when None
    one is allocated here with torch (the library itself allocates nothing);
    a caller's workspace must be a contiguous GPU tensor on C's device.
    Returns the status code."""
    import torch

    dtype = _dtype_code(A, B, C)
    named = (("A", A), ("B", B), ("C", C))
    _check_layout(named)
    M, K = A.shape[::-1] if trans_a else A.shape
    K2, N = B.shape[::-1] if trans_b else B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, "
                         f"C {tuple(C.shape)}")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _check_device(named + ((("workspace", workspace),) if workspace is not None else ()),
                  C.device)
    need = gemm_splitk_workspace_size(dtype, M, N, K, splits)
    if need < 0:
        return need
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=C.device)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        ws_ptr = workspace.data_ptr() if workspace.numel() > 0 else 0
        ws_bytes = workspace.numel() * workspace.element_size()
    return gemm_splitk(dtype, trans_a, trans_b, M, N, K, float(alpha), A.data_ptr(), _ld(A),
                       B.data_ptr(), _ld(B), float(beta), C.data_ptr(), _ld(C), splits,
                       ws_ptr, ws_bytes, _stream_handle(stream))


def gemm_stream(A, B, C, alpha: float = 1.0, beta: float = 0.0, workspace=None, stream=None,
                trans_a: bool = False, trans_b: bool = False) -> int:
    """Stream-K form of ``gemm`` on torch tensors (gemm_streamk).  ``workspace``
    is a device tensor of at least gemm_streamk_workspace_size bytes; when
    None one is allocated here with torch (the library itself allocates
    nothing); a caller's workspace must be a contiguous GPU tensor on C's
    device.  Shapes stream-K does not cover run as ``gemm``.  Returns the
    status code."""
    import torch

    dtype = _dtype_code(A, B, C)
    named = (("A", A), ("B", B), ("C", C))
    _check_layout(named)
    M, K = A.shape[::-1] if trans_a else A.shape
    K2, N = B.shape[::-1] if trans_b else B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, "
                         f"C {tuple(C.shape)}")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _check_device(named + ((("workspace", workspace),) if workspace is not None else ()),
                  C.device)
    need = gemm_streamk_workspace_size(dtype, M, N, K)
    if need < 0:
        return need
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=C.device)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        ws_ptr = workspace.data_ptr() if workspace.numel() > 0 else 0
        ws_bytes = workspace.numel() * workspace.element_size()
    return gemm_streamk(dtype, trans_a, trans_b, M, N, K, float(alpha), A.data_ptr(), _ld(A),
                        B.data_ptr(), _ld(B), float(beta), C.data_ptr(), _ld(C), ws_ptr,
                        ws_bytes, _stream_handle(stream))
