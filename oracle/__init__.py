"""CPU oracle for C = alpha*A*B + beta*C (fp64, plain loops).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline leg may import this package; the product path (the HIP library and
its binding) never does, and this package never imports the product.

The arithmetic lives in ``gemm_oracle.c`` (built with gcc into
``liboracle.so`` next to it); this module only marshals numpy arrays.  What
the oracle computes and which passage each part follows is stated at the top
of the C file.  The tests pin it against identity and permutation matrices,
rank-1 closed forms, small-integer matrices (exact), the alpha/beta readings,
exact rational arithmetic on sampled elements, numpy's float64 matmul, and
the linear-layer products with transposed operands.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gemm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_d = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64

GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-std=c11", "-shared", "-fPIC"]


def compile_source(src: str, out: str) -> str:
    """Compile one oracle C source into a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile liboracle.so (OpenMP, strict IEEE, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        compile_source(SOURCE, _LIB)
    return _LIB


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_d)


class Oracle:
    """numpy-facing wrapper around one build of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        for name in ("oracle_gemm", "oracle_gemm_ijk"):
            f = getattr(lib, name)
            f.restype = None
            f.argtypes = [_i64, _i64, _i64, ctypes.c_double, _d, _i64, _d, _i64,
                          ctypes.c_double, _d, _i64, _d, _d, _i64]
        lib.oracle_widen_f32.argtypes = [ctypes.c_void_p, _i64, _i64, _i64, _d]
        lib.oracle_widen_bf16.argtypes = [ctypes.c_void_p, _i64, _i64, _i64, _d]
        lib.oracle_widen_f16.argtypes = [ctypes.c_void_p, _i64, _i64, _i64, _d]
        lib.oracle_round_f32.argtypes = [_d, _i64, ctypes.c_void_p]
        lib.oracle_op.restype = None
        lib.oracle_op.argtypes = [_d, _i64, _i64, _i64, ctypes.c_int, _d]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        self.lib = lib

    def widen(self, x: np.ndarray, dtype: str) -> np.ndarray:
        """Exact fp64 values of an input matrix (fp32 array, bf16 or f16 bits)."""
        x = np.ascontiguousarray(x)
        rows, cols = x.shape
        out = np.empty((rows, cols), dtype=np.float64)
        if dtype == "f32":
            assert x.dtype == np.float32
            self.lib.oracle_widen_f32(x.ctypes.data, rows, cols, cols, _ptr(out))
        elif dtype == "bf16":
            assert x.dtype == np.uint16
            self.lib.oracle_widen_bf16(x.ctypes.data, rows, cols, cols, _ptr(out))
        elif dtype == "f16":
            assert x.dtype == np.uint16
            self.lib.oracle_widen_f16(x.ctypes.data, rows, cols, cols, _ptr(out))
        else:
            raise ValueError(dtype)
        return out

    def gemm64(self, A64, B64, C0_64, alpha: float, beta: float,
               order: str = "ikj", bias=None) -> np.ndarray:
        """alpha*A*B + beta*C0 (+ bias on every row) in fp64 on already-widened
        operands.

        ``C0_64`` may be given even when ``beta == 0``; the oracle must then
        ignore it (that reading is pinned by a test with a NaN-filled C0).
        """
        A64 = np.ascontiguousarray(A64, dtype=np.float64)
        B64 = np.ascontiguousarray(B64, dtype=np.float64)
        M, K = A64.shape
        K2, N = B64.shape
        assert K == K2
        R = np.empty((M, N), dtype=np.float64)
        if C0_64 is not None:
            C0_64 = np.ascontiguousarray(C0_64, dtype=np.float64)
            assert C0_64.shape == (M, N)
            cptr = _ptr(C0_64)
        else:
            if beta != 0.0:
                raise ValueError("beta != 0 needs C0")
            cptr = _d()
        bptr = _d()
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float64)
            assert bias.shape == (N,)
            bptr = _ptr(bias)
        fn = self.lib.oracle_gemm if order == "ikj" else self.lib.oracle_gemm_ijk
        fn(M, N, K, float(alpha), _ptr(A64), max(K, 1), _ptr(B64), max(N, 1),
           float(beta), cptr, max(N, 1), bptr, _ptr(R), max(N, 1))
        return R

    def op(self, X64: np.ndarray, trans: bool) -> np.ndarray:
        """op(X) of a stored fp64 matrix: X, or its transpose when trans."""
        X64 = np.ascontiguousarray(X64, dtype=np.float64)
        srows, scols = X64.shape
        rows, cols = (scols, srows) if trans else (srows, scols)
        out = np.empty((rows, cols), dtype=np.float64)
        self.lib.oracle_op(_ptr(X64), rows, cols, max(scols, 1), int(bool(trans)), _ptr(out))
        return out

    def gemm(self, A, B, C0, alpha: float, beta: float, dtype: str,
             order: str = "ikj", trans_a: bool = False, trans_b: bool = False,
             bias=None) -> np.ndarray:
        """Oracle result in fp64 for raw inputs (fp32 arrays, bf16 or f16 bits).

        A and B are given as stored: K x M when trans_a, N x K when trans_b;
        bias is None or N fp32 values added to every row."""
        A64 = self.op(self.widen(A, dtype), trans_a)
        B64 = self.op(self.widen(B, dtype), trans_b)
        C64 = self.widen(C0, "f32") if C0 is not None else None
        b64 = None if bias is None else self.widen(np.asarray(bias, np.float32)[None, :], "f32")[0]
        return self.gemm64(A64, B64, C64, alpha, beta, order, b64)

    def gemm_batched(self, As, Bs, C0s, alpha: float, beta: float, dtype: str,
                     trans_a: bool = False, trans_b: bool = False, biases=None) -> np.ndarray:
        """A batch of independent problems, one after another: As, Bs (stored
        shapes), C0s and biases are sequences (or 3-D / 2-D arrays) of the
        same length; C0s and biases may be None.  Returns [batch, M, N]."""
        out = []
        for z in range(len(As)):
            out.append(self.gemm(As[z], Bs[z], None if C0s is None else C0s[z], alpha, beta,
                                 dtype, trans_a=trans_a, trans_b=trans_b,
                                 bias=None if biases is None else biases[z]))
        return np.stack(out) if out else np.zeros((0, 0, 0))

    def round_f32(self, R64: np.ndarray) -> np.ndarray:
        """fp64 -> fp32, nearest-even."""
        R64 = np.ascontiguousarray(R64, dtype=np.float64)
        out = np.empty(R64.shape, dtype=np.float32)
        self.lib.oracle_round_f32(_ptr(R64), R64.size, out.ctypes.data)
        return out

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))


_default = None


def default() -> Oracle:
    """The oracle built from ``gemm_oracle.c`` (built on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _default = Oracle(_LIB)
    return _default


def widen(x, dtype):
    return default().widen(x, dtype)


def gemm64(A64, B64, C0_64, alpha, beta, order="ikj"):
    return default().gemm64(A64, B64, C0_64, alpha, beta, order)


def gemm(A, B, C0, alpha, beta, dtype, order="ikj", trans_a=False, trans_b=False, bias=None):
    return default().gemm(A, B, C0, alpha, beta, dtype, order, trans_a, trans_b, bias)


def gemm_batched(As, Bs, C0s, alpha, beta, dtype, trans_a=False, trans_b=False, biases=None):
    return default().gemm_batched(As, Bs, C0s, alpha, beta, dtype, trans_a, trans_b, biases)


def round_f32(R64):
    return default().round_f32(R64)


def num_threads():
    return default().num_threads()


def set_num_threads(n):
    default().set_num_threads(n)
