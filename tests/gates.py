"""Acceptance gates for a device GEMM result against the oracle.

* Integer-valued inputs: every partial sum is an integer below 2**24 and the
  alpha/beta used are dyadic with few bits, so every correct summation order
  gives the same fp32 number: the device result must equal the oracle's fp64
  result rounded to fp32, bit for bit.
* Otherwise: normwise  ||C - R||_F / ||R||_F <= 1e-5  and elementwise
  max |C - R| <= 1e-4 * sqrt(K) * s,  s = max(1, |alpha|) * sigma_A * sigma_B
  (sigma = the scale of the input distribution).  When ||R||_F == 0 only the
  elementwise bound applies.  Both are computed in fp64.

A 16-bit-input matrix unit is expected to land 1e-4..1e-3 away from an fp32
reference computed on the unrounded data (dilfish.github.io section 5.5); the
oracle here consumes the already-rounded bf16 / fp16 inputs, so only fp32
accumulation error remains (about 2**-24 * sqrt(K) relative) and the 1e-5
gate applies to the 16-bit inputs as well.
"""

import math

import numpy as np

NORM_TOL = 1e-5
ELEM_TOL = 1e-4


def errors(C, R64):
    C = np.asarray(C, dtype=np.float64)
    R64 = np.asarray(R64, dtype=np.float64)
    d = C - R64
    nref = float(np.linalg.norm(R64))
    nerr = float(np.linalg.norm(d))
    rel = nerr / nref if nref > 0 else (0.0 if nerr == 0 else math.inf)
    mx = float(np.max(np.abs(d))) if d.size else 0.0
    return rel, mx, nref


def elem_bound(K, alpha, sigma_a=1.0, sigma_b=1.0):
    s = max(1.0, abs(alpha)) * sigma_a * sigma_b
    return ELEM_TOL * math.sqrt(max(K, 1)) * s


def assert_close(C, R64, K, alpha, sigma_a=1.0, sigma_b=1.0, what=""):
    assert np.all(np.isfinite(C)), f"{what}: non-finite values in result"
    rel, mx, nref = errors(C, R64)
    eb = elem_bound(K, alpha, sigma_a, sigma_b)
    if nref > 0:
        assert rel <= NORM_TOL, f"{what}: normwise rel err {rel:.3e} > {NORM_TOL}"
    assert mx <= eb, f"{what}: max abs err {mx:.3e} > bound {eb:.3e}"
    return rel, mx


def assert_bit_exact(C, R32, what=""):
    C = np.asarray(C, dtype=np.float32)
    R32 = np.asarray(R32, dtype=np.float32)
    assert C.shape == R32.shape, f"{what}: shape {C.shape} != {R32.shape}"
    bad = np.flatnonzero(C.view(np.uint32) != R32.view(np.uint32))
    if bad.size:
        i = bad[0]
        raise AssertionError(
            f"{what}: {bad.size} of {C.size} elements differ; first at flat "
            f"{i}: got {C.flat[i]!r} want {R32.flat[i]!r}")
