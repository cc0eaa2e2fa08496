"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each pin is a function of an oracle object so that the same checks can be
run against mutated builds of the oracle source (bottom of this file): a
plausible mistake (transposed operand, dropped or mis-signed beta term,
missing alpha, shortened k range, beta applied to an unread C) must make at
least one pin fail.

Where the pins come from:
* the operation: C(i,j) = sum_k A(i,k) B(k,j), generalised to
  alpha*A*B + beta*C (elainafan.one "稠密矩阵乘法"; dilfish.github.io 5.2);
* row-major storage (chongfengling.github.io 2.2; elainafan.one "行主序");
* transposed operands: op(X) = X^T, and the three products of a linear layer
  stored as X [batch, in], W [out, in], and its bias added to every row
  (elainafan.one "全连接层"); batches against numpy's batched matmul;
* identity / permutation / rank-1 algebra, exact small-integer arithmetic,
  numpy's float64 matmul as an independent library routine, and exact
  rational arithmetic (``fractions.Fraction``) with the textbook fp64
  dot-product error bound (Higham, Accuracy and Stability of Numerical
  Algorithms, chapter 3).
"""

import os
import random
from fractions import Fraction

import numpy as np
import pytest

import gemm_inputs as gi
import oracle

U64 = 2.0 ** -53


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.default()


def _rng_f32(seed, rows, cols):
    return gi.draw(seed, rows, cols, "uniform", dtype="f32")


def _ints(seed, rows, cols):
    return gi.draw(seed, rows, cols, "int", dtype="f32")


# ---------------------------------------------------------------- pins

def pin_identity(o):
    """A = I gives B back (and B = I gives A back), scaled exactly."""
    n, m = 33, 47
    B = _rng_f32(11, n, m)
    C0 = _rng_f32(12, n, m)
    I = np.eye(n, dtype=np.float32)
    R = o.gemm(I, B, None, 1.0, 0.0, "f32")
    assert np.array_equal(R, B.astype(np.float64)), "I*B != B"
    R = o.gemm(I, B, C0, 1.5, 0.5, "f32")
    want = 1.5 * B.astype(np.float64) + 0.5 * C0.astype(np.float64)  # exact
    assert np.array_equal(R, want), "1.5*I*B + 0.5*C0 wrong"
    A = _rng_f32(13, m, n)
    R = o.gemm(A, I, None, 1.0, 0.0, "f32")
    assert np.array_equal(R, A.astype(np.float64)), "A*I != A"


def pin_permutation(o):
    """A = P permutes the rows of B; B = Q permutes the columns of A."""
    n = 29
    p = np.random.default_rng(3).permutation(n)
    P = np.zeros((n, n), np.float32)
    P[np.arange(n), p] = 1.0          # (P B)[i,:] = B[p[i],:]
    B = _rng_f32(21, n, 40)
    R = o.gemm(P, B, None, 1.0, 0.0, "f32")
    assert np.array_equal(R, B[p].astype(np.float64)), "P*B is not B[p]"
    A = _rng_f32(22, 31, n)
    # (A Q)[:, j] = A[:, q[j]] when Q[q[j], j] = 1
    q = np.random.default_rng(4).permutation(n)
    Q = np.zeros((n, n), np.float32)
    Q[q, np.arange(n)] = 1.0
    R = o.gemm(A, Q, None, 1.0, 0.0, "f32")
    assert np.array_equal(R, A[:, q].astype(np.float64)), "A*Q is not A[:, q]"


def pin_rank1(o):
    """A = u v^T, B = w z^T  =>  C = alpha (v.w) u z^T + beta C0, exactly."""
    M, K, N = 17, 23, 19
    r = np.random.default_rng(5)
    u, v = r.integers(-3, 4, M), r.integers(-3, 4, K)
    w, z = r.integers(-3, 4, K), r.integers(-3, 4, N)
    A = np.outer(u, v).astype(np.float32)
    B = np.outer(w, z).astype(np.float32)
    C0 = r.integers(-5, 6, (M, N)).astype(np.float32)
    vw = int(np.dot(v, w))
    R = o.gemm(A, B, C0, 1.5, -0.5, "f32")
    want = 1.5 * vw * np.outer(u, z).astype(np.float64) - 0.5 * C0.astype(np.float64)
    assert np.array_equal(R, want), "rank-1 closed form violated"
    ones = np.ones((5, 7), np.float32)
    R = o.gemm(ones, np.ones((7, 3), np.float32), None, 1.0, 0.0, "f32")
    assert np.all(R == 7.0), "all-ones product must equal K"


def pin_small_integers(o):
    """Integer inputs are exact in any order: equal numpy float64 matmul."""
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (64, 48, 80), (100, 1, 129)]:
        A = _ints(31 + M, M, K)
        B = _ints(32 + N, K, N)
        R = o.gemm(A, B, None, 1.0, 0.0, "f32")
        want = A.astype(np.float64) @ B.astype(np.float64)
        assert np.array_equal(R, want), f"integer product wrong at {M}x{N}x{K}"


def pin_alpha_beta(o):
    """alpha = 0 gives beta*C0; beta = 0 never reads C0; K = 0 gives beta*C0."""
    M, N, K = 9, 11, 13
    A, B, C0 = _ints(41, M, K), _ints(42, K, N), _ints(43, M, N)
    R = o.gemm(A, B, C0, 0.0, 0.5, "f32")
    assert np.array_equal(R, 0.5 * C0.astype(np.float64)), "alpha=0 must give beta*C0"
    nan = np.full((M, N), np.nan, np.float32)
    R = o.gemm(A, B, nan, 2.0, 0.0, "f32")
    want = 2.0 * (A.astype(np.float64) @ B.astype(np.float64))
    assert np.all(np.isfinite(R)), "beta=0 must not read C0"
    assert np.array_equal(R, want), "beta=0 result wrong"
    Z = np.zeros((M, 0), np.float32)
    R = o.gemm(Z, np.zeros((0, N), np.float32), C0, 1.0, -2.0, "f32")
    assert np.array_equal(R, -2.0 * C0.astype(np.float64)), "K=0 must give beta*C0"
    R = o.gemm(A, B, C0, 1.5, 0.5, "f32")
    want = 1.5 * (A.astype(np.float64) @ B.astype(np.float64)) + 0.5 * C0
    assert np.array_equal(R, want), "alpha=1.5, beta=0.5 on integers must be exact"


def pin_exact_rational(o):
    """Sampled elements lie within the fp64 dot-product bound of the exact
    rational value:  |R - exact| <= (K+2) u (|alpha| sum|a b| + |beta c|)."""
    M, N, K = 6, 5, 301
    A, B, C0 = _rng_f32(51, M, K), _rng_f32(52, K, N), _rng_f32(53, M, N)
    alpha, beta = 1.25, -0.75
    R = o.gemm(A, B, C0, alpha, beta, "f32")
    Af = [[Fraction(float(x)) for x in row] for row in A]
    Bf = [[Fraction(float(x)) for x in row] for row in B]
    for i in range(M):
        for j in range(N):
            prods = [Af[i][k] * Bf[k][j] for k in range(K)]
            exact = Fraction(alpha) * sum(prods) + Fraction(beta) * Fraction(float(C0[i, j]))
            mag = abs(alpha) * sum(abs(float(p)) for p in prods) + abs(beta * float(C0[i, j]))
            err = abs(Fraction(float(R[i, j])) - exact)
            assert float(err) <= (K + 2) * U64 * mag * 1.0001, \
                f"element ({i},{j}) off by {float(err):.3e}"


def pin_library_float64(o):
    """Random real inputs: agree with numpy's float64 matmul to ~K ulps."""
    M, N, K = 40, 36, 250
    A, B = _rng_f32(61, M, K), _rng_f32(62, K, N)
    R = o.gemm(A, B, None, 1.0, 0.0, "f32")
    want = A.astype(np.float64) @ B.astype(np.float64)
    scale = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    assert np.all(np.abs(R - want) <= 2 * K * U64 * scale), "disagrees with numpy"


def pin_bf16_inputs(o):
    """bf16 bits denote the upper half of an fp32 value (dilfish.github.io 5.5
    table: 8-bit exponent, 7-bit mantissa); the oracle must use that value."""
    bits = np.array([[0x3F80, 0xC000], [0x3FC0, 0x0000]], np.uint16)  # 1, -2; 1.5, 0
    eye = np.array([[0x3F80, 0x0000], [0x0000, 0x3F80]], np.uint16)   # identity
    R = o.gemm(bits, eye, None, 1.0, 0.0, "bf16")
    assert np.array_equal(R, np.array([[1.0, -2.0], [1.5, 0.0]])), "bf16 widening wrong"
    A = gi.draw(71, 20, 30, "int", dtype="bf16")
    B = gi.draw(72, 30, 10, "int", dtype="bf16")
    R = o.gemm(A, B, None, 1.0, 0.0, "bf16")
    want = gi.bf16_bits_to_fp32(A).astype(np.float64) @ gi.bf16_bits_to_fp32(B).astype(np.float64)
    assert np.array_equal(R, want), "bf16 integer product wrong"


def pin_f16_inputs(o):
    """f16 bits are IEEE 754 binary16 (dilfish.github.io 5.5 table: 5-bit
    exponent, 10-bit mantissa).  Hand-decoded values, then every one of the
    65536 patterns except the NaNs against numpy's own float16 conversion."""
    hand = np.array([[0x3C00, 0xC000, 0x0001, 0x7BFF, 0x8400, 0x3555]], np.uint16)
    # 0x3555: exponent 13, fraction 0x155 -> 1365/4096, the binary16 nearest 1/3
    want = [1.0, -2.0, 2.0 ** -24, 65504.0, -2.0 ** -14, 1365 / 4096]
    got = o.widen(hand, "f16")
    assert got[0].tolist() == want, "f16 hand-decoded values wrong"
    allbits = np.arange(65536, dtype=np.uint16)
    ref = allbits.view(np.float16).astype(np.float64)
    keep = ~np.isnan(ref)
    got = o.widen(allbits.reshape(256, 256), "f16").reshape(-1)
    assert np.array_equal(got[keep], ref[keep]), "f16 decoding disagrees with numpy"
    assert np.all(np.isnan(got[~keep])), "f16 NaN patterns must decode to NaN"
    # product through the GEMM: small integers are exact in binary16
    A = gi.draw(73, 20, 30, "int", dtype="f16")
    B = gi.draw(74, 30, 10, "int", dtype="f16")
    R = o.gemm(A, B, None, 1.0, 0.0, "f16")
    want = (A.view(np.float16).astype(np.float64) @ B.view(np.float16).astype(np.float64))
    assert np.array_equal(R, want), "f16 integer product wrong"


def pin_leading_dims_rectangular(o):
    """Non-square shapes keep rows and columns apart: row i of C depends on
    row i of A only, column j on column j of B only."""
    M, N, K = 7, 13, 5
    A = np.zeros((M, K), np.float32)
    B = np.zeros((K, N), np.float32)
    A[2, 3] = 2.0      # only A(2,3) != 0
    B[3, 11] = 5.0     # only B(3,11) != 0
    R = o.gemm(A, B, None, 1.0, 0.0, "f32")
    want = np.zeros((M, N))
    want[2, 11] = 10.0
    assert np.array_equal(R, want), "single-entry product lands in the wrong place"


def pin_transposed_permutation(o):
    """A stored as P with trans_a gives op(A) = P^T: (P^T B)[p[i], :] = B[i, :].
    B stored as Q with trans_b gives op(B) = Q^T: (A Q^T)[:, q[j]] = A[:, j].
    Square operands, so a mistake in op() cannot read outside them."""
    n = 23
    p = np.random.default_rng(13).permutation(n)
    P = np.zeros((n, n), np.float32)
    P[np.arange(n), p] = 1.0
    B = _rng_f32(91, n, n)
    R = o.gemm(P, B, None, 1.0, 0.0, "f32", trans_a=True)
    assert np.array_equal(R[p], B.astype(np.float64)), "op(A) = P^T does not undo P"
    q = np.random.default_rng(14).permutation(n)
    Q = np.zeros((n, n), np.float32)
    Q[q, np.arange(n)] = 1.0
    A = _rng_f32(92, n, n)
    R = o.gemm(A, Q, None, 1.0, 0.0, "f32", trans_b=True)
    # Q^T[j, q[j]] = 1, so column q[j] of A Q^T is column j of A
    assert np.array_equal(R[:, q], A.astype(np.float64)), "op(B) = Q^T wrong"


def pin_transposed_rank1(o):
    """Stored A = v u^T (K x M) with trans_a, stored B = z w^T (N x K) with
    trans_b: op(A) op(B) = (v.w) u z^T, exactly; non-square on purpose."""
    M, K, N = 17, 23, 29
    r = np.random.default_rng(15)
    u, v = r.integers(-3, 4, M), r.integers(-3, 4, K)
    w, z = r.integers(-3, 4, K), r.integers(-3, 4, N)
    A_s = np.outer(v, u).astype(np.float32)
    B_s = np.outer(z, w).astype(np.float32)
    C0 = r.integers(-5, 6, (M, N)).astype(np.float32)
    want = 1.5 * int(np.dot(v, w)) * np.outer(u, z).astype(np.float64) + 0.5 * C0
    for ta, tb, A, B in [(True, True, A_s, B_s), (True, False, A_s, B_s.T.copy()),
                         (False, True, A_s.T.copy(), B_s)]:
        R = o.gemm(A, B, C0, 1.5, 0.5, "f32", trans_a=ta, trans_b=tb)
        assert np.array_equal(R, want), f"rank-1 with trans_a={ta}, trans_b={tb} wrong"


def pin_linear_layer_products(o):
    """The three products of a linear layer stored as X [batch, in], W [out,
    in], G [batch, out] (elainafan.one "全连接层"): X W^T, G^T X and G W, on
    small integers, equal numpy's float64 matmul of the explicit transposes."""
    batch, d_in, d_out = 12, 40, 24
    X = _ints(101, batch, d_in)
    W = _ints(102, d_out, d_in)
    G = _ints(103, batch, d_out)
    x, w, g = (t.astype(np.float64) for t in (X, W, G))
    Y = o.gemm(X, W, None, 1.0, 0.0, "f32", trans_b=True)
    assert np.array_equal(Y, x @ w.T), "forward X W^T wrong"
    dW = o.gemm(G, X, None, 1.0, 0.0, "f32", trans_a=True)
    assert np.array_equal(dW, g.T @ x), "weight gradient G^T X wrong"
    dX = o.gemm(G, W, None, 1.0, 0.0, "f32")
    assert np.array_equal(dX, g @ w), "input gradient G W wrong"
    # both flags: X stored transposed ([in, batch]) with W as is, op() = X, W^T
    Y2 = o.gemm(X.T.copy(), W, None, 1.0, 0.0, "f32", trans_a=True, trans_b=True)
    assert np.array_equal(Y2, x @ w.T), "trans_a and trans_b together wrong"


def pin_linear_bias(o):
    """F.linear's bias (elainafan.one "全连接层": X W^T + b): b is added to
    every row after the BLAS form, unscaled; numpy's float64 matmul plus a
    broadcast add on small integers is exact."""
    batch, d_in, d_out = 12, 40, 24
    X, W = _ints(111, batch, d_in), _ints(112, d_out, d_in)
    b = _ints(113, 1, d_out)[0]
    C0 = _ints(114, batch, d_out)
    x, w, c0, bb = (t.astype(np.float64) for t in (X, W, C0, b))
    Y = o.gemm(X, W, C0, 1.5, 0.5, "f32", trans_b=True, bias=b)
    assert np.array_equal(Y, 1.5 * (x @ w.T) + 0.5 * c0 + bb[None, :]), "bias epilogue wrong"
    Y = o.gemm(X, W, None, 0.0, 0.0, "f32", trans_b=True, bias=b)
    assert np.array_equal(Y, np.broadcast_to(bb, (batch, d_out))), "alpha = 0: C must be the bias"
    Z = o.gemm(np.zeros((batch, 0), np.float32), np.zeros((d_out, 0), np.float32), C0, 1.0,
               -2.0, "f32", trans_b=True, bias=b)
    assert np.array_equal(Z, -2.0 * c0 + bb[None, :]), "K = 0: C must be beta*C0 + bias"


def pin_batched(o):
    """A batch is independent problems: numpy's batched matmul (np.matmul on
    3-D stacks) of the same stacks, with a shared and a per-problem operand."""
    nb, M, N, K = 3, 7, 9, 11
    A3 = np.stack([_ints(120 + z, M, K) for z in range(nb)])
    B = _ints(125, K, N)                                   # shared by every problem
    B3t = np.stack([_ints(130 + z, N, K) for z in range(nb)])  # stored transposed
    C03 = np.stack([_ints(135 + z, M, N) for z in range(nb)])
    bias = np.stack([_ints(140 + z, 1, N)[0] for z in range(nb)])
    a3, b, c03, bs = (t.astype(np.float64) for t in (A3, B, C03, bias))
    R = o.gemm_batched(A3, [B] * nb, C03, 2.0, -1.0, "f32", biases=bias)
    assert np.array_equal(R, 2.0 * np.matmul(a3, b) - c03 + bs[:, None, :]), "batch wrong"
    R = o.gemm_batched(A3, B3t, None, 1.0, 0.0, "f32", trans_b=True)
    want = np.matmul(a3, B3t.astype(np.float64).transpose(0, 2, 1))
    assert np.array_equal(R, want), "batch with stored-transposed B wrong"


PINS = [pin_identity, pin_permutation, pin_rank1, pin_small_integers,
        pin_alpha_beta, pin_exact_rational, pin_library_float64, pin_bf16_inputs,
        pin_f16_inputs, pin_leading_dims_rectangular, pin_transposed_permutation,
        pin_transposed_rank1, pin_linear_layer_products, pin_linear_bias, pin_batched]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_loop_orders_bit_identical(orc):
    """The threaded i-k-j order and the literal i-j-k loop agree bit for bit."""
    for (M, N, K) in [(1, 1, 1), (17, 33, 65), (64, 70, 300)]:
        A, B, C0 = _rng_f32(81, M, K), _rng_f32(82, K, N), _rng_f32(83, M, N)
        r1 = orc.gemm(A, B, C0, 1.5, 0.5, "f32", order="ikj")
        r2 = orc.gemm(A, B, C0, 1.5, 0.5, "f32", order="ijk")
        assert np.array_equal(r1.view(np.uint64), r2.view(np.uint64))


def test_tiny_brute_force(orc):
    """M, N, K in 1..8: a hand-written Python triple loop over the page's
    i-j-p order (elainafan.one matmul_cpu) in fp64 gives the same bits."""
    rnd = random.Random(9)
    for _ in range(40):
        M, N, K = rnd.randint(1, 8), rnd.randint(1, 8), rnd.randint(1, 8)
        A, B = _rng_f32(rnd.randint(0, 10**6), M, K), _rng_f32(rnd.randint(0, 10**6), K, N)
        R = orc.gemm(A, B, None, 1.0, 0.0, "f32")
        for i in range(M):
            for j in range(N):
                s = 0.0
                for p in range(K):
                    s += float(A[i, p]) * float(B[p, j])
                assert R[i, j] == s


def test_round_f32_nearest_even(orc):
    x = np.array([1.0 + 2**-24, 1.0 + 3 * 2**-24, -(1.0 + 2**-24 + 2**-40), 0.1])
    r = orc.round_f32(x)
    assert r.tolist() == [1.0, np.float32(1.0 + 2**-22), np.float32(-(1.0 + 2**-23)),
                          np.float32(0.1)]


# ------------------------------------------------- planted mistakes (CPU)

MUTANTS = {
    "transposed_B": ("acc[j] += a * brow[j];", "acc[j] += a * B[j * ldb + k];"),
    "transposed_A": ("const double a = A[i * lda + k];", "const double a = A[k * lda + i];"),
    "dropped_beta": ("if (beta != 0.0) r += beta * (*c0);", ""),
    "beta_sign": ("if (beta != 0.0) r += beta * (*c0);", "if (beta != 0.0) r -= beta * (*c0);"),
    "no_alpha": ("double r = alpha * acc;", "double r = acc;"),
    "reads_c_when_beta_zero": ("if (beta != 0.0) r += beta * (*c0);", "if (c0) r += beta * (*c0);"),
    "short_k": ("for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 0; k + 1 < K; ++k) {"),
    "acc_not_reset": ("for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;",
                      "if (i == 0) for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;"),
    "float_accumulator": ("acc[j] += a * brow[j];", "acc[j] = (float)(acc[j] + a * brow[j]);"),
    "f16_bias": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    "f16_subnormal": ("if (e == 0) v = ldexp((double)f, -24);",
                      "if (e == 0) v = ldexp((double)(1024 + f), -25);"),
    "f16_sign": ("return sign ? -v : v;", "return v;"),
    "op_ignores_trans": ("out[r * cols + c] = trans ? X[c * ld + r] : X[r * ld + c];",
                         "out[r * cols + c] = X[r * ld + c];"),
    "bias_dropped": ("return bias ? r + bias[j] : r;", "return r;"),
    "bias_one_column": ("return bias ? r + bias[j] : r;", "return bias ? r + bias[0] : r;"),
    "bias_subtracted": ("return bias ? r + bias[j] : r;", "return bias ? r - bias[j] : r;"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, mutant_dir):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    # plant the mistake in the threaded i-k-j path only (the one every
    # caller uses); the literal i-j-k loop stays intact
    head, sep, tail = src.partition("void oracle_gemm(")
    assert sep
    if old in tail:
        tail = tail.replace(old, new, 1)
    else:
        head = head.replace(old, new, 1)
    path_c = os.path.join(str(mutant_dir), f"{name}.c")
    with open(path_c, "w") as f:
        f.write(head + sep + tail)
    lib = oracle.compile_source(path_c, os.path.join(str(mutant_dir), f"lib{name}.so"))
    mutant = oracle.Oracle(lib)
    # stop at the first pin that objects: a mutant that indexes wrongly may
    # read past its buffers, and later pins would only widen that read
    failed = []
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, OverflowError):
            failed.append(pin.__name__)
            break
    assert failed, f"no pin catches the planted mistake {name!r}"
