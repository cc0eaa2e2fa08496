"""Seeded, version-stable synthetic inputs for the dense GEMM workloads.

This module is shared by the tests, the bench and the smoke check.  It holds
no GEMM arithmetic at all: it only draws numbers and rounds them to the input
precision a workload asks for.  Both the HIP library and the oracle consume
the arrays it returns; neither side draws numbers of its own.

Stream: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; the mixing constants are the ones of
Vigna's public-domain reference).  Element ``i`` of a stream is
``mix64(seed + (i + 1) * 0x9E3779B97F4A7C15)`` modulo 2**64, so any slice of a
matrix can be regenerated without the rest.

Distributions (row-major element order):

* ``uniform``  -- ``2 * ((z >> 40) * 2**-24) - 1``: uniform on [-1, 1) with
  step 2**-23, every value exact in fp32.
* ``int``      -- ``((z >> 32) mod 7) - 3``: integers in {-3..3}.  Products
  and sums of these stay exact in fp32 while ``9 K < 2**24``.
* ``normal``   -- Box-Muller in fp64 on consecutive pairs
  ``u1 = ((z0 >> 11) + 1) * 2**-53``, ``u2 = (z1 >> 11) * 2**-53``;
  the pair gives ``r cos(2 pi u2)`` and ``r sin(2 pi u2)``; scaled by sigma.

Precision: fp32 inputs are the fp64 draw rounded to nearest-even fp32.  bf16
inputs are that fp32 value rounded to nearest-even bf16 (the upper 16 bits,
returned as raw ``uint16`` bit patterns); f16 inputs are that fp32 value
rounded to nearest-even IEEE binary16 (numpy's conversion), also returned as
raw ``uint16`` bits.  The workloads never produce NaN or infinity.

Workloads: the pages tune a single operation, ``C = alpha*A*B + beta*C`` with
row-major A (M x K), B (K x N), C (M x N) (elainafan.one, "稠密矩阵乘法" and
"行主序").  ``WORKLOADS`` lists the shapes the library is checked and
measured on: a small square case, a ragged one that exercises edge masking
and the beta path, the FP32 4096^3 and BF16/FP16 8192^3 square cases the
pages' tuning ladders target (qwbw.cn, section 三 table at 4096^3), a skinny
decode-style case whose time is weight loading (dilfish.github.io, section
5.1 table, GEMV row), the BF16 square and skinny cases again with the
operands stored the way a linear layer keeps them, that layer's forward with
its bias, and a strided batch of independent products.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)

# Chunk size for streaming generation, so that huge matrices never need a
# second full-size uint64 temporary.
_CHUNK = 1 << 22


def splitmix64(seed: int, count: int, start: int = 0) -> np.ndarray:
    """Return elements ``start .. start+count-1`` of the SplitMix64 stream."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        z = z ^ (z >> np.uint64(31))
    return z


def _uniform(z: np.ndarray) -> np.ndarray:
    return (2.0 * ((z >> np.uint64(40)).astype(np.float64) * 2.0**-24) - 1.0)


def _ints(z: np.ndarray) -> np.ndarray:
    return ((z >> np.uint64(32)) % np.uint64(7)).astype(np.float64) - 3.0


def _normal(z: np.ndarray, start: int) -> np.ndarray:
    """Box-Muller on the aligned pairs (2p, 2p+1) of the stream."""
    assert start % 2 == 0 and z.size % 2 == 0
    z0 = z[0::2]
    z1 = z[1::2]
    u1 = ((z0 >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0**-53
    u2 = (z1 >> np.uint64(11)).astype(np.float64) * 2.0**-53
    r = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(z.size, dtype=np.float64)
    out[0::2] = r * np.cos(2.0 * math.pi * u2)
    out[1::2] = r * np.sin(2.0 * math.pi * u2)
    return out


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to nearest-even bf16; return the raw uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_fp32(h: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to the fp32 value they denote (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(seed: int, rows: int, cols: int, dist: str, sigma: float = 1.0,
         dtype: str = "f32") -> np.ndarray:
    """Draw a packed row-major ``rows x cols`` matrix.

    ``dtype`` is ``"f32"`` (returns float32), ``"bf16"`` or ``"f16"`` (return
    uint16 bit patterns).  ``dist`` is ``"uniform"``, ``"int"`` or ``"normal"``.
    """
    n = rows * cols
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
    elif dtype in ("bf16", "f16"):
        out = np.empty(n, dtype=np.uint16)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    for s in range(0, n, _CHUNK):
        cnt = min(_CHUNK, n - s)
        if dist == "normal" and cnt % 2:
            # keep Box-Muller pairs aligned: draw one extra, drop it
            z = splitmix64(seed, cnt + 1, s)
            v = _normal(z, s)[:cnt] * sigma
        else:
            z = splitmix64(seed, cnt, s)
            if dist == "uniform":
                v = _uniform(z)
            elif dist == "int":
                v = _ints(z)
            elif dist == "normal":
                v = _normal(z, s) * sigma
            else:
                raise ValueError(f"unknown distribution {dist!r}")
        v32 = v.astype(np.float32)  # round-to-nearest-even
        if dtype == "f32":
            out[s:s + cnt] = v32
        elif dtype == "bf16":
            out[s:s + cnt] = fp32_to_bf16_bits(v32)
        else:
            out[s:s + cnt] = v32.astype(np.float16).view(np.uint16)
    return out.reshape(rows, cols)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32", "bf16" or "f16" (input precision; C is always fp32)
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    dist: str           # "uniform", "int" or "normal"
    sigma: float = 1.0
    seed_base: int = 0
    trans_a: bool = False   # A stored K x M (op(A) = A^T)
    trans_b: bool = False   # B stored N x K (op(B) = B^T)
    batch: int = 1          # independent problems, stacked on a leading axis
    bias: bool = False      # a bias row of N floats per problem
    splits: int = 1         # split-K request (1: none, 0: automatic)
    streamk: bool = False   # run through the stream-K entry point

    @property
    def a_shape(self):
        """Stored shape of A."""
        return (self.K, self.M) if self.trans_a else (self.M, self.K)

    @property
    def b_shape(self):
        """Stored shape of B."""
        return (self.N, self.K) if self.trans_b else (self.K, self.N)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    def seeds(self):
        return self.seed_base + 1, self.seed_base + 2, self.seed_base + 3

    def with_ints(self) -> "Workload":
        """The integer-valued variant of the same shape (exact in any order)."""
        return dataclasses.replace(self, name=self.name + "_int", dist="int",
                                   sigma=1.0, seed_base=self.seed_base + 10)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "f32_256": Workload("f32_256", "f32", 256, 256, 256, 1.0, 0.0, "uniform",
                        seed_base=1000),
    "f32_1000_ragged": Workload("f32_1000_ragged", "f32", 1000, 1000, 1000,
                                1.5, 0.5, "uniform", seed_base=2000),
    "f32_4096": Workload("f32_4096", "f32", 4096, 4096, 4096, 1.0, 0.0,
                         "uniform", seed_base=3000),
    "bf16_8192": Workload("bf16_8192", "bf16", 8192, 8192, 8192, 1.0, 0.0,
                          "normal", seed_base=4000),
    "f16_8192": Workload("f16_8192", "f16", 8192, 8192, 8192, 1.0, 0.0, "normal",
                         seed_base=6000),
    "bf16_skinny_8x28672x8192": Workload("bf16_skinny_8x28672x8192", "bf16",
                                         8, 28672, 8192, 1.0, 0.0, "normal",
                                         sigma=0.02, seed_base=5000),
    # The linear-layer storage (input [batch, in], weight [out, in]): the
    # forward product X W^T has B stored N x K, the weight gradient G^T X has
    # A stored K x M (elainafan.one "全连接层").
    "bf16_8192_nt": Workload("bf16_8192_nt", "bf16", 8192, 8192, 8192, 1.0, 0.0,
                             "normal", seed_base=7000, trans_b=True),
    "bf16_8192_tn": Workload("bf16_8192_tn", "bf16", 8192, 8192, 8192, 1.0, 0.0,
                             "normal", seed_base=8000, trans_a=True),
    "bf16_skinny_8x28672x8192_nt": Workload("bf16_skinny_8x28672x8192_nt", "bf16",
                                            8, 28672, 8192, 1.0, 0.0, "normal",
                                            sigma=0.02, seed_base=9000, trans_b=True),
    # The same decode product with fp32 inputs: 940 MB of weight streamed once.
    "f32_skinny_8x28672x8192_nt": Workload("f32_skinny_8x28672x8192_nt", "f32",
                                           8, 28672, 8192, 1.0, 0.0, "normal",
                                           sigma=0.02, seed_base=19000, trans_b=True),
    # The linear layer's forward with its bias fused into the epilogue, and a
    # strided batch of independent products.
    "bf16_linear_bias_8192_nt": Workload("bf16_linear_bias_8192_nt", "bf16", 8192, 8192, 8192,
                                         1.0, 0.0, "normal", seed_base=10000, trans_b=True,
                                         bias=True),
    "bf16_bmm_16x2048": Workload("bf16_bmm_16x2048", "bf16", 2048, 2048, 2048, 1.0, 0.0,
                                 "normal", seed_base=11000, batch=16),
    # A mid-size decode batch (64 rows) against the same [out, in] weight:
    # still bound by streaming the weight once (64 FLOP per byte of it).
    "bf16_decode_64x28672x8192_nt": Workload("bf16_decode_64x28672x8192_nt", "bf16", 64, 28672,
                                             8192, 1.0, 0.0, "normal", sigma=0.02,
                                             seed_base=12000, trans_b=True),
    # Too few output tiles to fill the GPU: split-K (automatic slice count).
    "f32_1000_splitk": Workload("f32_1000_splitk", "f32", 1000, 1000, 1000, 1.5, 0.5,
                                "uniform", seed_base=13000, splits=0),
    "bf16_splitk_1024x1024x16384": Workload("bf16_splitk_1024x1024x16384", "bf16", 1024, 1024,
                                            16384, 1.0, 0.0, "normal", seed_base=14000,
                                            splits=0),
    # One GPU's share when the two headline BF16 products are split by
    # columns of B / C over 8 GPUs: 8 x 8192 x 3584 (skinny, 58.7 MB of B) and
    # 8192 x 1024 x 8192.  The skinny share has too few column strips to fill
    # the GPU and runs split-K (automatic slice count); the other fills it
    # with 512 tiles of 128 x 128 and runs unsplit.
    "bf16_skinny_shard_8x3584x8192": Workload("bf16_skinny_shard_8x3584x8192", "bf16", 8, 3584,
                                              8192, 1.0, 0.0, "normal", sigma=0.02,
                                              seed_base=15000, splits=0),
    "bf16_shard_8192x1024x8192": Workload("bf16_shard_8192x1024x8192", "bf16", 8192, 1024, 8192,
                                          1.0, 0.0, "normal", seed_base=16000),
    # 384 tiles of 256 x 256 for 256 CUs (one and a half waves) with a long K:
    # stream-K deals the K iterations out evenly instead of running a second,
    # half-empty wave of tiles.
    "bf16_streamk_6144x4096x8192": Workload("bf16_streamk_6144x4096x8192", "bf16", 6144, 4096,
                                            8192, 1.0, 0.0, "normal", seed_base=17000,
                                            streamk=True),
    # FP32 3000^3: 144 tiles of 256 x 256 fill 144 of the 256 CUs and 576
    # tiles of 128 x 128 take two waves of 512 slots, the second an eighth
    # full; stream-K deals the 64-deep K iterations out evenly.
    "f32_streamk_3000": Workload("f32_streamk_3000", "f32", 3000, 3000, 3000, 1.0, 0.0,
                                 "uniform", seed_base=18000, streamk=True),
}


def _stack(seed, batch, rows, cols, dist, sigma, dtype):
    """``batch`` matrices drawn as one stream (problem z is rows z*rows ..)."""
    x = draw(seed, batch * rows, cols, dist, sigma, dtype)
    return x if batch == 1 else x.reshape(batch, rows, cols)


def make_inputs(w: Workload):
    """Return ``(A, B, C0)`` for workload ``w`` (C0 is None when beta == 0).
    A and B have their stored shapes (``w.a_shape``, ``w.b_shape``), with a
    leading batch axis when ``w.batch > 1``."""
    sa, sb, sc = w.seeds()
    A = _stack(sa, w.batch, *w.a_shape, w.dist, w.sigma, w.dtype)
    B = _stack(sb, w.batch, *w.b_shape, w.dist, w.sigma, w.dtype)
    C0 = None
    if w.beta != 0.0:
        C0 = _stack(sc, w.batch, w.M, w.N, w.dist, w.sigma, "f32")
    return A, B, C0


def make_bias(w: Workload):
    """The bias rows of workload ``w``, fp32 [batch, N] (uniform on [-1, 1)),
    or None."""
    if not w.bias:
        return None
    return draw(w.seed_base + 4, w.batch, w.N, "uniform", 1.0, "f32")


def as_fp32(x: np.ndarray, dtype: str) -> np.ndarray:
    """The fp32 values an input array denotes (16-bit bits widened exactly)."""
    if dtype == "bf16":
        return bf16_bits_to_fp32(x)
    if dtype == "f16":
        return np.asarray(x, np.uint16).view(np.float16).astype(np.float32)
    return np.asarray(x, np.float32)
