"""The seeded generator: published SplitMix64 values, ranges, rounding."""

import numpy as np
import pytest

import gemm_inputs as gi


def test_splitmix64_published_sequence():
    # First outputs of SplitMix64 started from state 0 (Vigna's reference
    # implementation, splitmix64.c): the stream element i uses the state
    # after i+1 increments of the golden-ratio constant.
    z = gi.splitmix64(0, 3)
    assert [int(v) for v in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                   0x06C45D188009454F]


def test_slices_regenerate_independently():
    full = gi.splitmix64(1234, 1000)
    part = gi.splitmix64(1234, 100, start=500)
    assert np.array_equal(full[500:600], part)


@pytest.mark.parametrize("dist", ["uniform", "int", "normal"])
def test_deterministic_and_chunk_invariant(dist, monkeypatch):
    a = gi.draw(77, 37, 53, dist, dtype="f32")
    monkeypatch.setattr(gi, "_CHUNK", 64)  # force many chunks (incl. odd tail)
    b = gi.draw(77, 37, 53, dist, dtype="f32")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_uniform_range_and_grid():
    x = gi.draw(5, 200, 300, "uniform").astype(np.float64)
    assert x.min() >= -1.0 and x.max() < 1.0
    # every value is a multiple of 2**-23 (exact in fp32)
    assert np.all(np.floor(x * 2**23) == x * 2**23)
    assert abs(x.mean()) < 0.02


def test_int_values():
    x = gi.draw(6, 100, 100, "int")
    assert set(np.unique(x).tolist()) <= {-3.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0}
    assert len(np.unique(x)) == 7


def test_normal_moments():
    x = gi.draw(7, 400, 500, "normal", sigma=0.02).astype(np.float64)
    assert abs(x.mean()) < 0.02 * 0.02
    assert abs(x.std() / 0.02 - 1.0) < 0.01


def test_bf16_rounding_nearest_even():
    # bf16 keeps the upper 16 bits of fp32 (8-bit exponent, 7-bit stored
    # mantissa: dilfish.github.io section 5.5 table, BF16 row).
    vals = np.array([
        1.0,                       # exact: 0x3F80
        1.0 + 2**-8,               # half-way between 1 and 1+2^-7: ties to even -> 1.0
        1.0 + 3 * 2**-8,           # half-way, odd neighbour below: -> 1 + 2^-6
        1.0 + 2**-8 + 2**-20,      # just above half-way -> 1 + 2^-7
        -2.0,                      # 0xC000
        1.5,                       # 0x3FC0
    ], dtype=np.float32)
    bits = gi.fp32_to_bf16_bits(vals)
    assert [int(b) for b in bits] == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC000, 0x3FC0]
    back = gi.bf16_bits_to_fp32(bits)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2**-6, 1.0 + 2**-7, -2.0, 1.5]


def test_bf16_draw_is_representable():
    x = gi.draw(8, 64, 64, "normal", dtype="bf16")
    assert x.dtype == np.uint16
    v = gi.bf16_bits_to_fp32(x)
    # re-rounding an exact bf16 value is the identity
    assert np.array_equal(gi.fp32_to_bf16_bits(v), x)
    assert np.all(np.isfinite(v))


def test_workload_table():
    w = gi.WORKLOADS
    assert (w["f32_4096"].M, w["f32_4096"].N, w["f32_4096"].K) == (4096,) * 3
    s = w["bf16_skinny_8x28672x8192"]
    assert (s.M, s.N, s.K, s.dtype, s.sigma) == (8, 28672, 8192, "bf16", 0.02)
    r = w["f32_1000_ragged"]
    assert (r.alpha, r.beta) == (1.5, 0.5)
    assert r.with_ints().dist == "int" and r.with_ints().seed_base != r.seed_base
    A, B, C0 = gi.make_inputs(w["f32_256"])
    assert A.shape == (256, 256) and C0 is None


def test_f16_draw_rounding():
    # binary16 keeps 10 fraction bits (dilfish.github.io 5.5 table, FP16 row);
    # the generator rounds fp32 -> binary16 to nearest even
    x = gi.draw(9, 64, 64, "normal", dtype="f16")
    assert x.dtype == np.uint16
    v = gi.as_fp32(x, "f16")
    assert np.all(np.isfinite(v))
    assert np.array_equal(v.astype(np.float16).view(np.uint16), x)
    ref = gi.draw(9, 64, 64, "normal", dtype="f32")
    assert np.all(np.abs(v - ref) <= np.abs(ref) * 2.0**-11 + 2.0**-25)


def test_transposed_workloads_store_operands_transposed():
    w = gi.WORKLOADS["bf16_8192_nt"]
    assert (w.trans_a, w.trans_b) == (False, True)
    assert w.a_shape == (8192, 8192) and w.b_shape == (8192, 8192)
    s = gi.WORKLOADS["bf16_skinny_8x28672x8192_nt"]
    assert s.a_shape == (8, 8192) and s.b_shape == (28672, 8192)
    small = s.scaled(N=300, K=200)
    A, B, C0 = gi.make_inputs(small)
    assert A.shape == (8, 200) and B.shape == (300, 200)
    t = gi.WORKLOADS["bf16_8192_tn"].scaled(M=40, N=30, K=20)
    A, B, _ = gi.make_inputs(t)
    assert A.shape == (20, 40) and B.shape == (20, 30)
