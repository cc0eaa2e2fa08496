"""C-ABI library on the host: it loads, exports every declared symbol, and its
argument checks behave as the header states.  No call here reaches a kernel
launch (every one fails validation or is an empty quick return), so these
run without a GPU."""

import ctypes
import os
import re

import pytest

import dense_gemm_tuning_amd as dgt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dgt_gemm.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dgt.LIB_PATH):
        from dense_gemm_tuning_amd import build
        build.build()
    return dgt.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(dgt.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported by {dgt.LIB_PATH}"


def test_abi_version_and_status_strings(lib):
    assert dgt.gemm_abi_version() == 9
    for code in range(0, -10, -1):
        s = dgt.gemm_status_string(code)
        assert s.startswith("GEMM_")
    assert dgt.gemm_status_string(12345) == "unknown gemm status"


# fake, non-overlapping host addresses: never dereferenced on error paths
A_, B_, C_ = 0x100000, 0x200000, 0x300000


@pytest.mark.parametrize("fn", ["gemm_f32", "gemm_bf16", "gemm_f16"])
def test_argument_errors(lib, fn):
    f = getattr(dgt, fn)
    assert f(-1, 4, 4, 1.0, A_, 4, B_, 4, 0.0, C_, 4) == dgt.GEMM_ERR_DIM
    assert f(4, -1, 4, 1.0, A_, 4, B_, 4, 0.0, C_, 4) == dgt.GEMM_ERR_DIM
    assert f(4, 4, -1, 1.0, A_, 4, B_, 4, 0.0, C_, 4) == dgt.GEMM_ERR_DIM
    assert f(4, 4, 8, 1.0, A_, 7, B_, 4, 0.0, C_, 4) == dgt.GEMM_ERR_LD
    assert f(4, 6, 4, 1.0, A_, 4, B_, 5, 0.0, C_, 6) == dgt.GEMM_ERR_LD
    assert f(4, 6, 4, 1.0, A_, 4, B_, 6, 0.0, C_, 5) == dgt.GEMM_ERR_LD
    assert f(4, 4, 0, 1.0, A_, 0, B_, 4, 0.0, C_, 4) == dgt.GEMM_ERR_LD  # lda >= 1
    assert f(4, 4, 4, 1.0, A_, 4, B_, 4, 0.0, 0, 4) == dgt.GEMM_ERR_NULL
    assert f(4, 4, 4, 1.0, 0, 4, B_, 4, 0.0, C_, 4) == dgt.GEMM_ERR_NULL
    assert f(4, 4, 4, 1.0, A_, 4, 0, 4, 0.0, C_, 4) == dgt.GEMM_ERR_NULL
    # C overlapping A or B
    assert f(4, 4, 4, 1.0, A_, 4, B_, 4, 0.0, A_ + 8, 4) == dgt.GEMM_ERR_OVERLAP
    assert f(4, 4, 4, 1.0, A_, 4, B_, 4, 0.0, B_ - 16, 4) == dgt.GEMM_ERR_OVERLAP


@pytest.mark.parametrize("fn", ["gemm_f32", "gemm_bf16", "gemm_f16"])
def test_empty_c_is_a_no_op(lib, fn):
    f = getattr(dgt, fn)
    # quick return before any pointer check or launch
    assert f(0, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4) == dgt.GEMM_OK
    assert f(4, 0, 4, 1.0, 0, 4, 0, 1, 0.0, 0, 1) == dgt.GEMM_OK


def test_variant_checks(lib):
    v = dgt.gemm_f32_variant
    assert v(99, 4, 4, 4, 1.0, A_, 4, B_, 4, 0.0, C_, 4) == dgt.GEMM_ERR_VARIANT
    assert v(-1, 4, 4, 4, 1.0, A_, 4, B_, 4, 0.0, C_, 4) == dgt.GEMM_ERR_VARIANT
    # the skinny rung takes at most 64 rows
    assert v(dgt.VARIANT_SKINNY, 65, 4, 4, 1.0, A_, 4, B_, 4, 0.0, C_, 4) == dgt.GEMM_ERR_VARIANT
    for fn in (dgt.gemm_bf16_variant, dgt.gemm_f16_variant):
        assert fn(dgt.VARIANT_SKINNY, 65, 4, 4, 1.0, A_, 4, B_, 4, 0.0,
                  C_, 4) == dgt.GEMM_ERR_VARIANT
        assert fn(99, 4, 4, 4, 1.0, A_, 4, B_, 4, 0.0, C_, 4) == dgt.GEMM_ERR_VARIANT
    assert v(dgt.VARIANT_MFMA_REGS + 1, 4, 4, 4, 1.0, A_, 4, B_, 4, 0.0, C_, 4) == \
        dgt.GEMM_ERR_VARIANT


def test_fixed_tile_rungs_need_aligned_rows(lib):
    """The fixed-tile MFMA rungs run only the DMA kernels: rows that are not
    16-byte aligned (pitch or base) are refused on the host, before any HIP
    call; alpha == 0 reads neither operand and is not refused (NULL C stops
    that call before its launch)."""
    M = N = K = 64
    for rung in (dgt.VARIANT_MFMA_T256, dgt.VARIANT_MFMA_T128):
        # fp32: a pitch of 66 floats is 264 bytes, not a multiple of 16
        assert dgt.gemm_f32_variant(rung, M, N, K, 1.0, A_, 66, B_, N, 0.0, C_, N) == \
            dgt.GEMM_ERR_VARIANT
        assert dgt.gemm_f32_variant(rung, M, N, K, 1.0, A_ + 4, K, B_, N, 0.0, C_, N) == \
            dgt.GEMM_ERR_VARIANT
        # 16-bit: a pitch of 68 elements is 136 bytes
        for fn in (dgt.gemm_bf16_variant, dgt.gemm_f16_variant):
            assert fn(rung, M, N, K, 1.0, A_, K, B_, 68, 0.0, C_, N) == dgt.GEMM_ERR_VARIANT
            assert fn(rung, M, N, K, 1.0, A_, K, B_ + 2, N, 0.0, C_, N) == dgt.GEMM_ERR_VARIANT
        assert dgt.gemm_f32_variant(rung, M, N, K, 0.0, A_, 66, B_, N, 0.0, 0, N) == \
            dgt.GEMM_ERR_NULL


def test_alpha_zero_does_not_need_a_or_b(lib):
    # alpha == 0: A and B are not read, so NULL A/B is legal; the call then
    # reaches the launch of the scaling kernel -- only its argument checks are
    # exercised here, with a NULL C to stop it before any HIP call
    assert dgt.gemm_f32(4, 4, 4, 0.0, 0, 4, 0, 4, 1.0, 0, 4) == dgt.GEMM_ERR_NULL


def test_auto_dispatch(lib):
    sel = dgt.gemm_select_variant
    F32, BF16, F16 = dgt.DTYPE_F32, dgt.DTYPE_BF16, dgt.DTYPE_F16
    assert sel(BF16, 0, 0, 8, 28672, 8192, 8192, 28672, 28672) == dgt.VARIANT_SKINNY
    assert sel(BF16, 0, 1, 8, 28672, 8192, 8192, 8192, 28672) == dgt.VARIANT_SKINNY
    assert sel(F16, 0, 0, 8, 28672, 8192, 8192, 28672, 28672) == dgt.VARIANT_SKINNY
    assert sel(BF16, 0, 0, 16, 100, 100, 100, 100, 100) == dgt.VARIANT_SKINNY
    assert sel(BF16, 0, 0, 64, 100, 100, 100, 100, 100) == dgt.VARIANT_SKINNY
    assert sel(BF16, 0, 0, 65, 100, 100, 100, 100, 100) == dgt.VARIANT_MFMA
    assert sel(F16, 1, 1, 8192, 8192, 8192, 8192, 8192, 8192) == dgt.VARIANT_MFMA
    assert sel(F32, 0, 0, 4096, 4096, 4096, 4096, 4096, 4096) == dgt.VARIANT_MFMA
    assert sel(F32, 0, 0, 4, 4, 4, 3, 4, 4) == dgt.GEMM_ERR_LD
    assert sel(F32, 0, 0, -4, 4, 4, 4, 4, 4) == dgt.GEMM_ERR_DIM
    assert sel(3, 0, 0, 4, 4, 4, 4, 4, 4) == dgt.GEMM_ERR_ARG
    assert sel(-1, 0, 0, 4, 4, 4, 4, 4, 4) == dgt.GEMM_ERR_ARG
    assert sel(F32, 2, 0, 4, 4, 4, 4, 4, 4) == dgt.GEMM_ERR_ARG
    assert sel(F32, 0, -1, 4, 4, 4, 4, 4, 4) == dgt.GEMM_ERR_ARG


@pytest.mark.parametrize("dtype", [0, 1, 2])
def test_transposed_leading_dimensions(lib, dtype):
    """Stored shapes: A is K x M when trans_a (lda >= M), B is N x K when
    trans_b (ldb >= K); C is always M x N."""
    ex = dgt.gemm_ex
    M, N, K = 6, 10, 4
    for ta, tb in [(0, 0), (0, 1), (1, 0), (1, 1)]:
        lda = M if ta else K
        ldb = K if tb else N
        assert ex(dtype, ta, tb, 0, M, N, K, 1.0, A_, lda - 1, B_, ldb, 0.0, C_, N) == \
            dgt.GEMM_ERR_LD, (ta, tb)
        assert ex(dtype, ta, tb, 0, M, N, K, 1.0, A_, lda, B_, ldb - 1, 0.0, C_, N) == \
            dgt.GEMM_ERR_LD, (ta, tb)
        assert ex(dtype, ta, tb, 0, M, N, K, 1.0, A_, lda, B_, ldb, 0.0, C_, N - 1) == \
            dgt.GEMM_ERR_LD, (ta, tb)
        # legal pitches reach the pointer checks (NULL C stops before a launch)
        assert ex(dtype, ta, tb, 0, M, N, K, 1.0, A_, lda, B_, ldb, 0.0, 0, N) == \
            dgt.GEMM_ERR_NULL, (ta, tb)
    # bad flags and dtype are rejected first
    assert ex(dtype, 2, 0, 0, M, N, K, 1.0, A_, K, B_, N, 0.0, C_, N) == dgt.GEMM_ERR_ARG
    assert ex(dtype, 0, 3, 0, -1, N, K, 1.0, A_, K, B_, N, 0.0, C_, N) == dgt.GEMM_ERR_ARG
    assert ex(7, 0, 0, 0, M, N, K, 1.0, A_, K, B_, N, 0.0, C_, N) == dgt.GEMM_ERR_ARG
    assert ex(dtype, 0, 0, 9, M, N, K, 1.0, A_, K, B_, N, 0.0, C_, N) == dgt.GEMM_ERR_VARIANT
    assert ex(dtype, 1, 1, dgt.VARIANT_SKINNY, 65, N, K, 1.0, A_, 65, B_, K, 0.0, C_, N) == \
        dgt.GEMM_ERR_VARIANT


def test_transposed_overlap_uses_stored_extent(lib):
    """A stored K x M spans (K-1)*lda + M elements, not (M-1)*lda + K."""
    ex = dgt.gemm_ex
    M, N, K = 2, 4, 64           # A^T stored 64 x 2 with lda 2: 128 floats = 512 B
    a = 0x100000
    c_inside = a + 4 * 100       # inside the stored K x M extent, outside an M x K one
    assert ex(0, 1, 0, 0, M, N, K, 1.0, a, M, B_, N, 0.0, c_inside, N) == dgt.GEMM_ERR_OVERLAP
    b = 0x200000                 # B^T stored 4 x 64 (ldb 64): 256 floats
    c_in_b = b + 4 * 200
    assert ex(0, 0, 1, 0, M, N, K, 1.0, A_, K, b, K, 0.0, c_in_b, N) == dgt.GEMM_ERR_OVERLAP


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(dgt, "_lib", None)
    monkeypatch.setattr(dgt, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        dgt.gemm_abi_version()


def test_strided_batched_argument_checks(lib):
    sb = dgt.gemm_strided_batched
    M, N, K = 4, 8, 16
    # (dtype, ta, tb, variant, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C, ldc, sc,
    #  bias, sbias, batch)
    base = dict(dtype=0, ta=0, tb=0, variant=0, M=M, N=N, K=K, alpha=1.0, A=A_, lda=K, sa=M * K,
                B=B_, ldb=N, sb=K * N, beta=0.0, C=C_, ldc=N, sc=M * N, bias=0, sbias=0, batch=3)

    def call(**kw):
        a = dict(base, **kw)
        return sb(a["dtype"], a["ta"], a["tb"], a["variant"], a["M"], a["N"], a["K"], a["alpha"],
                  a["A"], a["lda"], a["sa"], a["B"], a["ldb"], a["sb"], a["beta"], a["C"],
                  a["ldc"], a["sc"], a["bias"], a["sbias"], a["batch"])

    # valid arguments reach the pointer checks (NULL C stops before a launch)
    assert call(C=0) == dgt.GEMM_ERR_NULL
    assert call(batch=-1) == dgt.GEMM_ERR_ARG
    assert call(sa=-1) == dgt.GEMM_ERR_ARG
    assert call(sc=1 << 48) == dgt.GEMM_ERR_ARG
    assert call(sbias=-4) == dgt.GEMM_ERR_ARG
    assert call(dtype=5) == dgt.GEMM_ERR_ARG
    assert call(tb=2) == dgt.GEMM_ERR_ARG
    assert call(lda=K - 1) == dgt.GEMM_ERR_LD
    assert call(variant=dgt.VARIANT_MFMA_REGS + 1) == dgt.GEMM_ERR_VARIANT
    # empty batch or empty C: nothing to do, no pointer needed
    assert call(batch=0, A=0, B=0, C=0) == dgt.GEMM_OK
    assert call(M=0, A=0, B=0, C=0) == dgt.GEMM_OK
    # problems of one batch writing the same C elements
    assert call(sc=M * N - 1) == dgt.GEMM_ERR_OVERLAP
    assert call(sc=0) == dgt.GEMM_ERR_OVERLAP
    assert call(sc=0, batch=1, C=0) == dgt.GEMM_ERR_NULL   # one problem: stride unused
    # C reaching into the last A of the batch (A spans 3 problems of M*K floats)
    assert call(C=A_ + 4 * (2 * M * K + 5)) == dgt.GEMM_ERR_OVERLAP
    # C overlapping the bias of a later problem
    bias = 0x400000
    assert call(bias=bias, sbias=N, C=bias + 4 * (2 * N + 1)) == dgt.GEMM_ERR_OVERLAP
    # A and B may overlap each other and repeat: only C's writes matter
    assert call(B=A_, sb=0, C=0) == dgt.GEMM_ERR_NULL
    # skinny rung still limited to M <= 64
    assert call(variant=dgt.VARIANT_SKINNY, M=65, sc=65 * N) == dgt.GEMM_ERR_VARIANT


def test_splitk_planning(lib):
    sl, ws = dgt.gemm_splitk_slices, dgt.gemm_splitk_workspace_size
    F32, BF16 = dgt.DTYPE_F32, dgt.DTYPE_BF16
    # 1000^3 fp32: 64 tiles of 128 x 128 for 256 workgroup slots (one per CU)
    # -> 4 slices of 256 (the last 232 deep)
    assert sl(F32, 1000, 1000, 1000, 0) == 4
    assert ws(F32, 1000, 1000, 1000, 0) == 4 * 1000 * 1000 * 4
    # 512 x 512 fp32 with K = 8192: 16 tiles -> 16 slices of 512
    assert sl(F32, 512, 512, 8192, 0) == 16
    # 1024 x 1024 bf16 with K = 16384: 64 tiles of 128 x 128 for 512 slots
    # (two per CU) -> 8 slices
    assert sl(BF16, 1024, 1024, 16384, 0) == 8
    # 8192 x 1024 bf16: 512 tiles of 128 x 128 fill the slots unsplit
    assert sl(BF16, 8192, 1024, 8192, 0) == 1
    # enough tiles already, or K too short to split: one slice, no workspace
    assert sl(BF16, 8192, 8192, 8192, 0) == 1 and ws(BF16, 8192, 8192, 8192, 0) == 0
    assert sl(F32, 1000, 1000, 128, 0) == 1       # one 128-deep slice covers K
    # requests: slice length rounds up to a multiple of 128
    assert sl(F32, 100, 100, 1000, 3) == 3       # 3 x 384 >= 1000
    assert sl(F32, 100, 100, 1000, 7) == 4       # ceil(1000/7) = 143 rounds up to 256: 4 slices
    assert sl(F32, 100, 100, 300, 5) == 3        # 128-deep slices: 128, 128, 44
    assert sl(F32, 100, 100, 1000, 1) == 1
    assert 32 < sl(F32, 100, 100, 100000, 1000) <= 64  # capped at 64 (rounding: 61)
    assert sl(F32, 100, 100, 1000, -1) == dgt.GEMM_ERR_ARG
    assert sl(9, 100, 100, 1000, 0) == dgt.GEMM_ERR_ARG
    assert sl(F32, -1, 100, 1000, 0) == dgt.GEMM_ERR_DIM


def test_splitk_argument_checks(lib):
    f = dgt.gemm_splitk
    M, N, K = 64, 64, 4096
    need = dgt.gemm_splitk_workspace_size(0, M, N, K, 4)
    assert need == 4 * M * N * 4
    W = 0x800000
    args = lambda **kw: dict(dict(dtype=0, ta=0, tb=0, M=M, N=N, K=K, alpha=1.0, A=A_, lda=K,
                                  B=B_, ldb=N, beta=0.0, C=C_, ldc=N, splits=4, ws=W,
                                  wsb=need), **kw)

    def call(**kw):
        a = args(**kw)
        return f(a["dtype"], a["ta"], a["tb"], a["M"], a["N"], a["K"], a["alpha"], a["A"],
                 a["lda"], a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], a["splits"], a["ws"],
                 a["wsb"])

    assert call(splits=-1) == dgt.GEMM_ERR_ARG
    assert call(wsb=-1) == dgt.GEMM_ERR_ARG
    assert call(dtype=3) == dgt.GEMM_ERR_ARG
    assert call(lda=K - 1) == dgt.GEMM_ERR_LD
    assert call(ws=0) == dgt.GEMM_ERR_WORKSPACE
    assert call(wsb=need - 4) == dgt.GEMM_ERR_WORKSPACE
    assert call(C=0) == dgt.GEMM_ERR_NULL
    assert call(ws=C_ + 64) == dgt.GEMM_ERR_OVERLAP           # workspace overlaps C
    assert call(ws=A_ - 64) == dgt.GEMM_ERR_OVERLAP           # ... or A
    # one slice is plain gemm_ex: no workspace needed (stops at the NULL C)
    assert call(splits=1, ws=0, wsb=0, C=0) == dgt.GEMM_ERR_NULL
    # empty C: nothing to do
    assert call(M=0, A=0, B=0, C=0, ws=0) == dgt.GEMM_OK


def test_splitk_noalloc_argument_checks(lib):
    """gemm_splitk_noalloc refuses a shape whose partials exceed the fixed
    scratch, and every other argument error as gemm_splitk does, on the host
    before any HIP call (fake pointers: nothing here reaches a launch)."""
    f = dgt.gemm_splitk_noalloc

    def call(dtype=0, ta=0, tb=0, M=64, N=64, K=4096, A=A_, lda=4096, B=B_, ldb=64, C=C_,
             ldc=64, splits=4):
        return f(dtype, ta, tb, M, N, K, 1.0, A, lda, B, ldb, 0.0, C, ldc, splits)

    # 8 slices of 2048 x 2048 fp32 partials = 128 MiB > the 64 MiB scratch
    assert dgt.gemm_splitk_workspace_size(0, 2048, 2048, 16384, 8) > dgt.NOALLOC_SCRATCH_BYTES
    assert call(M=2048, N=2048, K=16384, lda=16384, ldb=2048, ldc=2048, splits=8) == \
        dgt.GEMM_ERR_SCRATCH
    assert call(splits=-1) == dgt.GEMM_ERR_ARG
    assert call(dtype=3) == dgt.GEMM_ERR_ARG
    assert call(ta=2) == dgt.GEMM_ERR_ARG
    assert call(lda=100) == dgt.GEMM_ERR_LD
    assert call(M=-1) == dgt.GEMM_ERR_DIM
    assert call(C=0) == dgt.GEMM_ERR_NULL
    assert call(A=0) == dgt.GEMM_ERR_NULL
    # one slice is plain gemm_ex (stops at the NULL C); an empty C does nothing
    assert call(splits=1, C=0) == dgt.GEMM_ERR_NULL
    assert call(M=0, A=0, B=0, C=0) == dgt.GEMM_OK
    assert dgt.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert "GEMM_ERR_SCRATCH" in dgt.gemm_status_string(dgt.GEMM_ERR_SCRATCH)


def test_streamk_argument_checks(lib):
    """gemm_streamk's host checks (fake pointers: every call here fails
    validation or needs no launch)."""
    f = dgt.gemm_streamk
    M, N, K = 1024, 1024, 1024
    need = dgt.gemm_streamk_workspace_size(1, M, N, K)
    # 16 tiles x 8 iterations of 128 k: 128 workgroups x two 256 x 256 fp32 tiles
    assert need == 2 * 128 * 256 * 256 * 4
    # 4 tiles x 2 iterations: 8 workgroups; 32 x 32 tiles x 64: 256 (the CUs)
    assert dgt.gemm_streamk_workspace_size(1, 512, 512, 256) == 2 * 8 * 256 * 256 * 4
    assert dgt.gemm_streamk_workspace_size(1, 8192, 8192, 8192) == 2 * 256 * 256 * 256 * 4
    # FP32: iterations of 64 k (16 tiles x 16 = 256 workgroups); 4 tiles x 4
    assert dgt.gemm_streamk_workspace_size(0, M, N, K) == 2 * 256 * 256 * 256 * 4
    assert dgt.gemm_streamk_workspace_size(0, 512, 512, 256) == 2 * 16 * 256 * 256 * 4
    assert dgt.gemm_streamk_workspace_size(0, 64, N, K) == 0     # skinny
    assert dgt.gemm_streamk_workspace_size(1, 64, N, K) == 0     # skinny
    assert dgt.gemm_streamk_workspace_size(1, M, N, 0) == 0
    assert dgt.gemm_streamk_workspace_size(3, M, N, K) == dgt.GEMM_ERR_ARG
    assert dgt.gemm_streamk_workspace_size(1, -1, N, K) == dgt.GEMM_ERR_DIM
    # disjoint fake ranges: A and B 2 MiB each, C 4 MiB, the workspace 128 MiB
    A, B, C, W = 0x1000000, 0x2000000, 0x3000000, 0x10000000

    def call(dtype=1, ta=0, tb=0, M=M, N=N, K=K, A=A, lda=K, B=B, ldb=N, C=C, ldc=N, ws=W,
             wsb=need):
        return f(dtype, ta, tb, M, N, K, 1.0, A, lda, B, ldb, 0.0, C, ldc, ws, wsb)

    assert call(dtype=3) == dgt.GEMM_ERR_ARG
    assert call(wsb=-1) == dgt.GEMM_ERR_ARG
    assert call(tb=2) == dgt.GEMM_ERR_ARG
    assert call(lda=K - 1) == dgt.GEMM_ERR_LD
    assert call(M=-1) == dgt.GEMM_ERR_DIM
    assert call(C=0) == dgt.GEMM_ERR_NULL
    assert call(ws=0) == dgt.GEMM_ERR_WORKSPACE
    assert call(wsb=need - 16) == dgt.GEMM_ERR_WORKSPACE
    assert call(ws=W + 8) == dgt.GEMM_ERR_WORKSPACE           # not 16-byte aligned
    assert call(ws=C + 64) == dgt.GEMM_ERR_OVERLAP            # workspace overlaps C
    assert call(ws=B - 1024) == dgt.GEMM_ERR_OVERLAP          # ... or B
    assert call(C=A + 64) == dgt.GEMM_ERR_OVERLAP             # C overlaps A
    assert call(M=0, A=0, B=0, C=0) == dgt.GEMM_OK            # empty C: nothing to do
    # FP32 takes stream-K too (4-byte elements: A and B 4 MiB each, the
    # workspace 128 MiB), so it needs the workspace
    need32 = dgt.gemm_streamk_workspace_size(0, M, N, K)
    assert call(dtype=0, ws=0, wsb=need32) == dgt.GEMM_ERR_WORKSPACE
    assert call(dtype=0, wsb=need32 - 16) == dgt.GEMM_ERR_WORKSPACE
    assert call(dtype=0, wsb=need32, ws=C + 64) == dgt.GEMM_ERR_OVERLAP
