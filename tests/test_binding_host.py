"""The torch-facing calls of the binding (gemm, gemm_batched, gemm_split,
gemm_stream) reject host tensors, column-strided views and mis-shaped bias
rows before anything reaches the library.  Runs without a GPU: the library
loader is replaced by one that fails the test if it is ever reached."""

import pytest

torch = pytest.importorskip("torch")
import dense_gemm_tuning_amd as dgt  # noqa: E402


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def boom():
        raise AssertionError("a rejected call reached the library")
    monkeypatch.setattr(dgt, "_load", boom)


def test_gemm_rejects_host_tensors():
    A, B, C = torch.zeros(8, 4), torch.zeros(4, 6), torch.zeros(8, 6)
    with pytest.raises(ValueError, match="GPU tensor"):
        dgt.gemm(A, B, C)


def test_gemm_rejects_column_strided_views():
    X = torch.zeros(8, 8)
    with pytest.raises(ValueError, match="unit column stride"):
        dgt.gemm(X[:, ::2], torch.zeros(4, 6), torch.zeros(8, 6))
    with pytest.raises(ValueError, match="unit column stride"):
        dgt.gemm(torch.zeros(8, 4), torch.zeros(4, 6), torch.zeros(8, 12)[:, ::2])


def test_gemm_rejects_wrong_dimensions_and_shapes():
    with pytest.raises(ValueError, match="dimensions"):
        dgt.gemm(torch.zeros(2, 8, 4), torch.zeros(4, 6), torch.zeros(8, 6))
    with pytest.raises(ValueError, match="shape mismatch"):
        dgt.gemm(torch.zeros(8, 4), torch.zeros(5, 6), torch.zeros(8, 6))


def test_gemm_split_rejects_host_and_strided_tensors():
    A, B, C = torch.zeros(8, 4), torch.zeros(4, 6), torch.zeros(8, 6)
    with pytest.raises(ValueError, match="GPU tensor"):
        dgt.gemm_split(A, B, C, splits=2)
    with pytest.raises(ValueError, match="unit column stride"):
        dgt.gemm_split(torch.zeros(8, 8)[:, ::2], B, C, splits=2)
    with pytest.raises(ValueError, match="dimensions"):
        dgt.gemm_split(A[None], B, C, splits=2)
    ws = torch.zeros(64, dtype=torch.uint8)[::2]
    with pytest.raises(ValueError, match="contiguous"):
        dgt.gemm_split(A, B, C, splits=2, workspace=ws)


def test_gemm_stream_rejects_host_and_strided_tensors():
    A, B, C = torch.zeros(8, 4), torch.zeros(4, 6), torch.zeros(8, 6)
    with pytest.raises(ValueError, match="GPU tensor"):
        dgt.gemm_stream(A, B, C)
    with pytest.raises(ValueError, match="unit column stride"):
        dgt.gemm_stream(torch.zeros(8, 8)[:, ::2], B, C)
    with pytest.raises(ValueError, match="dimensions"):
        dgt.gemm_stream(A[None], B, C)
    with pytest.raises(ValueError, match="shape mismatch"):
        dgt.gemm_stream(A, torch.zeros(5, 6), C)
    ws = torch.zeros(64, dtype=torch.uint8)[::2]
    with pytest.raises(ValueError, match="contiguous"):
        dgt.gemm_stream(A, B, C, workspace=ws)


def test_gemm_batched_rejects_host_and_strided_tensors():
    A, B, C = torch.zeros(3, 8, 4), torch.zeros(3, 4, 6), torch.zeros(3, 8, 6)
    with pytest.raises(ValueError, match="GPU tensor"):
        dgt.gemm_batched(A, B, C)
    with pytest.raises(ValueError, match="unit column stride"):
        dgt.gemm_batched(torch.zeros(3, 8, 8)[:, :, ::2], B, C)
    with pytest.raises(ValueError, match="2-D or"):
        dgt.gemm_batched(torch.zeros(2, 8, 4), B, C)


@pytest.mark.parametrize("shape", [(2, 6), (4, 6), (7,), (3, 5), (1, 1, 6)])
def test_gemm_batched_rejects_bias_of_the_wrong_shape(shape):
    """A [b, N] bias with b other than 1 or batch would be read past its end
    (b < batch) or silently truncated; a bias of the wrong length or rank is
    refused too."""
    A, B, C = torch.zeros(3, 8, 4), torch.zeros(3, 4, 6), torch.zeros(3, 8, 6)
    with pytest.raises(ValueError, match="bias"):
        dgt.gemm_batched(A, B, C, bias=torch.zeros(*shape))


def test_gemm_batched_host_bias_is_refused():
    """Accepted bias shapes still have to live on C's GPU."""
    A, B, C = torch.zeros(3, 8, 4), torch.zeros(3, 4, 6), torch.zeros(3, 8, 6)
    for shape in [(6,), (1, 6), (3, 6)]:
        with pytest.raises(ValueError, match="GPU tensor"):
            dgt.gemm_batched(A, B, C, bias=torch.zeros(*shape))
