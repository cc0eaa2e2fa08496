"""Marshalling helpers shared by the GPU parity tests: numpy <-> torch device
tensors and one library call.  No arithmetic of the method lives here."""

import sys

import numpy as np

import gemm_inputs as gi

TORCH_DTYPE = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    """numpy (fp32, or bf16/f16 bits) -> torch device tensor of the library's type."""
    import torch
    if dtype in ("bf16", "f16"):
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
        return t.view(getattr(torch, TORCH_DTYPE[dtype]))
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def bits16(x, dtype):
    """fp32 values that are exact in the 16-bit format -> its raw bits."""
    x = np.ascontiguousarray(x, np.float32)
    if dtype == "bf16":
        return gi.fp32_to_bf16_bits(x)
    return x.astype(np.float16).view(np.uint16)


def as_input(x, dtype):
    """fp32 values exact in `dtype` -> the array the library takes."""
    return np.ascontiguousarray(x, np.float32) if dtype == "f32" else bits16(x, dtype)


def run_gemm(variant, dtype, A, B, C0, alpha, beta, stream=None, trans_a=False,
             trans_b=False):
    """Copy stored operands to the GPU, run one call, return (status, C as numpy).
    A is K x M when trans_a, B is N x K when trans_b; C0 None -> C starts NaN."""
    import torch

    import dense_gemm_tuning_amd as dgt
    M = A.shape[1] if trans_a else A.shape[0]
    N = B.shape[0] if trans_b else B.shape[1]
    dA, dB = to_dev(A, dtype), to_dev(B, dtype)
    dC = (torch.from_numpy(np.ascontiguousarray(C0, np.float32)).cuda() if C0 is not None
          else torch.full((M, N), float("nan"), device="cuda"))
    st = dgt.gemm(dA, dB, dC, alpha, beta, variant=variant, stream=stream,
                  trans_a=trans_a, trans_b=trans_b)
    torch.cuda.synchronize()
    return st, dC.cpu().numpy()
