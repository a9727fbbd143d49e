"""bitlinear_forward_noalloc (the forward for callers that cannot allocate)
against bitlinear_forward, through the C ABI.

Two prefill calls in a row, the second on a smaller problem (so the scratch
array holds the first call's codes when the second starts), a decode call, a
call on a second stream, and an over-limit call that must fail before any
launch.  Outputs must equal bitlinear_forward's bit for bit (the same kernels
run) and the oracle's within the usual 1e-5 relative bound.
"""
import ctypes

import numpy as np
import pytest
import torch

import bitlinear_absmean_ternarise_bit_amd as bl
import oracle as O
from bitlinear_absmean_ternarise_bit_amd import abi
from bitlinear_absmean_ternarise_bit_amd.workloads import random_problem

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def dev_x(P):
    if P.x_dtype == "bf16":
        return torch.from_numpy(P.X_bf16_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(P.X).to(DEV)


def check_y(y, yr):
    y = np.asarray(y, dtype=np.float64)
    yr = np.asarray(yr, dtype=np.float64)
    assert np.all(np.abs(y - yr) <= 1e-5 * np.abs(yr))


def call_noalloc(X, packed, gamma, K, Y, stream):
    lib = abi.load()
    dt = abi.BF16 if X.dtype == torch.bfloat16 else abi.F32
    return lib.bitlinear_forward_noalloc(ctypes.c_void_p(X.data_ptr()), dt, X.shape[0], K,
                                         ctypes.c_void_p(packed.data_ptr()), packed.shape[0],
                                         ctypes.c_void_p(gamma.data_ptr()), ctypes.c_void_p(Y.data_ptr()),
                                         ctypes.c_void_p(stream))


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_forward(order):
    stream = torch.cuda.current_stream(DEV).cuda_stream
    # prefill, then a smaller prefill (stale codes of the first call in the
    # scratch array), then a decode-path call
    for M, K, N, dt in [(3000, 2000, 1500, "bf16"), (300, 520, 600, "f32"), (5, 700, 90, "bf16")]:
        say(f"noalloc M={M} K={K} N={N} {dt}")
        P = random_problem(M, K, N, seed=M + K + N, x_dtype=dt)
        packed, gamma = bl.quantize_weights(torch.from_numpy(P.W).to(DEV))
        X = dev_x(P)
        Y_ref = bl.forward(X, packed, gamma, K)
        Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        assert call_noalloc(X, packed, gamma, K, Y, stream) == abi.OK
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_ref)
        check_y(Y.cpu().numpy(), O.bitlinear_forward(P.X, P.W)["Y"])


def test_noalloc_on_another_stream_and_over_limit():
    P = random_problem(700, 1000, 333, seed=9, x_dtype="bf16")
    packed, gamma = bl.quantize_weights(torch.from_numpy(P.W).to(DEV))
    X = dev_x(P)
    Y_ref = bl.forward(X, packed, gamma, P.K)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(DEV)
    Y = torch.zeros((P.M, P.N), dtype=torch.float32, device=DEV)
    with torch.cuda.stream(s):
        assert call_noalloc(X, packed, gamma, P.K, Y, s.cuda_stream) == abi.OK
    s.synchronize()
    assert torch.equal(Y, Y_ref)
    # 16384 tokens of K = 8192 need 128 MiB of codes: refused, nothing launched
    Xbig = torch.empty((16384, 8192), dtype=torch.bfloat16, device=DEV)
    pk = torch.empty((64, bl.packed_words(8192)), dtype=torch.int32, device=DEV)
    Ybig = torch.empty((16384, 64), dtype=torch.float32, device=DEV)
    assert call_noalloc(Xbig, pk, gamma, 8192, Ybig, torch.cuda.current_stream(DEV).cuda_stream) == abi.ERR_WORKSPACE
