"""Pins for the oracle's STE backward (dX = dY W_hat, dW = (dY^T A_hat) * range mask).

[PMV] = the produtoramaxvision.com.br article on BitNet b1.58: its STE passage
takes the quantiser's gradient as the identity inside the valid range.  [MBC]
= the shadowgraph.io multimodal bitnet.cpp page: BitLinear trains with a
straight-through estimator.  The oracle's closed-form gradients are pinned
against torch autograd (float64, CPU) run on the straight-through construction
(clamp for the range, detach for the quantisation), against loops on tiny
inputs, and by boundary and rounding cases.  CPU only.
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle.bitlinear_oracle import _to_bf16_values
from bitlinear_absmean_ternarise_bit_amd.workloads import f32_to_bf16_bits, bf16_bits_to_f32, random_problem


def bf16(x):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, np.float32)))


def test_bf16_rounding_ties_to_even():
    one = np.float32(1.0)
    x = np.array([one + np.float32(2.0 ** -8), one + np.float32(3 * 2.0 ** -8), -(one + np.float32(2.0 ** -8)),
                  np.float32(1.0 + 2.0 ** -9)], np.float32)
    got = _to_bf16_values(x)
    assert got.tolist() == [1.0, 1.015625, -1.0, 1.0]
    # agrees with the input generator's own bfloat16 cast on random values
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 37
    assert np.array_equal(_to_bf16_values(r), bf16(r))


def test_dequantised_activations():
    P = random_problem(6, 300, 1, seed=1, x_scale=3.0)
    gA, Xq, _ = O.absmax_quantize(P.X)
    A = O.dequant_activations_bf16(Xq, gA)
    assert not np.any(A.view(np.uint32) & 0xFFFF)  # bfloat16 values
    exact = gA.astype(np.float64)[:, None] / 127.0 * Xq
    assert np.all(np.abs(A - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-30)


def test_weight_mask_boundary():
    g = np.float32(0.02)
    d = np.float32(g + O.EPS32)
    inside = d                                   # W / d == 1 exactly
    outside = np.nextafter(d, np.float32(1.0))  # just beyond
    W = np.array([[inside, -inside, outside, -outside, 0.0]], np.float32)
    assert (W / d)[0, 0] == 1.0
    assert O.ste_weight_mask(W, g).tolist() == [[True, True, False, False, True]]


@pytest.mark.parametrize("M,K,N", [(3, 20, 7), (17, 130, 45), (8, 256, 96)])
def test_against_torch_autograd(M, K, N):
    rng = np.random.default_rng(M * K + N)
    P = random_problem(M, K, N, seed=M + K + N)
    # a few weights pushed outside the clip range so the mask matters
    W = P.W.copy()
    W[rng.random(W.shape) < 0.1] *= 4.0
    g, q, _ = O.quantize_weights(W)
    gA, Xq, _ = O.absmax_quantize(P.X)
    dY = bf16(rng.standard_normal((M, N)))
    ref = O.ste_backward(dY, q, g, Xq, gA, W)
    assert 0 < ref["mask"].mean() < 1

    d = float(np.float32(g) + O.EPS32)
    w = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    x = torch.tensor(P.X, dtype=torch.float64, requires_grad=True)
    w_c = torch.clamp(w, -d, d)                                  # gradient 1 inside the range, 0 outside
    w_hat = w_c + (torch.tensor(q * float(np.float32(g)), dtype=torch.float64) - w_c).detach()
    x_hat = x + (torch.tensor(ref["A_hat"], dtype=torch.float64) - x).detach()
    y = x_hat @ w_hat.T
    y.backward(torch.tensor(dY, dtype=torch.float64))
    # the float32 rounding of the oracle's outputs is the only difference
    assert np.allclose(ref["dX"], x.grad.numpy(), rtol=2 ** -23, atol=0)
    assert np.allclose(ref["dW"], w.grad.numpy(), rtol=2 ** -23, atol=0)


def test_loops_on_a_tiny_problem():
    rng = np.random.default_rng(4)
    M, K, N = 2, 5, 3
    W = (0.05 * rng.standard_normal((N, K))).astype(np.float32)
    X = rng.standard_normal((M, K)).astype(np.float32)
    g, q, _ = O.quantize_weights(W)
    gA, Xq, _ = O.absmax_quantize(X)
    dY = bf16(rng.standard_normal((M, N)))
    ref = O.ste_backward(dY, q, g, Xq, gA, W)
    A = ref["A_hat"]
    mask = ref["mask"]
    for m in range(M):
        for k in range(K):
            s = 0.0
            for n in range(N):  # add for +1, subtract for -1, skip 0
                s += float(dY[m, n]) if q[n, k] == 1 else (-float(dY[m, n]) if q[n, k] == -1 else 0.0)
            assert ref["dX"][m, k] == np.float32(s * float(np.float32(g)))
    for n in range(N):
        for k in range(K):
            s = sum(float(dY[m, n]) * float(A[m, k]) for m in range(M))
            assert ref["dW"][n, k] == (np.float32(s) if mask[n, k] else 0.0)


def test_mask_bits_hand_worked():
    # row 0: k = 0, 3, 31 in range -> bits 0, 3, 31 of word 0 = 0x80000009;
    # k = 32 in range -> bit 0 of word 1 = 0x1 (K = 33: bits past K stay 0)
    mask = np.zeros((2, 33), dtype=bool)
    mask[0, [0, 3, 31, 32]] = True
    mask[1, 1] = True
    words = O.pack_mask_bits(mask)
    assert words.dtype == np.uint32 and words.shape == (2, 2)
    assert words.tolist() == [[0x80000009, 0x1], [0x2, 0x0]]


def test_mask_bits_round_trip():
    rng = np.random.default_rng(9)
    for K in (1, 31, 32, 33, 64, 1000):
        mask = rng.random((7, K)) < 0.7
        words = O.pack_mask_bits(mask)
        assert words.shape == (7, -(-K // 32))
        assert np.array_equal(O.unpack_mask_bits(words, K), mask)
        if K % 32:
            assert not np.any(words[:, -1] >> np.uint32(K % 32))  # bits past K are 0
