"""STE backward on the GPU (through the C ABI) against the oracle.

Bit-exact: the transposed packed codes, the range-mask bits and the positions
where dW is masked to zero.  dX and dW: the products dY * code and dY * A_hat are exact in float32
and the GPU sums them in float32 (bf16 matrix cores), so each result may differ
from the oracle's exact sum by at most L * 2^-24 * sum|products| (L = the
contraction length, one rounding per addition) plus one final rounding.
"""
import numpy as np
import pytest
import torch

import bitlinear_absmean_ternarise_bit_amd as bl
import oracle as O
from bitlinear_absmean_ternarise_bit_amd import abi
from bitlinear_absmean_ternarise_bit_amd.workloads import f32_to_bf16_bits, bf16_bits_to_f32, random_problem

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def bound_check(got, ref, absprod, L):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    tol = L * 2.0 ** -24 * absprod + 2.0 ** -23 * np.abs(ref)
    bad = np.abs(got - ref) > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"mismatch at {idx.tolist()}: gpu {got[tuple(idx.T)]} ref {ref[tuple(idx.T)]}")
    # rounding errors stay far below the worst case: a dropped or misplaced
    # product (about sum|products| / L) would show in the median
    nz = absprod > 0
    if nz.any():
        med = float(np.median(np.abs(got - ref)[nz] / absprod[nz]))
        assert med < 2.0 ** -20, med


def setup(M, K, N, seed, outside=0.1):
    rng = np.random.default_rng(seed)
    P = random_problem(M, K, N, seed=seed, x_dtype="bf16")
    W = P.W.copy()
    W[rng.random(W.shape) < outside] *= 4.0  # weights outside the clip range: masked gradient
    bits = f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    dY = bf16_bits_to_f32(bits)
    Wd = torch.from_numpy(W).to(DEV)
    packed, gamma = bl.quantize_weights(Wd)
    X = torch.from_numpy(P.X_bf16_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    Xq, ga, _ = bl.quantize_activations(X)
    packedT, mask = bl.pack_transposed(Wd, gamma)
    dYd = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return P, W, dY, gamma, Xq, ga, packedT, mask, dYd


@pytest.mark.parametrize("N,K", [(1, 1), (70, 33), (129, 300), (640, 1000), (16, 4097)])
def test_pack_transposed_bit_exact(N, K):
    say(f"pack_transposed N={N} K={K}")
    P = random_problem(1, K, N, seed=N * K)
    W = torch.from_numpy(P.W).to(DEV)
    packed, gamma = bl.quantize_weights(W)
    Wm = P.W.copy()
    Wm[::3] *= 3.0  # some weights outside the clip range: mask bits 0
    Wm_d = torch.from_numpy(Wm).to(DEV)
    pT, mask = bl.pack_transposed(Wm_d, gamma)
    pT_only, _ = bl.pack_transposed(Wm_d, gamma)
    torch.cuda.synchronize()
    g, q, _ = O.quantize_weights(P.W)
    assert pT.shape == (K, bl.packed_words(N))
    qm = O.ternary_codes(Wm, g)  # the codes of Wm under P.W's gamma
    assert np.array_equal(pT.cpu().numpy().view(np.uint32), O.pack_codes(np.ascontiguousarray(qm.T)))
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), O.pack_mask_bits(O.ste_weight_mask(Wm, g)))
    assert torch.equal(pT, pT_only)


BWD_CASES = [(1, 64, 64), (37, 300, 130), (128, 256, 192), (200, 1000, 520), (65, 130, 1100), (300, 64, 7),
             (77, 2000, 264), (513, 96, 1032)]


@pytest.mark.parametrize("M,K,N", BWD_CASES)
def test_backward_parity(M, K, N):
    say(f"backward M={M} K={K} N={N}")
    P, W, dY, gamma, Xq, ga, packedT, mask, dYd = setup(M, K, N, seed=M + K + N)
    dX, dW = bl.backward(dYd, packedT, gamma, Xq, ga, mask, K)
    torch.cuda.synchronize()
    g, q, _ = O.quantize_weights(W)
    rga, rxq, _ = O.absmax_quantize(P.X)
    assert np.array_equal(Xq.cpu().numpy()[:, :K], rxq)
    ref = O.ste_backward(dY, q, g, rxq, rga, W)
    absX = (np.abs(dY).astype(np.float64) @ np.abs(q).astype(np.float64)) * float(g)
    bound_check(dX.cpu().numpy(), ref["dX"], absX, N)
    absW = np.abs(dY).astype(np.float64).T @ np.abs(ref["A_hat"]).astype(np.float64)
    got_w = dW.cpu().numpy()
    assert np.all(got_w[~ref["mask"]] == 0.0)
    bound_check(got_w, ref["dW"], absW, M)


@pytest.mark.parametrize("M,K,N", [(1, 64, 64), (77, 2000, 264), (513, 96, 1032), (200, 1000, 520), (64, 512, 8)])
def test_backward_dw_paths_agree(M, K, N):
    """dW from dY and the codes as they lie (rows 16-byte aligned, N % 8 == 0)
    and from transposed copies (dY at an address that is not 16-byte
    aligned) are the same bits: both feed the matrix cores the same operands
    in the same order.  dX likewise (dY read in place vs a padded copy)."""
    say(f"backward dW paths M={M} K={K} N={N}")
    P, W, dY, gamma, Xq, ga, packedT, mask, dYd = setup(M, K, N, seed=3 * M + K + N)
    flat = torch.empty((M * N + 8,), dtype=torch.bfloat16, device=DEV)
    dYu = flat[1:1 + M * N].view(M, N)  # 2 bytes past a 16-byte boundary
    dYu.copy_(dYd)
    assert dYu.data_ptr() % 16 != 0 and dYd.data_ptr() % 16 == 0
    dX, dW = bl.backward(dYd, packedT, gamma, Xq, ga, mask, K)
    dXu, dWu = bl.backward(dYu, packedT, gamma, Xq, ga, mask, K)
    torch.cuda.synchronize()
    assert torch.equal(dW, dWu) and torch.equal(dX, dXu)


def test_backward_one_output_at_a_time():
    P, W, dY, gamma, Xq, ga, packedT, mask, dYd = setup(50, 200, 90, seed=7)
    dX, dW = bl.backward(dYd, packedT, gamma, Xq, ga, mask, 200)
    dX1, n1 = bl.backward(dYd, packedT, gamma, Xq, ga, mask, 200, need_dw=False)
    n2, dW2 = bl.backward(dYd, packedT, gamma, Xq, ga, mask, 200, need_dx=False)
    torch.cuda.synchronize()
    assert n1 is None and n2 is None
    assert torch.equal(dX, dX1) and torch.equal(dW, dW2)


def test_backward_in_graph():
    """Captured into a HIP graph, replays match the eager call, with eager
    work and synchronisations between the replays."""
    P, W, dY, gamma, Xq, ga, packedT, mask, dYd = setup(256, 512, 640, seed=10)
    ws = torch.empty((abi.load().bitlinear_backward_workspace_bytes(256, 640, 512),), dtype=torch.uint8,
                     device=DEV)
    dX0, dW0 = bl.backward(dYd, packedT, gamma, Xq, ga, mask, 512, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dXg, dWg = bl.backward(dYd, packedT, gamma, Xq, ga, mask, 512, workspace=ws)
    for i in range(3):
        dXg.zero_()
        dWg.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dXg, dX0) and torch.equal(dWg, dW0), i
        e1, e2 = bl.backward(dYd, packedT, gamma, Xq, ga, mask, 512, workspace=ws)  # eager work between
        torch.cuda.synchronize()
        assert torch.equal(e1, dX0) and torch.equal(e2, dW0)


def test_backward_7b_ffn_shape_full():
    # the 7B-like prefill projection (2048 x 4096 -> 11008): every element of dX and dW
    M, K, N = 2048, 4096, 11008
    say(f"backward {M}x{K}x{N} (full compare)")
    P, W, dY, gamma, Xq, ga, packedT, mask, dYd = setup(M, K, N, seed=11, outside=0.05)
    dX, dW = bl.backward(dYd, packedT, gamma, Xq, ga, mask, K)
    torch.cuda.synchronize()
    g, q, _ = O.quantize_weights(W)
    rga, rxq, _ = O.absmax_quantize(P.X)
    ref = O.ste_backward(dY, q, g, rxq, rga, W)
    absX = (np.abs(dY).astype(np.float64) @ np.abs(q).astype(np.float64)) * float(g)
    bound_check(dX.cpu().numpy(), ref["dX"], absX, N)
    del absX
    absW = np.abs(dY).astype(np.float64).T @ np.abs(ref["A_hat"]).astype(np.float64)
    got_w = dW.cpu().numpy()
    assert np.all(got_w[~ref["mask"]] == 0.0)
    bound_check(got_w, ref["dW"], absW, M)


def test_backward_errors():
    lib = abi.load()
    z = torch.zeros((4, 4), dtype=torch.bfloat16, device=DEV)
    g = torch.ones((1,), device=DEV)
    assert lib.bitlinear_backward(z.data_ptr(), 4, 4, 4, None, g.data_ptr(), None, None, None, None, None,
                                  None, 0, None) == abi.ERR_NULL
    with pytest.raises(bl.BitLinearError) as e:
        bl.backward(z, torch.zeros((4, 4), dtype=torch.int32, device=DEV), g,
                    torch.zeros((4, 64), dtype=torch.int8, device=DEV), g.repeat(4),
                    torch.zeros((4, 1), dtype=torch.int32, device=DEV), 4,
                    workspace=torch.empty((16,), dtype=torch.uint8, device=DEV))
    assert e.value.status == abi.ERR_WORKSPACE
