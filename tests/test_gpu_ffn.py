"""The BitNet FFN block (BitLinear up -> ReLU^2 -> BitLinear down) on the GPU,
through the C ABI, against the oracle.

Bit-exact: the hidden ReLU^2 activations (both sides form them in the same
float32 chain, which decides the down projection's INT8 codes).  Y within
|Y - Y_ref| <= 1e-5 |Y_ref|.  The decode and prefill paths agree bit for bit.
"""
import numpy as np
import pytest
import torch

import bitlinear_absmean_ternarise_bit_amd as bl
import oracle as O
from bitlinear_absmean_ternarise_bit_amd import abi
from bitlinear_absmean_ternarise_bit_amd.workloads import make_ffn_workload, random_problem

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
RTOL = 1e-5


def say(*a):
    print(*a, flush=True)


def check_y(y, yr):
    y = np.asarray(y, dtype=np.float64)
    yr = np.asarray(yr, dtype=np.float64)
    ok = np.abs(y - yr) <= RTOL * np.abs(yr)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"Y mismatch at {idx.tolist()}: gpu {y[tuple(idx.T)]} ref {yr[tuple(idx.T)]}")


def dev_x(X, dt):
    if dt == "bf16":
        from bitlinear_absmean_ternarise_bit_amd.workloads import f32_to_bf16_bits
        return torch.from_numpy(f32_to_bf16_bits(X).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(X).to(DEV)


def problem(M, D, F, Do, seed, dt):
    P = random_problem(M, D, F, seed=seed, x_dtype=dt)
    rng = np.random.default_rng(seed + 1)
    Wd = (0.03 * rng.standard_normal((Do, F))).astype(np.float32)
    return P.X, P.W, Wd


def run(X, Wu, Wd, dt, path="auto"):
    up = bl.quantize_weights(torch.from_numpy(Wu).to(DEV))
    down = bl.quantize_weights(torch.from_numpy(Wd).to(DEV))
    Y, A = bl.ffn_forward(dev_x(X, dt), up, down, path=path, return_hidden=True)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), A.cpu().numpy()


FFN_CASES = [
    (1, 64, 64, 64, "f32", "decode"),
    (3, 300, 170, 90, "bf16", "decode"),
    (8, 2048, 5632, 2048, "bf16", "decode"),
    (16, 100, 3000, 77, "f32", "decode"),
    (16, 200, 4032, 100, "bf16", "decode"),   # the widest hidden layer the decode path takes at 16 tokens
    (40, 200, 300, 130, "bf16", "prefill"),
    (300, 1000, 650, 333, "f32", "prefill"),
    (5, 513, 260, 64, "bf16", "prefill"),
]


@pytest.mark.parametrize("M,D,F,Do,dt,path", FFN_CASES)
def test_ffn_parity(M, D, F, Do, dt, path):
    say(f"ffn M={M} D={D} F={F} D_out={Do} {dt} {path}")
    X, Wu, Wd = problem(M, D, F, Do, seed=M + D + F + Do, dt=dt)
    Y, A = run(X, Wu, Wd, dt, path)
    ref = O.ffn_forward(X if dt == "f32" else np.asarray(dev_x(X, dt).float().cpu()), Wu, Wd)
    assert np.array_equal(A, ref["A"])
    check_y(Y, ref["Y"])


def test_ffn_decode_and_prefill_agree_bitwise():
    X, Wu, Wd = problem(12, 640, 900, 200, seed=31, dt="bf16")
    Yd, Ad = run(X, Wu, Wd, "bf16", "decode")
    Yp, Ap = run(X, Wu, Wd, "bf16", "prefill")
    assert np.array_equal(Ad, Ap) and np.array_equal(Yd, Yp)


def test_ffn_batched_layers():
    L, M, D, F, Do = 4, 5, 256, 384, 192
    Xs, ups, downs, refs = [], [], [], []
    for l in range(L):
        X, Wu, Wd = problem(M, D, F, Do, seed=200 + l, dt="f32")
        Xs.append(torch.from_numpy(X))
        ups.append(bl.quantize_weights(torch.from_numpy(Wu).to(DEV)))
        downs.append(bl.quantize_weights(torch.from_numpy(Wd).to(DEV)))
        refs.append(O.ffn_forward(X, Wu, Wd))
    Xb = torch.stack(Xs).to(DEV)
    up = (torch.stack([p for p, _ in ups]), torch.cat([g for _, g in ups]))
    down = (torch.stack([p for p, _ in downs]), torch.cat([g for _, g in downs]))
    for path in ("decode", "prefill"):
        Y, A = bl.ffn_forward(Xb, up, down, path=path, return_hidden=True)
        torch.cuda.synchronize()
        for l in range(L):
            assert np.array_equal(A[l].cpu().numpy(), refs[l]["A"])
            check_y(Y[l].cpu().numpy(), refs[l]["Y"])


def test_ffn_batched_whole_layer_workgroups():
    """600 blocks with F = Do = 1000: both projections' decode launches give
    one workgroup a whole layer (its waves take every fourth block of 16 rows,
    the last block half past the end); batched equals single-block calls bit
    for bit, and sampled blocks match the oracle."""
    L, M, D, F, Do = 600, 2, 256, 1000, 1000
    g = torch.Generator(device=DEV)
    g.manual_seed(600)
    Wu = torch.randn((L, F, D), generator=g, device=DEV) * 0.02
    Wd = torch.randn((L, Do, F), generator=g, device=DEV) * 0.03
    X = torch.randn((L, M, D), generator=g, device=DEV).to(torch.bfloat16)
    up = (torch.empty((L, F, bl.packed_words(D)), dtype=torch.int32, device=DEV),
          torch.empty((L,), dtype=torch.float32, device=DEV))
    down = (torch.empty((L, Do, bl.packed_words(F)), dtype=torch.int32, device=DEV),
            torch.empty((L,), dtype=torch.float32, device=DEV))
    for l in range(L):
        bl.quantize_weights(Wu[l], out_packed=up[0][l], out_gamma=up[1][l:l + 1])
        bl.quantize_weights(Wd[l], out_packed=down[0][l], out_gamma=down[1][l:l + 1])
    Y, A = bl.ffn_forward(X, up, down, path="decode", return_hidden=True)
    torch.cuda.synchronize()
    for l in (0, 1, L // 2, L - 1):
        Yl, Al = bl.ffn_forward(X[l], (up[0][l], up[1][l:l + 1]), (down[0][l], down[1][l:l + 1]),
                                path="decode", return_hidden=True)
        torch.cuda.synchronize()
        assert torch.equal(Al, A[l]) and torch.equal(Yl, Y[l]), l
    for l in (0, L - 1):
        ref = O.ffn_forward(X[l].float().cpu().numpy(), Wu[l].cpu().numpy(), Wd[l].cpu().numpy())
        assert np.array_equal(A[l].cpu().numpy(), ref["A"])
        check_y(Y[l].cpu().numpy(), ref["Y"])


def test_ffn_all_negative_preactivations_give_zero():
    X = np.abs(np.random.default_rng(3).standard_normal((4, 128))).astype(np.float32)
    Wu = -np.abs(np.random.default_rng(4).standard_normal((96, 128))).astype(np.float32) * 0.02
    Wd = np.random.default_rng(5).standard_normal((64, 96)).astype(np.float32) * 0.02
    for path in ("decode", "prefill"):
        Y, A = run(X, Wu, Wd, "f32", path)
        assert not A.any() and not Y.any()


def test_ffn_workload_decode_full():
    say("ffn workload ffn_block_decode_m8_d2048_f5632")
    P = make_ffn_workload("ffn_block_decode_m8_d2048_f5632")
    up = bl.quantize_weights(torch.from_numpy(P.W_up).to(DEV))
    down = bl.quantize_weights(torch.from_numpy(P.W_down).to(DEV))
    X = torch.from_numpy(P.X_bf16_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    Y, A = bl.ffn_forward(X, up, down, return_hidden=True)
    torch.cuda.synchronize()
    ref = O.ffn_forward(P.X, P.W_up, P.W_down)
    assert np.array_equal(A.cpu().numpy(), ref["A"])
    check_y(Y.cpu().numpy(), ref["Y"])
    # ReLU^2 zeroes roughly half of the hidden units
    assert 0.3 < float(np.mean(ref["A"] == 0)) < 0.7


def test_ffn_workload_prefill_full():
    say("ffn workload ffn_block_prefill_m2048_d4096_f11008 (hidden layer and Y of every token)")
    P = make_ffn_workload("ffn_block_prefill_m2048_d4096_f11008")
    up = bl.quantize_weights(torch.from_numpy(P.W_up).to(DEV))
    down = bl.quantize_weights(torch.from_numpy(P.W_down).to(DEV))
    X = torch.from_numpy(P.X_bf16_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    Y, A = bl.ffn_forward(X, up, down, return_hidden=True)
    torch.cuda.synchronize()
    g_up, q_up, _ = O.quantize_weights(P.W_up)
    g_dn, q_dn, _ = O.quantize_weights(P.W_down)
    assert up[1].item() == float(g_up) and down[1].item() == float(g_dn)
    ref = O.ffn_from_codes(P.X, q_up, g_up, q_dn, g_dn)
    assert np.array_equal(A.cpu().numpy(), ref["A"])
    check_y(Y.cpu().numpy(), ref["Y"])


def test_ffn_errors():
    up = bl.quantize_weights(torch.zeros((64, 64), device=DEV))
    down = bl.quantize_weights(torch.zeros((64, 64), device=DEV))
    X = torch.zeros((20, 64), device=DEV)
    with pytest.raises(bl.BitLinearError) as e:
        bl.ffn_forward(X, up, down, path="decode")  # 20 tokens exceed the decode kernel
    assert e.value.status == abi.ERR_SHAPE
