"""The LUT contraction on the GPU, through the C ABI, against the oracle's LUT form.

Bit-exact: the INT32 accumulators (the oracle's lut_gemv, which its pins tie
to the plain definition); Y within |Y - Y_ref| <= 1e-5 |Y_ref|.  The LUT
forward must also equal the matrix-core forward bit for bit (same codes, same
epilogue).
"""
import numpy as np
import pytest
import torch

import bitlinear_absmean_ternarise_bit_amd as bl
import oracle as O
from bitlinear_absmean_ternarise_bit_amd import abi
from bitlinear_absmean_ternarise_bit_amd.workloads import make_workload, random_problem

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
RTOL = 1e-5


def say(*a):
    print(*a, flush=True)


def dev_x(P):
    if P.x_dtype == "bf16":
        return torch.from_numpy(P.X_bf16_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(P.X).to(DEV)


def check_y(y, yr):
    y = np.asarray(y, dtype=np.float64)
    yr = np.asarray(yr, dtype=np.float64)
    ok = np.abs(y - yr) <= RTOL * np.abs(yr)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"Y mismatch at {idx.tolist()}: gpu {y[tuple(idx.T)]} ref {yr[tuple(idx.T)]}")


LUT_CASES = [
    (1, 1, 1, "f32"),            # one weight: a single unit, the slice's second unit absent
    (1, 64, 256, "bf16"),        # one unit per row, one full workgroup of rows
    (2, 100, 257, "f32"),        # a second workgroup holding one row
    (3, 128, 300, "bf16"),       # exactly one slice
    (5, 1001, 1000, "bf16"),     # ragged K, odd slice count
    (8, 2048, 5632, "bf16"),
    (16, 700, 129, "f32"),       # the largest token count (two tables per thread)
    (9, 333, 70, "bf16"),
    (1, 4096, 2050, "f32"),
    (4, 20000, 64, "bf16"),      # long rows: many slices
]


@pytest.mark.parametrize("M,K,N,dt", LUT_CASES)
def test_forward_lut_parity(M, K, N, dt):
    say(f"forward_lut M={M} K={K} N={N} {dt}")
    P = random_problem(M, K, N, seed=M + 7 * K + 13 * N, x_dtype=dt)
    W = torch.from_numpy(P.W).to(DEV)
    X = dev_x(P)
    packed, gamma = bl.quantize_weights(W)
    Y, acc = bl.forward_lut(X, packed, gamma, K, return_acc=True)
    Y2, acc2 = bl.forward(X, packed, gamma, K, return_acc=True)
    torch.cuda.synchronize()
    g, q, _ = O.quantize_weights(P.W)
    ref = O.lut_forward(P.X, q, g)
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    check_y(Y.cpu().numpy(), ref["Y"])
    assert torch.equal(acc, acc2) and torch.equal(Y, Y2)


def test_forward_lut_from_oracle_packed_words():
    # the lookups alone: words packed by the oracle, extreme codes in the tables
    M, K, N = 4, 1234, 150
    rng = np.random.default_rng(23)
    q = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    X = rng.choice(np.array([-3.0, 3.0, 0.0], np.float32), size=(M, K))
    X[:, ::5] = 127.0  # every token holds many codes of 127 (the table's largest magnitude)
    packed = torch.from_numpy(O.pack_codes(q).view(np.int32)).to(DEV)
    gamma = torch.tensor([0.0375], dtype=torch.float32, device=DEV)
    Y, acc = bl.forward_lut(torch.from_numpy(X).to(DEV), packed, gamma, K, return_acc=True)
    torch.cuda.synchronize()
    ref = O.lut_forward(X, q, np.float32(0.0375))
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    check_y(Y.cpu().numpy(), ref["Y"])


def test_worked_example_lut():
    # the article's Zero-GEMM example (acc = -149) through the LUT path
    x = np.array([[42, -18, 105, -7, 88, 12, -64, 3, 127]], np.float32)
    w = np.array([[1, 0, -1, 1, 0, -1, 1, -1, 0]], np.float32) * np.float32(0.02)
    packed, gamma = bl.quantize_weights(torch.from_numpy(w).to(DEV))
    Y, acc = bl.forward_lut(torch.from_numpy(x).to(DEV), packed, gamma, 9, return_acc=True)
    torch.cuda.synchronize()
    assert acc.item() == -149
    assert Y.item() == float(np.float32(-149.0 * float(O.absmean_gamma(w))))


def test_forward_lut_batched_layers():
    L, M, K, N = 5, 3, 700, 300
    Ps = [random_problem(M, K, N, seed=500 + l, x_dtype="bf16") for l in range(L)]
    X = torch.stack([dev_x(P) for P in Ps])
    q = [bl.quantize_weights(torch.from_numpy(P.W).to(DEV)) for P in Ps]
    packed = torch.stack([p for p, _ in q])
    gamma = torch.cat([g for _, g in q])
    Yb, accb = bl.forward_lut(X, packed, gamma, K, return_acc=True)
    Yd = bl.forward_batched(X, packed, gamma, K)
    torch.cuda.synchronize()
    for l, P in enumerate(Ps):
        g, ql, _ = O.quantize_weights(P.W)
        ref = O.lut_forward(P.X, ql, g)
        assert np.array_equal(accb[l].cpu().numpy(), ref["acc"])
        check_y(Yb[l].cpu().numpy(), ref["Y"])
    assert torch.equal(Yb, Yd)


def test_forward_lut_limits():
    lib = abi.load()
    X17 = torch.zeros((17, 64), dtype=torch.float32, device=DEV)
    packed = torch.zeros((10, bl.packed_words(64)), dtype=torch.int32, device=DEV)
    gamma = torch.ones((1,), dtype=torch.float32, device=DEV)
    with pytest.raises(bl.BitLinearError) as e:
        bl.forward_lut(X17, packed, gamma, 64)
    assert e.value.status == abi.ERR_SHAPE
    ws = torch.empty((lib.bitlinear_lut_workspace_bytes(1, 1, 64),), dtype=torch.uint8, device=DEV)
    with pytest.raises(bl.BitLinearError) as e:
        bl.forward_lut(X17[:1], packed, gamma, 64, workspace=ws[:-1])
    assert e.value.status == abi.ERR_WORKSPACE


@pytest.mark.parametrize("name", ["single_m4_k256_n128", "decode_m1_k2048_n2048",
                                  "decode_ffn_up_m8_k2048_n5632"])
def test_workload_full_lut(name):
    say(f"workload {name} LUT")
    P = make_workload(name)
    W = torch.from_numpy(P.W).to(DEV)
    packed, gamma = bl.quantize_weights(W)
    Y, acc = bl.forward_lut(dev_x(P), packed, gamma, P.K, return_acc=True)
    torch.cuda.synchronize()
    g, q, _ = O.quantize_weights(P.W)
    ref = O.lut_forward(P.X, q, g)
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    check_y(Y.cpu().numpy(), ref["Y"])
