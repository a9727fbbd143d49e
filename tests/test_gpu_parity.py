"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: gamma, packed ternary codes, INT8 activation codes, gamma_A, code
sums and INT32 accumulators.  Y: elementwise |Y - Y_ref| <= 1e-5 |Y_ref|, and
Y_ref == 0 exactly where the accumulator is 0.
"""
import numpy as np
import pytest
import torch

import bitlinear_absmean_ternarise_bit_amd as bl
import oracle as O
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


def u32(t):
    return t.cpu().numpy().view(np.uint32)


def check_y(y, yr):
    y = np.asarray(y, dtype=np.float64)
    yr = np.asarray(yr, dtype=np.float64)
    ok = np.abs(y - yr) <= RTOL * np.abs(yr)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"Y mismatch at {idx.tolist()}: gpu {y[tuple(idx.T)]} ref {yr[tuple(idx.T)]}")


def run_full(P, path="auto"):
    W = torch.from_numpy(P.W).to(DEV)
    X = dev_x(P)
    packed, gamma = bl.quantize_weights(W)
    Y, acc = bl.forward(X, packed, gamma, P.K, path=path, return_acc=True)
    torch.cuda.synchronize()
    return packed, gamma, Y, acc


# ---------------------------------------------------------------------------
# a1 + a2: gamma and packed codes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(1, 1), (3, 100), (70, 300), (128, 256), (257, 1000), (33, 4097),
                                 (2048, 2048)])
def test_quantize_weights_bit_exact(N, K):
    say(f"quantize_weights N={N} K={K}")
    P = random_problem(1, K, N, seed=N + K)
    packed, gamma = bl.quantize_weights(torch.from_numpy(P.W).to(DEV))
    torch.cuda.synchronize()
    g, q, pk = O.quantize_weights(P.W)
    assert gamma.item() == float(g)
    assert np.array_equal(u32(packed), pk)


@pytest.mark.parametrize("kind", ["wide_exponents", "large", "tiny", "zeros", "constant", "ties"])
def test_quantize_weights_special_values(kind):
    say(f"quantize_weights special {kind}")
    rng = np.random.default_rng(3)
    N, K = 96, 520
    if kind == "wide_exponents":
        W = (np.exp2(rng.uniform(-149, 120, (N, K))) * rng.choice([-1, 1], (N, K))).astype(np.float32)
        W[rng.random((N, K)) < 0.1] = 0
    elif kind == "large":
        W = (300.0 * rng.standard_normal((N, K))).astype(np.float32)
    elif kind == "tiny":
        W = (1e-30 * rng.standard_normal((N, K))).astype(np.float32)
    elif kind == "zeros":
        W = np.zeros((N, K), np.float32)
    elif kind == "constant":
        W = np.full((N, K), -0.75, np.float32)
    else:  # values at exactly half of gamma + eps
        W = np.full((N, K), 0.01, np.float32)
        for _ in range(20):
            d = np.float32(O.absmean_gamma(W) + O.EPS32)
            W[:, :8] = np.float32(d * np.float32(0.5)) * np.array([1, -1] * 4, np.float32)
    packed, gamma = bl.quantize_weights(torch.from_numpy(W).to(DEV))
    torch.cuda.synchronize()
    g, q, pk = O.quantize_weights(W)
    assert gamma.item() == float(g)
    assert np.array_equal(u32(packed), pk)


def test_gamma_independent_of_grid_scheduling():
    # repeated calls and transposed layouts give the same gamma (the sum is exact)
    P = random_problem(1, 3000, 1111, seed=5)
    W = torch.from_numpy(P.W).to(DEV)
    gs = {bl.quantize_weights(W)[1].item() for _ in range(5)}
    gs.add(bl.quantize_weights(W.t().contiguous())[1].item())
    gs.add(bl.quantize_weights(W.flatten().flip(0).reshape(3000, 1111).contiguous())[1].item())
    torch.cuda.synchronize()
    assert gs == {float(O.absmean_gamma(P.W))}


# ---------------------------------------------------------------------------
# a3: activation codes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,dt", [(1, 1, "f32"), (5, 100, "bf16"), (7, 64, "f32"), (33, 2048, "bf16"),
                                    (6, 4096, "bf16"), (3, 2048, "f32"), (5, 4096, "f32"), (2, 8192, "f32"),
                                    (3, 4104, "bf16"), (2, 16384, "bf16"), (3, 11008, "f32"),
                                    (2, 16384, "f32"), (1, 20000, "f32"), (2, 33000, "bf16"),
                                    (4, 8191, "f32"), (9, 8192, "bf16"), (130, 136, "bf16")])
def test_quantize_activations_bit_exact(M, K, dt):
    say(f"quantize_activations M={M} K={K} {dt}")
    P = random_problem(M, K, 1, seed=M * K, x_dtype=dt, x_scale=2.0)
    X = dev_x(P)
    Xq, ga, rs = bl.quantize_activations(X)
    torch.cuda.synchronize()
    rga, rxq, rrs = O.absmax_quantize(P.X)
    assert np.array_equal(ga.cpu().numpy(), rga)
    xq = Xq.cpu().numpy()
    assert np.array_equal(xq[:, :K], rxq)
    assert not xq[:, K:].any()
    assert np.array_equal(rs.cpu().numpy(), rrs)


def test_quantize_activations_ties_and_zero_token():
    # a token whose scale is exactly 1 and whose values sit on .5 ties, plus an all-zero token
    g = np.float32(127.0)
    while np.float32(np.float32(127) / np.float32(g + O.EPS32)) != np.float32(1):
        g = np.nextafter(g, np.float32(0))
    row = np.array([g, 0.5, 1.5, 2.5, -0.5, -2.5, 3.5, 126.5] + [0.25] * 56, np.float32)
    X = np.stack([row, np.zeros_like(row), -row])
    Xq, ga, rs = bl.quantize_activations(torch.from_numpy(X).to(DEV))
    torch.cuda.synchronize()
    rga, rxq, rrs = O.absmax_quantize(X)
    assert np.array_equal(Xq.cpu().numpy()[:, :64], rxq)
    assert rxq[0, :8].tolist() == [127, 0, 2, 2, 0, -2, 4, 126]
    assert np.array_equal(ga.cpu().numpy(), rga) and np.array_equal(rs.cpu().numpy(), rrs)


# ---------------------------------------------------------------------------
# a4..a6: the forward on both paths
# ---------------------------------------------------------------------------

FORWARD_CASES = [
    # (M, K, N, dtype, path)
    (1, 64, 16, "f32", "decode"),
    (1, 9, 1, "f32", "decode"),
    (3, 100, 77, "bf16", "decode"),
    (8, 2048, 5632, "bf16", "decode"),
    (16, 1000, 300, "f32", "decode"),
    (16, 4000, 129, "bf16", "decode"),
    (1, 2048, 2048, "bf16", "prefill"),
    (17, 300, 257, "f32", "prefill"),
    (300, 520, 600, "bf16", "prefill"),
    (257, 200, 513, "f32", "prefill"),
    (512, 1088, 768, "bf16", "prefill"),
    (40, 4096, 1000, "bf16", "auto"),
    (1024, 640, 6144, "bf16", "prefill"),   # 128 x 256 tiles
    (2000, 1050, 6200, "f32", "prefill"),   # 256 x 256 tiles, ragged M, N and a half K stage
    (2048, 200, 11008, "bf16", "prefill"),  # 1.34 rounds of big tiles: columns split over two launches
    (2048, 200, 11000, "f32", "prefill"),   # same split, ragged N: partial last row block in the second
    (1, 65472, 64, "bf16", "decode"),       # the longest row the decode path holds on chip (Kp + 16 = 65488)
    (16, 3000, 333, "f32", "decode"),       # float32 rows over 4 KiB: the wave quantiser's two passes
    (7, 8192, 200, "f32", "decode"),        # 32 KiB float32 rows, seven tokens over four waves
    # single calls whose token rows (at most 4 16-byte chunks per lane) are
    # requested before the weights: one token per wave, then five to eight
    # tokens (some waves with two), float32 rows at the 4 KiB limit
    (3, 2048, 100, "bf16", "decode"),
    (4, 1024, 64, "f32", "decode"),
    (5, 512, 96, "bf16", "decode"),
    (6, 1024, 40, "f32", "decode"),
]


# Persistent prefill workgroups (one per CU) walking several tiles each: tile
# counts above 256, with and without the XCD remap (count % 8), one-stage and
# half-stage K, ragged M and N.
PERSISTENT_CASES = [
    (4100, 1050, 5000, "bf16"),  # 340 tiles (no remap), half K stage, ragged M and N
    (4096, 640, 5120, "f32"),    # 320 tiles (remapped), five stages
    (4096, 100, 5120, "bf16"),   # one stage per tile
    (4096, 64, 5120, "f32"),     # a single half stage per tile
]


def test_prefill_largest_k():
    """K = 2^20, the largest the library accepts: 16384 stages per tile and
    accumulators up to 127 * 2^20 in magnitude, still exact in INT32."""
    M, K, N = 20, 1 << 20, 50
    say(f"prefill largest K M={M} K={K} N={N}")
    P = random_problem(M, K, N, seed=7, x_dtype="f32")
    packed, gamma, Y, acc = run_full(P, path="prefill")
    ref = O.bitlinear_forward(P.X, P.W)
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    check_y(Y.cpu().numpy(), ref["Y"])


def test_prefill_token_chunks():
    """M * Kp above 2^31 code bytes: the GEMM runs the tokens in chunks (its
    buffer offsets are 32-bit).  X is a seeded 64-token block repeated down
    33000 rows, so every output row has an oracle value: that of its row in
    the block.  The chunk boundary (row 32640 with 128-row tiles) lies inside
    the range, and so does a ragged last tile."""
    R, K, N, M = 64, 65536, 64, 33000
    assert M * K > 2 ** 31
    say(f"prefill token chunks M={M} K={K} N={N}")
    P = random_problem(R, K, N, seed=11, x_dtype="bf16")
    ref = O.bitlinear_forward(P.X, P.W)
    W = torch.from_numpy(P.W).to(DEV)
    X = dev_x(P).repeat((M + R - 1) // R, 1)[:M].contiguous()
    packed, gamma = bl.quantize_weights(W)
    Y, acc = bl.forward(X, packed, gamma, K, path="prefill", return_acc=True)
    torch.cuda.synchronize()
    del X
    rows = np.arange(M) % R
    assert np.array_equal(acc.cpu().numpy(), ref["acc"][rows])
    check_y(Y.cpu().numpy(), ref["Y"][rows])


@pytest.mark.parametrize("M,K,N,dt", PERSISTENT_CASES)
def test_prefill_persistent_tiles(M, K, N, dt):
    say(f"prefill persistent M={M} K={K} N={N} {dt}")
    P = random_problem(M, K, N, seed=M + 3 * K + 5 * N, x_dtype=dt)
    W = torch.from_numpy(P.W).to(DEV)
    X = dev_x(P)
    packed, gamma = bl.quantize_weights(W)
    Y, acc = bl.forward(X, packed, gamma, K, path="prefill", return_acc=True)
    Y_only = bl.forward(X, packed, gamma, K, path="prefill")
    torch.cuda.synchronize()
    ref = O.bitlinear_forward(P.X, P.W)
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    check_y(Y.cpu().numpy(), ref["Y"])
    assert torch.equal(Y, Y_only)  # the Y-only epilogue equals the one that also stores acc


@pytest.mark.parametrize("M,K,N,dt,path", FORWARD_CASES)
def test_forward_parity(M, K, N, dt, path):
    say(f"forward M={M} K={K} N={N} {dt} {path}")
    P = random_problem(M, K, N, seed=M + 7 * K + 13 * N, x_dtype=dt)
    packed, gamma, Y, acc = run_full(P, path)
    ref = O.bitlinear_forward(P.X, P.W)
    assert gamma.item() == float(ref["gamma"])
    assert np.array_equal(u32(packed), ref["packed"])
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    check_y(Y.cpu().numpy(), ref["Y"])


def test_worked_example_on_gpu():
    # the article's Zero-GEMM example (acc = -149), K = 9 (ragged) on both paths
    x = np.array([[42, -18, 105, -7, 88, 12, -64, 3, 127]], np.float32)
    w = np.array([[1, 0, -1, 1, 0, -1, 1, -1, 0]], np.float32) * np.float32(0.02)
    packed, gamma = bl.quantize_weights(torch.from_numpy(w).to(DEV))
    for path in ("decode", "prefill"):
        Y, acc = bl.forward(torch.from_numpy(x).to(DEV), packed, gamma, 9, path=path, return_acc=True)
        torch.cuda.synchronize()
        assert acc.item() == -149
        assert Y.item() == float(np.float32(-149.0 * float(O.absmean_gamma(w))))


def test_decode_and_prefill_agree_bitwise():
    P = random_problem(16, 2050, 333, seed=21, x_dtype="bf16")
    W = torch.from_numpy(P.W).to(DEV)
    X = dev_x(P)
    packed, gamma = bl.quantize_weights(W)
    Yd, ad = bl.forward(X, packed, gamma, P.K, path="decode", return_acc=True)
    Yp, ap = bl.forward(X, packed, gamma, P.K, path="prefill", return_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(ad, ap)
    assert torch.equal(Yd, Yp)


def test_forward_quantized_matches_forward():
    P = random_problem(70, 333, 140, seed=31, x_dtype="bf16")
    W = torch.from_numpy(P.W).to(DEV)
    X = dev_x(P)
    packed, gamma = bl.quantize_weights(W)
    Xq, ga, rs = bl.quantize_activations(X)
    Yq, aq = bl.forward_quantized(Xq, ga, rs, packed, gamma, P.K, return_acc=True)
    Yf, af = bl.forward(X, packed, gamma, P.K, path="prefill", return_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(aq, af) and torch.equal(Yq, Yf)
    assert np.array_equal(aq.cpu().numpy(), O.bitlinear_forward(P.X, P.W)["acc"])


def test_forward_deterministic():
    P = random_problem(300, 700, 300, seed=4, x_dtype="bf16")
    W = torch.from_numpy(P.W).to(DEV)
    X = dev_x(P)
    packed, gamma = bl.quantize_weights(W)
    outs = [bl.forward(X, packed, gamma, P.K) for _ in range(5)]
    outs += [bl.forward(X[:8], packed, gamma, P.K) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:5]:
        assert torch.equal(o, outs[0])
    for o in outs[6:]:
        assert torch.equal(o, outs[5])
    assert torch.equal(outs[5], outs[0][:8])


def test_row_independence():
    P = random_problem(40, 300, 70, seed=6, x_dtype="f32")
    W = torch.from_numpy(P.W).to(DEV)
    X = dev_x(P)
    packed, gamma = bl.quantize_weights(W)
    Y = bl.forward(X, packed, gamma, P.K)
    rows = [bl.forward(X[m:m + 1].contiguous(), packed, gamma, P.K) for m in (0, 13, 39)]
    torch.cuda.synchronize()
    for r, m in zip(rows, (0, 13, 39)):
        assert torch.equal(r[0], Y[m])


def test_zero_weights_rows_and_tokens():
    P = random_problem(20, 200, 90, seed=8, x_dtype="f32")
    W, X = P.W.copy(), P.X.copy()
    W[[0, 5, 89]] = 0
    X[[3, 19]] = 0
    for path in ("decode", "prefill"):
        Xd = torch.from_numpy(X[:16] if path == "decode" else X).to(DEV)
        packed, gamma = bl.quantize_weights(torch.from_numpy(W).to(DEV))
        Y = bl.forward(Xd, packed, gamma, 200, path=path).cpu().numpy()
        assert not Y[:, [0, 5, 89]].any()
        assert not Y[3].any()
        ref = O.bitlinear_forward(Xd.cpu().numpy(), W)
        check_y(Y, ref["Y"])
    # gamma = 0: every code is 0 and Y is 0
    packed, gamma = bl.quantize_weights(torch.zeros((33, 70), device=DEV))
    Y = bl.forward(torch.from_numpy(P.X).to(DEV)[:, :70].contiguous(), packed, gamma, 70)
    torch.cuda.synchronize()
    assert gamma.item() == 0.0 and not Y.any()


def test_forward_batched_matches_single_calls():
    L, M, K, N = 5, 3, 1000, 200
    Ps = [random_problem(M, K, N, seed=100 + l, x_dtype="bf16") for l in range(L)]
    X = torch.stack([dev_x(P) for P in Ps])
    q = [bl.quantize_weights(torch.from_numpy(P.W).to(DEV)) for P in Ps]
    packed = torch.stack([p for p, _ in q])
    gamma = torch.cat([g for _, g in q])
    Yb = bl.forward_batched(X, packed, gamma, K)
    torch.cuda.synchronize()
    for l, P in enumerate(Ps):
        Ys = bl.forward(X[l], packed[l], gamma[l:l + 1], K)
        assert torch.equal(Yb[l], Ys)
        check_y(Yb[l].cpu().numpy(), O.bitlinear_forward(P.X, P.W)["Y"])


# ---------------------------------------------------------------------------
# The named workloads at their full sizes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["single_m4_k256_n128", "decode_m1_k2048_n2048",
                                  "decode_ffn_up_m8_k2048_n5632"])
def test_workload_full(name):
    say(f"workload {name}")
    P = make_workload(name)
    packed, gamma, Y, acc = run_full(P)
    ref = O.bitlinear_forward(P.X, P.W)
    assert gamma.item() == float(ref["gamma"])
    assert np.array_equal(u32(packed), ref["packed"])
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    check_y(Y.cpu().numpy(), ref["Y"])
    if name == "decode_ffn_up_m8_k2048_n5632":
        zero_frac = float(np.mean(ref["q"] == 0))
        assert abs(zero_frac - 0.3101) < 0.005  # roughly a third of the weights are zero


def test_workload_prefill_m2048_k4096_n11008_full():
    say("workload prefill_ffn_m2048_k4096_n11008 (full compare)")
    P = make_workload("prefill_ffn_m2048_k4096_n11008")
    packed, gamma, Y, acc = run_full(P)
    g, q, pk = O.quantize_weights(P.W)
    assert gamma.item() == float(g)
    assert np.array_equal(u32(packed), pk)
    Xq, ga, rs = bl.quantize_activations(dev_x(P))
    rga, rxq, rrs = O.absmax_quantize(P.X)
    assert np.array_equal(Xq.cpu().numpy(), rxq) and np.array_equal(ga.cpu().numpy(), rga)
    racc = O.zero_gemm(rxq, q)
    assert np.array_equal(acc.cpu().numpy(), racc)
    check_y(Y.cpu().numpy(), O.dequant(racc, g, rga))


def test_workload_prefill_m8192_k8192_n28672_full():
    """The 70B-like FFN projection compared in full: gamma, every packed word,
    every activation code, and all 8192 x 28672 accumulators and outputs
    (the oracle's exact contraction in chunks of 2048 tokens).  Both epilogues
    run at this size: the one that also stores the accumulators, and the
    Y-only one that bitlinear_forward uses, which must give the same Y."""
    say("workload prefill_ffn_m8192_k8192_n28672 (full compare)")
    P = make_workload("prefill_ffn_m8192_k8192_n28672")
    W = torch.from_numpy(P.W).to(DEV)
    packed, gamma = bl.quantize_weights(W)
    del W
    X = dev_x(P)
    Y, acc = bl.forward(X, packed, gamma, P.K, return_acc=True)
    Y_only = bl.forward(X, packed, gamma, P.K)
    Xq, ga, rs = bl.quantize_activations(X)
    torch.cuda.synchronize()
    assert torch.equal(Y_only, Y)
    del Y_only
    zr = torch.from_numpy(P.notes["zero_rows"]).to(DEV)
    assert not Y[:, zr].any()  # zero weight rows give zero output columns
    acc_h = acc.cpu().numpy()
    y_h = Y.cpu().numpy()
    del acc, Y
    g, q, pk = O.quantize_weights(P.W)
    assert gamma.item() == float(g)
    assert np.array_equal(u32(packed), pk)
    assert abs(float(np.mean(q == 0)) - 0.579) < 0.005
    rga, rxq, rrs = O.absmax_quantize(P.X)
    assert np.array_equal(Xq.cpu().numpy(), rxq)
    assert np.array_equal(ga.cpu().numpy(), rga) and np.array_equal(rs.cpu().numpy(), rrs)
    for r0 in range(0, P.M, 2048):
        say(f"  tokens {r0}..{r0 + 2047}")
        racc = O.zero_gemm(rxq[r0:r0 + 2048], q)
        assert np.array_equal(acc_h[r0:r0 + 2048], racc)
        check_y(y_h[r0:r0 + 2048], O.dequant(racc, g, rga[r0:r0 + 2048]))
