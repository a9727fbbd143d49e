"""The decode step exactly as the benchmark times it (one batched launch over a
pool of >= 1 GiB of packed weights), checked against the oracle on sampled
layers: every output of the sampled layers, bit-exact codes, Y to 1e-5."""
import numpy as np
import pytest
import torch

import bench
import bitlinear_absmean_ternarise_bit_amd as bl
import oracle as O

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("workload,fmt", [("decode_m1_k2048_n2048", "2bit"),
                                          ("decode_m1_k2048_n2048", "radix3"),
                                          ("decode_ffn_up_m8_k2048_n5632", "2bit"),
                                          ("decode_ffn_up_m8_k2048_n5632", "radix3")])
def test_bench_decode_pool(workload, fmt):
    from bitlinear_absmean_ternarise_bit_amd.workloads import make_workload
    P0 = make_workload(workload)
    row_bytes = bl.r3_row_bytes(P0.K) if fmt == "radix3" else bl.packed_words(P0.K) * 4
    L = max(8, -(-(1 << 30) // (P0.N * row_bytes)))  # the benchmark's default pool
    keep = sorted({0, 1, L // 2, L - 1})
    say(f"bench pool {workload} {fmt}: L={L}, checking layers {keep}")
    P, X, packed, gamma, _, Ws = bench.build_decode_pool(torch, bl, DEV, workload, L, fmt, keep=keep)
    Y = torch.empty((L, P.M, P.N), dtype=torch.float32, device=DEV)
    if fmt == "radix3":
        bl.forward_r3(X, packed, gamma, P.K, out=Y)
    else:
        bl.forward_batched(X, packed, gamma, P.K, out=Y)
    torch.cuda.synchronize()
    for l in keep:
        g, q, pk = O.quantize_weights(Ws[l])
        assert gamma[l].item() == float(g)
        want = O.pack_codes_r3(q) if fmt == "radix3" else pk
        got = packed[l].cpu().numpy()
        assert np.array_equal(got if fmt == "radix3" else got.view(np.uint32), want)
        ref = O.forward_from_codes(X[l].float().cpu().numpy(), q, g)
        y = Y[l].cpu().numpy().astype(np.float64)
        yr = ref["Y"].astype(np.float64)
        assert np.all(np.abs(y - yr) <= 1e-5 * np.abs(yr)), l
    del X, packed, Y
    torch.cuda.empty_cache()
