"""One decode layer per call, for a kernel trace:

    rocprofv3 --kernel-trace --stats -d OUT -- python -m bitlinear_absmean_ternarise_bit_amd.profile_single_layer

Each call is one forward of one layer (bitlinear_forward on the decode path)
of the d_model-2048 projection (1 x 2048 x 2048) and of the small-batch FFN
up-projection (8 x 2048 x 5632), rotating over 64 distinct layers so the
weights come from HBM; the trace gives the kernel's own duration, which the
host-side loop cannot show (there the launch latency dominates).
"""
from __future__ import annotations

import torch

from . import forward, packed_words, quantize_weights


def main(calls: int = 512, layers: int = 64) -> None:
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    for M, K, N in ((1, 2048, 2048), (8, 2048, 5632)):
        X = torch.randn((layers, M, K), generator=g, device=dev).to(torch.bfloat16)
        packed = torch.empty((layers, N, packed_words(K)), dtype=torch.int32, device=dev)
        gamma = torch.empty((layers,), dtype=torch.float32, device=dev)
        W = torch.empty((N, K), dtype=torch.float32, device=dev)
        for l in range(layers):
            W.normal_(0.0, 0.02, generator=g)
            quantize_weights(W, out_packed=packed[l], out_gamma=gamma[l:l + 1])
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        for i in range(calls):
            l = i % layers
            forward(X[l], packed[l], gamma[l:l + 1], K, out=Y)
        torch.cuda.synchronize()
        print(f"{calls} single-layer calls of {M}x{K}x{N} done", flush=True)


if __name__ == "__main__":
    main()
