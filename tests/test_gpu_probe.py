"""The attainable-peak probes (the benchmark's libbitlinear_probe.so) touch exactly
the bytes they are timed on: the streaming read folds every word of its slice
(checked against a host emulation of the access pattern), the copy
reproduces its source, and the MFMA loop is deterministic."""
import numpy as np
import pytest
import torch

import bitlinear_absmean_ternarise_bit_amd as bl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def stream():
    return torch.cuda.current_stream(DEV).cuda_stream


def test_probe_stream_read_folds_every_word():
    blocks, per_block = 6, 3 * 32768
    rng = np.random.default_rng(5)
    host = rng.integers(0, 2 ** 32, size=blocks * per_block // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    out = torch.zeros(blocks * 256, dtype=torch.int32, device=DEV)
    lib = bl.abi.load_probe()
    bl.abi.check("probe", lib.bitlinear_probe_stream(src.data_ptr(), None, blocks * per_block, blocks,
                                                      out.data_ptr(), stream()))
    torch.cuda.synchronize()
    # thread t of block b: wave w = t // 64, lane l = t % 64 reads the 16-byte
    # vectors at w*8192 + l*16 + u*1024 + i*32768 (u < 8) of its slice
    words = host.reshape(blocks, per_block // 32768, 4, 8, 64, 4)  # [b, i, w, u, l, 4 words]
    expect = np.bitwise_xor.reduce(words, axis=(1, 3, 5))          # [b, w, l]
    assert np.array_equal(out.cpu().numpy().view(np.uint32), expect.reshape(-1))


def test_probe_stream_copy():
    n = 4 * 32768 * 5
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (n // 4,), dtype=torch.int32, device=DEV)
    dst = torch.zeros_like(src)
    lib = bl.abi.load_probe()
    bl.abi.check("probe", lib.bitlinear_probe_stream(src.data_ptr(), dst.data_ptr(), n, 5, None, stream()))
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_probe_mfma_deterministic():
    lib = bl.abi.load_probe()
    a = torch.empty(4 * 256, dtype=torch.int32, device=DEV)
    b = torch.empty_like(a)
    bl.abi.check("probe", lib.bitlinear_probe_mfma_i8(7, 4, a.data_ptr(), stream()))
    bl.abi.check("probe", lib.bitlinear_probe_mfma_i8(7, 4, b.data_ptr(), stream()))
    torch.cuda.synchronize()
    assert torch.equal(a, b) and bool((a != 0).any())


def test_probe_mfma_bf16_exact():
    """Small-integer bf16 operands: every product and partial sum is exact,
    so each thread's sum is a fixed value, the same on every call and equal
    to the plain matrix product's (operands rebuilt from the lane pattern)."""
    import numpy as np
    lib = bl.abi.load_probe()
    a = torch.empty(4 * 256, dtype=torch.float32, device=DEV)
    b = torch.empty_like(a)
    bl.abi.check("probe", lib.bitlinear_probe_mfma_bf16(5, 4, a.data_ptr(), stream()))
    bl.abi.check("probe", lib.bitlinear_probe_mfma_bf16(5, 4, b.data_ptr(), stream()))
    torch.cuda.synchronize()
    assert torch.equal(a, b) and bool((a != 0).any())
    # one 32x32x16 product: lane l holds A[l % 32][8 (l / 32) + i] and B[8 (l / 32) + i][l % 32]
    A = np.zeros((32, 16)); B = np.zeros((16, 32))
    for l in range(64):
        for i in range(8):
            A[l % 32, 8 * (l // 32) + i] = (l + i) & 3
            B[8 * (l // 32) + i, l % 32] = (3 * l + i) & 1
    C = A @ B  # lane l's 16 accumulator elements are 16 entries of column l % 32
    # thread sum = 8 accumulators x 5 iterations x (its 16 entries of C); the
    # total over a wave is 8 * 5 * C.sum()
    got = a.cpu().numpy().reshape(4, 4, 64).sum(axis=2)  # per wave
    assert np.allclose(got, 8 * 5 * C.sum())
