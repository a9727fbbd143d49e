"""The prefill GEMM's operand addressing, replayed on the host.

The GEMM reads its two code arrays through buffer resources whose size is the
array's size; a load whose lane offset (plus the instruction's immediate) is
past the size reads zeros, and that is how rows past M or N stay in bounds.
The scalar offset of a buffer load is not part of that range check, so the
whole offset must be in the lane offset.  This test repeats the kernel's
tile placement and its per-thread offset arithmetic (set_tile / gload in
csrc/prefill.hip, and the tile choice of launch_prefill_gemm) for ragged
shapes and checks, for every load of every stage of every tile:

* a load of a real row (token < M, weight row < N) lies inside its array;
* a load of a row past the end has a lane offset at or past the array's size,
  so it reads zeros.

No GPU is used.
"""
import numpy as np
import pytest

BK = 128
KCUS = 256


def padded_k(K):
    return (K + 63) // 64 * 64


def tile_launches(M, N):
    """The (BM, BN, WM, WN, n0, ncols) launches of launch_prefill_gemm for M x N."""
    def tiles(bm, bn):
        return ((M + bm - 1) // bm) * ((N + bn - 1) // bn)
    big = tiles(256, 256)
    rounds, rest = big // KCUS, big % KCUS
    if 1 <= rounds < 4 and rest > 0 and rest * 4 < 3 * KCUS:
        tm_big, tm_half = (M + 255) // 256, (M + 127) // 128
        nA = (rounds * KCUS // tm_big) * 256
        while nA > 0 and tm_half * ((N - nA + 255) // 256) > KCUS:
            nA -= 256
        if 0 < nA < N:
            return [(256, 256, 4, 2, 0, nA), (128, 256, 2, 4, nA, N - nA)]
    if big >= 192:
        return [(256, 256, 4, 2, 0, N)]
    if tiles(128, 256) >= 192:
        return [(128, 256, 2, 4, 0, N)]
    return [(128, 128, 2, 2, 0, N)]


def place(t, tiles_m, tiles_n, BM, BN, group=8):
    num = tiles_m * tiles_n
    if num % 8 == 0:
        t = (t & 7) * (num >> 3) + (t >> 3)
    g = t // (group * tiles_n)
    first_m = g * group
    gsize = min(tiles_m - first_m, group)
    in_group = t - g * group * tiles_n
    return (first_m + in_group % gsize) * BM, (in_group // gsize) * BN


def replay(M, K, N):
    """Check every activation and packed-code load of the prefill GEMM."""
    Kp = padded_k(K)
    units = Kp // 64
    niter = (Kp + BK - 1) // BK
    checked = 0
    for BM, BN, WM, WN, ncol0, Ncols in tile_launches(M, N):
        threads = 64 * WM * WN
        tid = np.arange(threads, dtype=np.int64)
        a_r, a_c = tid >> 3, tid & 7
        b_r, b_c = tid >> 1, tid & 1
        a_loads = BM * 8 // threads
        a_row_step = (threads // 8) * Kp
        # tokens are run in chunks of < 2^31 code bytes (32-bit offsets)
        chunk = ((1 << 31) - 1) // Kp // BM * BM
        bytes_b = Ncols * (Kp // 4)
        assert bytes_b < (1 << 31)
        for r0 in range(0, M, chunk):
            Mc = min(M - r0, chunk)
            bytes_a = Mc * Kp
            assert bytes_a < (1 << 31)
            tiles_m, tiles_n = (Mc + BM - 1) // BM, (Ncols + BN - 1) // BN
            for t in range(tiles_m * tiles_n):
                m0, n0 = place(t, tiles_m, tiles_n, BM, BN)
                voff_a = (m0 + a_r) * Kp + 16 * a_c
                b_n = n0 + b_r
                b_ok = b_n < Ncols
                b_blk = np.where(b_ok, (b_n & ~15) * units * 16, 0x80000000)
                b_j = np.where(b_ok, b_n & 15, 0)
                b_R = np.where(b_ok, np.minimum(16, Ncols - (b_n & ~15)), 0)
                for it in range(niter):
                    k0 = it * BK
                    a_adj = np.where(k0 + 16 * a_c >= Kp, 64, 0)
                    a_base = voff_a + k0 - a_adj
                    for q in range(a_loads):
                        off = a_base + q * a_row_step   # lane offset: all of it
                        assert off.max() < (1 << 32)    # no 32-bit wrap
                        row = m0 + a_r + (threads // 8) * q
                        ok = row < Mc
                        assert np.all(off[ok] + 16 <= bytes_a), (M, K, N, BM, t, it, q)
                        assert np.all(off[ok] >= 0)
                        # the loaded k range is that of this slot (or, in a final
                        # half stage, the 64 codes before it)
                        assert np.all(off[ok] // Kp == row[ok])
                        assert np.all(off[~ok] >= bytes_a), (M, K, N, BM, t, it, q)
                        checked += int(ok.sum())
                    u = 2 * it + b_c
                    u = np.where(u >= units, u - 1, u)
                    cu = u >> 2
                    W = np.minimum(4, units - 4 * cu)
                    voff_b = b_blk + (cu * b_R * 4 + b_j * W + (u & 3)) * 16
                    assert np.all(voff_b[b_ok] + 16 <= bytes_b)
                    assert np.all(voff_b[~b_ok] >= bytes_b)
                    assert voff_b.max() < (1 << 32)
    return checked


@pytest.mark.parametrize("M,K,N", [
    (20, 1 << 20, 50),      # 128 x 128 tiles, K = 2^20: rows 20..127 of the tile are past M
    (2000, 4096, 700),      # ragged last tile of 256 x 256 tiles
    (40, 200, 130),         # a half K stage and ragged M and N
    (2000, 1050, 6200),     # ragged M and N, half K stage, several tile rounds
    (2048, 200, 11000),     # the two-launch column split, ragged N in the second launch
    (300, 520, 600),
])
def test_prefill_load_offsets_stay_in_bounds(M, K, N):
    assert replay(M, K, N) > 0


def test_row_step_in_scalar_offset_would_escape():
    """The check above does catch the original mistake: with the row step in
    the scalar offset, only the lane offset is compared with the size, and
    rows past M at q >= 1 pass the check while addressing memory past the
    array.  Replaying that form for M = 20, K = 2^20 finds such loads."""
    M, K, N = 20, 1 << 20, 50
    Kp = padded_k(K)
    BM, threads = 128, 256
    tid = np.arange(threads)
    a_r, a_c = tid >> 3, tid & 7
    voff = a_r * Kp + 16 * a_c
    bytes_a = M * Kp
    escaped = 0
    for q in range(BM * 8 // threads):
        row = a_r + (threads // 8) * q
        lane_ok = voff + 16 <= bytes_a            # what the hardware compares
        real = voff + q * (threads // 8) * Kp     # where the load would go
        escaped += int(np.sum(lane_ok & (row >= M) & (real + 16 > bytes_a)))
    assert escaped > 0
