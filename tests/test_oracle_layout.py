"""Pins for the memory order of packed rows (16-row blocks, 4-unit chunks).

The layout is the library's own: the article on BitNet b1.58 fixes only the
bits per weight (its memory-wall section for 2 bits, its bitnet.cpp section
for radix-3).  Pinned by hand-worked orders, a closed-form address that is
computed differently from the oracle's loops, and invariants.  CPU only.
"""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tagged(N, U):
    """Units whose 16 bytes name their (row, unit): bytes 0-1 row, 2-3 unit."""
    rows = np.zeros((N, U, 16), np.uint8)
    for n in range(N):
        for u in range(U):
            rows[n, u, 0:2] = [n & 255, n >> 8]
            rows[n, u, 2:4] = [u & 255, u >> 8]
            rows[n, u, 4] = 0xA5
    return rows


def order(flat):
    units = flat.reshape(-1, 16)
    return [[int(a[0]) | int(a[1]) << 8, int(a[2]) | int(a[3]) << 8] for a in units]


def closed_form_offset(n, u, N, U):
    """Byte offset of unit u of row n, as the kernels compute it."""
    b, j = divmod(n, 16)
    c, g = divmod(u, 4)
    R = min(16, N - 16 * b)
    W = min(4, U - 4 * c)
    return 16 * b * U * 16 + c * R * 64 + j * W * 16 + g * 16


def test_hand_worked_orders():
    with open(os.path.join(GOLDEN, "interleave_order.json")) as f:
        g = json.load(f)
    assert order(O.interleave_units(tagged(3, 5))) == g["N3_U5"]
    assert order(O.interleave_units(tagged(18, 2))) == g["N18_U2"]


@pytest.mark.parametrize("N,U", [(1, 1), (1, 7), (3, 5), (16, 4), (17, 9), (33, 8), (40, 13), (5, 3)])
def test_closed_form_address_and_round_trip(N, U):
    rows = tagged(N, U)
    flat = O.interleave_units(rows)
    assert flat.size == N * U * 16
    for n in range(N):
        for u in range(U):
            off = closed_form_offset(n, u, N, U)
            assert np.array_equal(flat[off:off + 16], rows[n, u]), (n, u)
    assert np.array_equal(O.deinterleave_units(flat, N, U), rows)


def test_single_row_is_row_major_and_full_chunks_are_contiguous():
    rows = tagged(1, 11)
    assert np.array_equal(O.interleave_units(rows), rows.reshape(-1))
    # 16 rows x 4 units = one contiguous KiB per chunk, rows in order
    rows = tagged(32, 8)
    flat = O.interleave_units(rows)
    for blk in range(2):
        for c in range(2):
            piece = flat[(blk * 2 + c) * 1024:(blk * 2 + c + 1) * 1024]
            assert np.array_equal(piece.reshape(16, 4, 16), rows[16 * blk:16 * blk + 16, 4 * c:4 * c + 4])


def test_blocks_keep_their_rows_bytes_together():
    N, U = 37, 6
    rows = tagged(N, U)
    flat = O.interleave_units(rows)
    for b0 in range(0, N, 16):
        R = min(16, N - b0)
        span = flat[b0 * U * 16:(b0 + R) * U * 16]
        assert sorted(map(tuple, order(span))) == [(n, u) for n in range(b0, b0 + R) for u in range(U)]


def test_packed_formats_use_the_layout():
    rng = np.random.default_rng(4)
    q = rng.integers(-1, 2, size=(19, 300)).astype(np.int8)
    # 2-bit: units are four words of 16 weights
    words = O.pack_codes(q)
    per_row = O.pack_codes(q[5:6])  # a single row is stored row-major
    flat = words.view(np.uint8).reshape(-1)
    U = O.padded_k(300) // 64
    for u in range(U):
        off = closed_form_offset(5, u, 19, U)
        assert np.array_equal(flat[off:off + 16], per_row.view(np.uint8).reshape(-1)[16 * u:16 * u + 16])
    # radix-3: units are 16 bytes of 80 weights
    p3 = O.pack_codes_r3(q)
    one = O.pack_codes_r3(q[18:19]).reshape(-1)
    U3 = O.r3_padded_k(300) // 80
    for u in range(U3):
        off = closed_form_offset(18, u, 19, U3)
        assert np.array_equal(p3.reshape(-1)[off:off + 16], one[16 * u:16 * u + 16])
    assert np.array_equal(O.unpack_codes(words, 300), q) and np.array_equal(O.unpack_codes_r3(p3, 300), q)
