"""Pins for the oracle's radix-3 packing (five ternary weights per byte).

[PMV §4] = the section of the produtoramaxvision.com.br article on BitNet b1.58
about how bitnet.cpp speeds up CPU inference: its LUT-GEMM figure (a group of
ternary weights indexed as a base-3 number of c = q + 1) and its Radix-3
packing (3^5 = 243 <= 256, 1.60 bits per weight, 94.9% of the byte's states).
The byte encoding (ceil(256 v / 243)) and the row layout are this library's
reading; the pins below fix them by hand-worked values, brute force over all
243 values and invariants.  CPU only.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "radix3_byte.json")) as f:
        return json.load(f)


def _digits_by_divmod(v):
    out = []
    for _ in range(5):
        out.append(v % 3)
        v //= 3
    return out[::-1]


def test_lut_figure_indices():
    g = _golden()["figure_index_four_weights"]
    assert O.r3_value([0, 0, 0, 0]) == g["all_minus_one"]
    assert O.r3_value([1, 1, 1, 1]) == g["all_zero"]
    assert O.r3_value([2, 2, 2, 2]) == g["all_plus_one"]
    # the 81 four-weight indices are exactly 0..80
    vals = sorted(O.r3_value(c) for c in itertools.product(range(3), repeat=4))
    assert vals == list(range(81))


def test_density_closed_forms():
    g = _golden()
    assert 3 ** 5 == 243 <= 256
    assert round(100 * 243 / 256, 1) == g["state_fraction_percent"]
    for N, K in [(1, 80), (3, 160), (7, 2080)]:
        assert O.r3_packed_bytes(N, K) * 8 / (N * K) == g["bits_per_weight"]
    # ragged K pads to a multiple of 80 weights, 16 bytes per 80
    assert O.r3_padded_k(1) == 80 and O.r3_padded_k(80) == 80 and O.r3_padded_k(81) == 160
    assert O.r3_packed_bytes(2, 2048) == 2 * 26 * 16


def test_hand_worked_byte():
    h = _golden()["hand_worked_byte"]
    c = [q + 1 for q in h["ternary"]]
    assert c == h["offset_digits"]
    assert O.r3_value(c) == h["value"]
    assert O.r3_byte(h["value"]) == h["byte"]
    assert O.r3_value_of_byte(h["byte"]) == h["value"]
    q = np.zeros((1, 20), dtype=np.int8)
    q[0, [0, 4, 8, 12, 16]] = h["ternary"]  # byte 0 holds k = 0, 4, 8, 12, 16
    p = O.pack_codes_r3(q)
    assert p.shape == (1, 16)
    assert p[0, 0] == h["byte"]
    assert np.all(p[0, 1:] == O.r3_byte(121))  # all-zero weights and padding


def test_encoding_is_one_to_one():
    bytes_ = [O.r3_byte(v) for v in range(243)]
    assert len(set(bytes_)) == 243 and min(bytes_) == 0 and max(bytes_) == 255
    assert bytes_ == sorted(bytes_)
    for v, b in enumerate(bytes_):
        assert O.r3_value_of_byte(b) == v
    unused = sorted(set(range(256)) - set(bytes_))
    assert len(unused) == 13
    for b in unused:
        with pytest.raises(ValueError):
            O.r3_value_of_byte(b)
    with pytest.raises(ValueError):
        O.r3_byte(243)


def test_digits_come_out_by_multiplying_by_three():
    # The property a decoder relies on: read the byte as a fraction of 256;
    # multiplying by 3 gives the next digit (most significant first) above
    # bit 8 and the rest below it.  Brute force over every value.
    def chain(b):
        out, r = [], b
        for _ in range(5):
            y = 3 * r
            out.append(y >> 8)
            r = y & 255
        return out

    for v in range(243):
        assert chain(O.r3_byte(v)) == _digits_by_divmod(v)
    # the ceiling matters: flooring breaks the property for almost every value
    assert sum(chain((256 * v) // 243) != _digits_by_divmod(v) for v in range(243)) == 242


@pytest.mark.parametrize("K", [1, 4, 19, 20, 21, 79, 80, 81, 160, 333, 2048])
def test_round_trip_and_agreement_with_2bit(K):
    rng = np.random.default_rng(K)
    q = rng.integers(-1, 2, size=(5, K)).astype(np.int8)
    p = O.pack_codes_r3(q)
    assert p.dtype == np.uint8 and p.shape == (5, O.r3_padded_k(K) // 5)
    assert np.array_equal(O.unpack_codes_r3(p, K), q)
    assert np.array_equal(O.unpack_codes_r3(p, K), O.unpack_codes(O.pack_codes(q), K))
    # the padded tail decodes to zero weights
    Kp = O.r3_padded_k(K)
    assert np.all(O.unpack_codes_r3(p, Kp)[:, K:] == 0)


def test_single_weight_positions():
    # one +1 at k sets digit t = (k % 20) // 4 of byte 4 (k // 20) + k % 4
    K = 160
    for k in range(K):
        q = np.zeros((1, K), dtype=np.int8)
        q[0, k] = 1
        p = O.pack_codes_r3(q)
        want = np.full(K // 5, O.r3_byte(121), dtype=np.uint8)
        t = (k % 20) // 4
        want[4 * (k // 20) + k % 4] = O.r3_byte(121 + 3 ** (4 - t))
        assert np.array_equal(p[0], want), k


def test_negation_mirrors_value():
    # q -> -q maps c -> 2 - c, so v -> 242 - v
    rng = np.random.default_rng(7)
    q = rng.integers(-1, 2, size=(3, 100)).astype(np.int8)
    a = O.pack_codes_r3(q).astype(np.int64)
    b = O.pack_codes_r3(-q).astype(np.int64)
    va = (243 * a) >> 8
    vb = (243 * b) >> 8
    assert np.all(va + vb == 242)


def test_invalid_bytes_raise():
    p = np.full((1, 16), O.r3_byte(121), dtype=np.uint8)
    p[0, 3] = 1  # encodes nothing
    with pytest.raises(ValueError):
        O.unpack_codes_r3(p, 80)
