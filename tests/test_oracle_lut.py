"""Pins for the oracle's LUT contraction (the CPU prior art, kept as a comparison).

[PMV §4] = the section of the produtoramaxvision.com.br article on BitNet b1.58
about how bitnet.cpp speeds up CPU inference.  Its LUT-GEMM figure: a block of
four INT8 activations has 3^4 = 81 ternary weight combinations, a table of 81
pre-sums is built, and the packed weights index it; three rows are printed
(index 0 = all -1, 40 = all 0, 80 = all +1), stored in
``tests/golden/lut_figure.json``.  The pins fix the table against those rows,
against an enumeration of the sign patterns by a different mechanism
(itertools.product), against symmetry and range invariants, and the whole LUT
contraction against the plain definition and the article's worked Zero-GEMM
example.  CPU only.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_figure_sizes():
    g = _load("lut_figure.json")
    assert O.LUT_GROUP == g["group"] == 4
    assert O.LUT_ENTRIES == g["entries"] == 3 ** 4


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_figure_rows(seed):
    a = np.random.default_rng(seed).integers(-127, 128, size=4)
    T = O.lut_table(a)
    for row in _load("lut_figure.json")["printed_rows"]:
        signs = row["signs"]
        assert O.lut_index([s + 1 for s in signs]) == row["index"]
        assert T[row["index"]] == sum(s * int(x) for s, x in zip(signs, a))


def test_enumeration_order():
    """itertools.product over (-1, 0, 1) enumerates the sign patterns with the
    first weight most significant: position i of that enumeration is index i."""
    a = [17, -90, 3, 127]
    T = O.lut_table(a)
    for i, signs in enumerate(itertools.product((-1, 0, 1), repeat=4)):
        assert O.lut_index([s + 1 for s in signs]) == i
        assert list(O.lut_digits(i)) == [s + 1 for s in signs]
        assert T[i] == int(np.dot(signs, a))


def test_negation_symmetry_and_range():
    rng = np.random.default_rng(5)
    for _ in range(50):
        a = rng.integers(-127, 128, size=4)
        T = O.lut_table(a)
        assert np.array_equal(T[::-1], -T)  # flipping every weight negates the pre-sum
        assert T[40] == 0
    T = O.lut_table([127, -127, 127, -127])
    assert T.max() == 508 and T.min() == -508  # fits int16 for codes in [-127, 127]


def test_index_rejects_non_ternary():
    with pytest.raises(ValueError):
        O.lut_index([0, 1, 3, 1])
    with pytest.raises(ValueError):
        O.lut_digits(81)


def test_worked_example():
    g = _load("zero_gemm_worked_example.json")
    x = np.array([g["activations_int8"]], np.int8)
    w = np.array([g["ternary_weights"]], np.int8)
    acc = O.lut_gemv(x, w)
    assert acc.shape == (1, 1) and int(acc[0, 0]) == g["running_accumulator"][-1] == -149


@pytest.mark.parametrize("M,K,N", [(1, 4, 3), (2, 9, 5), (3, 30, 7), (1, 63, 4)])
def test_matches_add_subtract_skip(M, K, N):
    rng = np.random.default_rng(M * 1000 + K)
    Xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    q = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    assert np.array_equal(O.lut_gemv(Xq, q), O.zero_gemm_naive(Xq, q))


@pytest.mark.parametrize("M,K,N", [(8, 2048, 64), (4, 257, 33), (16, 1026, 17), (1, 5, 1)])
def test_matches_definition(M, K, N):
    rng = np.random.default_rng(K)
    Xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    q = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    assert np.array_equal(O.lut_gemv(Xq, q), O.zero_gemm(Xq, q))


def test_lut_forward_equals_forward():
    rng = np.random.default_rng(11)
    X = rng.standard_normal((3, 200)).astype(np.float32)
    W = (rng.standard_normal((40, 200)) * 0.02).astype(np.float32)
    gamma = O.absmean_gamma(W)
    q = O.ternary_codes(W, gamma)
    a = O.lut_forward(X, q, gamma)
    b = O.forward_from_codes(X, q, gamma)
    for k in ("acc", "Y", "Xq", "gamma_a"):
        assert np.array_equal(a[k], b[k]), k
