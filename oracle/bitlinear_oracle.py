"""Plain CPU oracle for the BitNet b1.58 BitLinear forward.

TEST INFRASTRUCTURE ONLY.  The tests, the package's smoke check and the
benchmark's CPU-baseline leg import this module; the product path never does,
and this module imports nothing from the product package.

It is written to be read against the pages, not to be fast: numpy in float32
where the method works in float32, float64/exact integers where it
accumulates, and pure-Python loops for the literal add/subtract/skip form.

Citations
---------
[PMV] is the produtoramaxvision.com.br blog article on BitNet b1.58 (ternary
quantisation, the BitLinear layer and Zero-GEMM).  Its sections:

* [PMV §1]  why 1.58 bits per weight: the AbsMean weight equations (gamma and
  the RoundClip to {-1, 0, +1}), the reconstruction W_hat = gamma * W_q, and the
  per-token AbsMax INT8 activation equations;
* [PMV §2]  how BitLinear removes multiplications (Zero-GEMM): add for +1,
  subtract for -1, skip for 0, INT32 accumulation, the worked 8-element
  example, and the single rescale of A_q x W_q^T by gamma_A * gamma / 127;
* [PMV §3]  the memory wall: 2-bit packing, 0.25 byte per weight;
* [PMV §4]  how bitnet.cpp speeds up CPU inference: the 81-entry LUT figure
  for four weights and the Radix-3 packing of five weights per byte;
* [PMV §6]  the trade-offs section: attention, SwiGLU-style activations and
  RMSNorm stay in floating point (or INT8).

[MBC] is the shadowgraph.io page on a hybrid multimodal architecture around
bitnet.cpp; its bit_layers.py section lists BitLinear, the ternary and 8-bit
quantisers and ReLU^2 as the activation BitNet specifies.

Readings where the article leaves a step open:

* eps = 1e-5 as a float32 constant, added in float32 (the article names an eps
  but not its value; 1e-5 is the value the lifelog blog's demo uses).
* "Round" is round-half-to-even (numpy ``rint``).
* gamma is per tensor, a float32 result of a float64 accumulation, read as:
  the sum of |W| is the float64 number nearest the exact sum (what an
  error-free float64 accumulation gives, i.e. ``math.fsum``), divided by N*K
  in float64, then rounded to float32.
* The activation scale is grouped as the article writes it:
  s = fp32(127 / fp32(gamma_A + eps)), then each code is rint(fp32(x * s)),
  clipped to [-128, 127].
* The dequantisation multiplies by gamma_A * gamma / 127 exactly as written
  (no eps there); this oracle forms it in float64 and rounds once to float32.
* The 2-bit layout is this library's own encoding (the article fixes only
  the size, two bits per weight): code c = q + 1 in {0, 1, 2}; rows padded to a
  multiple of 64 weights with c = 1 (a zero weight); row n is a run of
  little-endian 32-bit words, word j covers k in [16j, 16j + 16), and bits
  [8b + 2i, 8b + 2i + 1] of word j hold the code of k = 16j + 4i + b.
* The LUT contraction (a comparison to the matrix-core path) takes blocks of
  four consecutive activations; its table index is the base-3 number of the
  block's codes c = q + 1, first weight most significant, which is the digit
  order the LUT figure's rows 0 / 40 / 80 fix.
* Both packed formats (2-bit and radix-3) cut each row into 16-byte units and
  store the units of 16 consecutive rows interleaved: see
  :func:`interleave_units`.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against the article's worked example, brute force, ``math.fsum``, closed forms
or invariants; none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np

EPS32 = np.float32(1e-5)
PAD_MULTIPLE = 64  # packed rows hold a multiple of 64 weights


# ---------------------------------------------------------------------------
# a1: AbsMean scale  [PMV §1, AbsMean equation]
# ---------------------------------------------------------------------------

def exact_abs_sum_units(W: np.ndarray) -> int:
    """Exact sum of |W| as a Python integer in units of 2**-149.

    Every finite float32 magnitude is an integer significand times a power of
    two: |w| = Msig * 2**(s - 149) with s = max(e - 1, 0), where e is the
    biased exponent field and Msig includes the implicit bit for e >= 1.
    Significands are summed per exponent (float64 weights in ``bincount`` stay
    exact because every running total stays below 2**53 for < 2**29 values),
    then the bins are combined as exact Python integers.
    """
    a = np.ascontiguousarray(W, dtype=np.float32).ravel()
    if a.size >= (1 << 29):
        raise ValueError("exact_abs_sum_units: more than 2**29 values")
    if not np.all(np.isfinite(a)):
        raise ValueError("exact_abs_sum_units: non-finite weight")
    bits = a.view(np.uint32) & np.uint32(0x7FFFFFFF)
    e = (bits >> np.uint32(23)).astype(np.int64)
    m = (bits & np.uint32(0x7FFFFF)).astype(np.int64)
    sig = np.where(e > 0, m | (1 << 23), m)
    s = np.maximum(e - 1, 0)
    bins = np.bincount(s, weights=sig.astype(np.float64), minlength=254)
    total = 0
    for shift in np.nonzero(bins)[0]:
        total += int(bins[shift]) << int(shift)
    return total


def abs_sum_f64(W: np.ndarray) -> float:
    """The float64 number nearest the exact sum of |W| (round half to even)."""
    units = exact_abs_sum_units(W)
    return math.ldexp(float(units), -149) if units else 0.0


def absmean_gamma(W: np.ndarray) -> np.float32:
    """gamma = (1 / (n*m)) * sum |W_ij|  [PMV §1, AbsMean equation], per tensor.

    Accumulation: nearest float64 to the exact sum; float64 division by the
    element count; one rounding to float32.
    """
    W = np.asarray(W, dtype=np.float32)
    if W.size == 0:
        raise ValueError("absmean_gamma: empty weight matrix")
    return np.float32(abs_sum_f64(W) / float(W.size))


def absmean_gamma_fsum(W: np.ndarray) -> np.float32:
    """Same definition via ``math.fsum`` (correctly rounded float64 sum); small inputs only."""
    W = np.asarray(W, dtype=np.float32)
    vals = np.abs(W.astype(np.float64)).ravel().tolist()
    return np.float32(math.fsum(vals) / float(W.size))


# ---------------------------------------------------------------------------
# a2: RoundClip ternarisation and 2-bit packing  [PMV §1 RoundClip, §3 2-bit pack]
# ---------------------------------------------------------------------------

def ternary_codes(W: np.ndarray, gamma) -> np.ndarray:
    """W_q = Round(Clip(W / (gamma + eps), -1, 1)) in {-1, 0, +1}  [PMV §1].

    float32 throughout: d = fp32(gamma + eps), t = fp32(W / d) (IEEE division),
    clip to [-1, 1], round half to even.
    """
    W = np.asarray(W, dtype=np.float32)
    d = np.float32(np.float32(gamma) + EPS32)
    t = W / d
    assert t.dtype == np.float32
    c = np.clip(t, np.float32(-1.0), np.float32(1.0))
    return np.rint(c).astype(np.int8)


def padded_k(K: int) -> int:
    return ((K + PAD_MULTIPLE - 1) // PAD_MULTIPLE) * PAD_MULTIPLE


# ---------------------------------------------------------------------------
# Memory order of packed rows (this library's layout; the article fixes only
# the bits per weight).  A packed row is a run of U 16-byte units.  Rows are
# taken in blocks of 16 consecutive rows (the last block holds the N % 16 rows
# left over, if any) and a block's units in chunks of 4 consecutive units (the
# last chunk holds the U % 4 units left over, if any).  Blocks follow each
# other; within a block the chunks follow each other; within a chunk each row
# of the block, in order, stores its units of that chunk contiguously.  So 16
# full rows x 4 units make one contiguous 1 KiB piece, and a row block takes
# as many bytes as the same rows stored one after another.
# ---------------------------------------------------------------------------

ROW_BLOCK = 16
UNIT_CHUNK = 4


def interleave_units(rows: np.ndarray) -> np.ndarray:
    """Row-major units [N, U, 16] (uint8) -> the packed buffer as flat uint8, in memory order."""
    rows = np.asarray(rows, dtype=np.uint8)
    N, U, sixteen = rows.shape
    assert sixteen == 16
    out = []
    for b0 in range(0, N, ROW_BLOCK):
        R = min(ROW_BLOCK, N - b0)
        for c0 in range(0, U, UNIT_CHUNK):
            W = min(UNIT_CHUNK, U - c0)
            for j in range(R):
                out.append(rows[b0 + j, c0:c0 + W].reshape(-1))
    return np.concatenate(out) if out else np.zeros(0, np.uint8)


def deinterleave_units(flat: np.ndarray, N: int, U: int) -> np.ndarray:
    """Inverse of :func:`interleave_units`: flat uint8 buffer -> units [N, U, 16]."""
    flat = np.asarray(flat, dtype=np.uint8).reshape(-1)
    if flat.size != N * U * 16:
        raise ValueError("deinterleave_units: buffer size does not match N x U units")
    rows = np.empty((N, U, 16), dtype=np.uint8)
    pos = 0
    for b0 in range(0, N, ROW_BLOCK):
        R = min(ROW_BLOCK, N - b0)
        for c0 in range(0, U, UNIT_CHUNK):
            W = min(UNIT_CHUNK, U - c0)
            for j in range(R):
                rows[b0 + j, c0:c0 + W] = flat[pos:pos + 16 * W].reshape(W, 16)
                pos += 16 * W
    return rows


def pack_codes(q: np.ndarray) -> np.ndarray:
    """Pack ternary codes [N, K] into uint32 words [N, padded_k(K) // 16].

    Layout: see the module docstring; the returned array's memory order is
    the packed buffer (rows interleaved by :func:`interleave_units`), so only
    for N = 1 is row n of the array row n of the matrix.  0.25 byte per
    weight  [PMV §3].
    """
    q = np.asarray(q)
    N, K = q.shape
    Kp = padded_k(K)
    c = np.ones((N, Kp), dtype=np.uint32)
    c[:, :K] = (q.astype(np.int64) + 1).astype(np.uint32)
    c = c.reshape(N, Kp // 16, 4, 4)  # [n, word j, i, b] -> k = 16j + 4i + b
    words = np.zeros((N, Kp // 16), dtype=np.uint32)
    for i in range(4):
        for b in range(4):
            words |= c[:, :, i, b] << np.uint32(8 * b + 2 * i)
    # memory order: 16-byte units (four words) of 16-row blocks interleaved
    units = words.astype('<u4').view(np.uint8).reshape(N, Kp // 64, 16)
    return interleave_units(units).view('<u4').reshape(N, Kp // 16)


def unpack_codes(words: np.ndarray, K: int) -> np.ndarray:
    """Inverse of :func:`pack_codes`; returns int8 codes [N, K] (raises on field value 3)."""
    words = np.asarray(words, dtype=np.uint32)
    N, nw = words.shape
    if nw % 4:
        raise ValueError("unpack_codes: rows are not whole 16-byte units")
    units = deinterleave_units(words.astype('<u4').view(np.uint8), N, nw // 4)
    words = units.reshape(N, nw * 4).view('<u4').astype(np.uint32)
    out = np.empty((N, nw, 4, 4), dtype=np.int64)
    for i in range(4):
        for b in range(4):
            out[:, :, i, b] = (words >> np.uint32(8 * b + 2 * i)) & np.uint32(3)
    if np.any(out == 3):
        raise ValueError("unpack_codes: invalid 2-bit field (3)")
    return (out.reshape(N, nw * 16)[:, :K] - 1).astype(np.int8)


# ---------------------------------------------------------------------------
# Radix-3 packing: five ternary weights per byte  [PMV §4, Radix-3 packing]
# ---------------------------------------------------------------------------
#
# The article fixes the count (five weights per byte, 3^5 = 243 <= 256, 1.60
# bits per weight) and, through its LUT figure, that a group of ternary
# weights is indexed as a base-3 number of the offset digits c = q + 1 (all -1
# gives index 0, all 0 gives 40 and all +1 gives 80 for four weights).  The
# rest is this library's reading:
#
# * v = sum_t c_t * 3^(4-t) over the byte's five weights, first weight most
#   significant;
# * the byte stores v scaled to the byte range, ceil(256 * v / 243): a
#   one-to-one map of the 243 values (inverse v = floor(243 * byte / 256)),
#   chosen so that a decoder can read the digits most-significant first by
#   multiplying the byte, as a fraction of 256, by three;
# * a row of K weights is padded with c = 1 (zero weights) to a multiple of 80;
#   byte 4j + b of a row (b = 0..3) holds the weights k = 20j + 4t + b for
#   t = 0..4, so 16-byte units of a row cover 80 consecutive weights; rows are
#   interleaved in memory like the 2-bit format's (:func:`interleave_units`).

R3_UNIT = 80  # weights per 16 bytes of a radix-3 row
R3_DIGITS = 5


def r3_padded_k(K: int) -> int:
    return ((K + R3_UNIT - 1) // R3_UNIT) * R3_UNIT


def r3_packed_bytes(N: int, K: int) -> int:
    return N * r3_padded_k(K) // R3_DIGITS


def r3_value(c5) -> int:
    """Base-3 number of five offset codes c in {0,1,2}, the first most significant."""
    v = 0
    for c in c5:
        if c not in (0, 1, 2):
            raise ValueError("r3_value: offset code outside {0, 1, 2}")
        v = 3 * v + int(c)
    return v


def r3_byte(v: int) -> int:
    """Stored byte of the base-3 value v in [0, 242]: ceil(256 v / 243)."""
    if not 0 <= v <= 242:
        raise ValueError("r3_byte: value outside [0, 242]")
    return (256 * v + 242) // 243


def r3_value_of_byte(b: int) -> int:
    """Inverse of :func:`r3_byte`; raises for the 13 bytes that encode nothing."""
    v = (243 * int(b)) >> 8
    if r3_byte(v) != int(b):
        raise ValueError("r3_value_of_byte: byte %d is not a radix-3 encoding" % b)
    return v


def pack_codes_r3(q: np.ndarray) -> np.ndarray:
    """Pack ternary codes [N, K] into bytes [N, r3_padded_k(K) // 5] (layout above)."""
    q = np.asarray(q)
    N, K = q.shape
    Kp = r3_padded_k(K)
    c = np.ones((N, Kp), dtype=np.int64)
    c[:, :K] = q.astype(np.int64) + 1
    c = c.reshape(N, Kp // 20, R3_DIGITS, 4)  # [n, word j, digit t, byte b]: k = 20j + 4t + b
    v = np.zeros((N, Kp // 20, 4), dtype=np.int64)
    for t in range(R3_DIGITS):
        v = 3 * v + c[:, :, t, :]
    out = (256 * v + 242) // 243
    units = out.reshape(N, Kp // R3_UNIT, 16).astype(np.uint8)
    return interleave_units(units).reshape(N, Kp // R3_DIGITS)


def unpack_codes_r3(packed: np.ndarray, K: int) -> np.ndarray:
    """Inverse of :func:`pack_codes_r3`; int8 codes [N, K] (raises on a byte that encodes nothing)."""
    packed = np.asarray(packed, dtype=np.uint8)
    N, nb = packed.shape
    if nb % 16:
        raise ValueError("unpack_codes_r3: rows are not whole 16-byte units")
    b = deinterleave_units(packed, N, nb // 16).reshape(N, nb).astype(np.int64)
    v = (243 * b) >> 8
    if np.any((256 * v + 242) // 243 != b):
        raise ValueError("unpack_codes_r3: byte that is not a radix-3 encoding")
    v = v.reshape(N, nb // 4, 4)
    c = np.empty((N, nb // 4, R3_DIGITS, 4), dtype=np.int64)
    for t in range(R3_DIGITS - 1, -1, -1):  # least significant digit is the last weight
        c[:, :, t, :] = v % 3
        v = v // 3
    return (c.reshape(N, nb * R3_DIGITS)[:, :K] - 1).astype(np.int8)


# ---------------------------------------------------------------------------
# a3: per-token AbsMax INT8  [PMV §1, AbsMax equations]
# ---------------------------------------------------------------------------

def absmax_quantize(X: np.ndarray):
    """gamma_A = max_k |A_k| per token; A_q = Clip(Round(A * (127 / (gamma_A + eps))), -128, 127).

    Returns (gamma_A float32 [M], Xq int8 [M, K], rowsum int64 [M]) where rowsum
    is the exact sum of each token's codes.  float32 arithmetic, true division,
    round half to even.
    """
    X = np.asarray(X, dtype=np.float32)
    gA = np.max(np.abs(X), axis=1).astype(np.float32)
    den = (gA + EPS32).astype(np.float32)
    s = (np.float32(127.0) / den).astype(np.float32)
    v = X * s[:, None]
    assert v.dtype == np.float32
    Xq = np.clip(np.rint(v), -128, 127).astype(np.int8)
    return gA, Xq, Xq.astype(np.int64).sum(axis=1)


# ---------------------------------------------------------------------------
# a4/a5: Zero-GEMM contraction with INT32 accumulation  [PMV §2]
# ---------------------------------------------------------------------------

def zero_gemm_dot(xq, q) -> int:
    """One output, literally as the article's Zero-GEMM: +1 adds, -1 subtracts, 0 skips."""
    acc = 0
    for a, w in zip(xq, q):
        w = int(w)
        if w == 1:
            acc += int(a)
        elif w == -1:
            acc -= int(a)
        elif w != 0:
            raise ValueError("zero_gemm_dot: weight not ternary")
    if not -(1 << 31) <= acc < (1 << 31):
        raise OverflowError("zero_gemm_dot: INT32 accumulator overflow")
    return acc


def zero_gemm_naive(Xq: np.ndarray, q: np.ndarray) -> np.ndarray:
    """acc[m, n] = zero_gemm_dot(Xq[m], q[n]) for every pair (small inputs only)."""
    M, N = Xq.shape[0], q.shape[0]
    acc = np.empty((M, N), dtype=np.int64)
    for m in range(M):
        xr = Xq[m].tolist()
        for n in range(N):
            acc[m, n] = zero_gemm_dot(xr, q[n].tolist())
    return acc


def zero_gemm(Xq: np.ndarray, q: np.ndarray) -> np.ndarray:
    """acc = A_q x W_q^T as exact integers, via a float64 matrix product.

    Every partial sum is an integer of magnitude <= 128 * K < 2**53, so the
    float64 product is exact whatever order the library sums in.
    """
    Xq = np.asarray(Xq)
    q = np.asarray(q)
    K = Xq.shape[1]
    if 128 * K >= (1 << 53):
        raise ValueError("zero_gemm: K too large for an exact float64 contraction")
    acc = Xq.astype(np.float64) @ q.astype(np.float64).T
    return acc.astype(np.int64)


# ---------------------------------------------------------------------------
# a6: dequantisation  [PMV §2, rescale by gamma_A * gamma / 127]
# ---------------------------------------------------------------------------

def dequant(acc: np.ndarray, gamma, gamma_a: np.ndarray) -> np.ndarray:
    """Y[m, n] = acc[m, n] * gamma * gamma_A[m] / 127, formed in float64, rounded once to float32."""
    acc = np.asarray(acc, dtype=np.float64)
    g = float(np.float32(gamma))
    ga = np.asarray(gamma_a, dtype=np.float32).astype(np.float64)
    return (acc * g * ga[:, None] / 127.0).astype(np.float32)


# ---------------------------------------------------------------------------
# Whole forward
# ---------------------------------------------------------------------------

def quantize_weights(W: np.ndarray):
    """Offline half of BitLinear: (gamma, codes, packed words)."""
    gamma = absmean_gamma(W)
    q = ternary_codes(W, gamma)
    return gamma, q, pack_codes(q)


def bitlinear_forward(X: np.ndarray, W: np.ndarray) -> Dict[str, np.ndarray]:
    """Full BitLinear forward Y = dequant(A_q x W_q^T); returns every intermediate."""
    gamma, q, packed = quantize_weights(W)
    gA, Xq, rowsum = absmax_quantize(X)
    acc = zero_gemm(Xq, q)
    Y = dequant(acc, gamma, gA)
    return {"gamma": gamma, "q": q, "packed": packed, "gamma_a": gA, "Xq": Xq,
            "rowsum": rowsum, "acc": acc, "Y": Y}


def forward_from_codes(X: np.ndarray, q: np.ndarray, gamma) -> Dict[str, np.ndarray]:
    """Forward for already-ternarised weights (codes + gamma)."""
    gA, Xq, rowsum = absmax_quantize(X)
    acc = zero_gemm(Xq, q)
    return {"gamma_a": gA, "Xq": Xq, "rowsum": rowsum, "acc": acc,
            "Y": dequant(acc, gamma, gA)}


def sampled_forward(X: np.ndarray, q: np.ndarray, gamma, rows, cols) -> Dict[str, np.ndarray]:
    """Outputs for a subset of tokens (rows) and output channels (cols) only.

    Each token's quantisation depends only on that token, and each output only
    on one token and one weight row, so a sample is computed exactly as the
    full forward would compute it.
    """
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    gA, Xq, rowsum = absmax_quantize(np.asarray(X)[rows])
    acc = zero_gemm(Xq, np.asarray(q)[cols])
    return {"gamma_a": gA, "Xq": Xq, "rowsum": rowsum, "acc": acc,
            "Y": dequant(acc, gamma, gA)}


# ---------------------------------------------------------------------------
# BitNet FFN block: BitLinear up -> ReLU^2 -> BitLinear down
# [MBC bit_layers.py: ReLU^2 activation; PMV §6: non-linear parts in floating
# point; PMV §1 AbsMax: each BitLinear quantises its own input per token]
#
# Reading: the block is Y = BitLinear_down(ReLU^2(BitLinear_up(X))) with no
# norm inside (norms stay outside, in floating point).  The up projection's
# output H is formed in float32 as the kernels form every output:
# H = fp32(fp32(acc) * s), s = fp32(fp32(gamma * gamma_A) / 127).  Because H
# decides the INT8 codes of the down projection, both sides form it in that
# same precision; A = ReLU^2(H) = fp32(max(H, 0)^2).  The final Y is rescaled
# like any BitLinear output (float64, rounded once).
# ---------------------------------------------------------------------------

def dequant_f32(acc: np.ndarray, gamma, gamma_a: np.ndarray) -> np.ndarray:
    """H[m, n] = fp32(fp32(acc) * fp32(fp32(gamma * gamma_A[m]) / 127)): three float32 roundings."""
    acc = np.asarray(acc)
    g = np.float32(gamma)
    ga = np.asarray(gamma_a, dtype=np.float32)
    s = ((g * ga).astype(np.float32) / np.float32(127.0)).astype(np.float32)
    h = acc.astype(np.float32) * s[:, None]
    assert h.dtype == np.float32
    return h


def relu2(H: np.ndarray) -> np.ndarray:
    """ReLU^2 in float32: fp32(max(h, 0) * max(h, 0))  [MBC bit_layers.py]."""
    r = np.maximum(np.asarray(H, dtype=np.float32), np.float32(0.0))
    a = r * r
    assert a.dtype == np.float32
    return a + np.float32(0.0)  # -0.0 -> +0.0


def ffn_from_codes(X, q_up, g_up, q_down, g_down) -> Dict[str, np.ndarray]:
    """The FFN block from ternary codes and scales of both projections."""
    gA, Xq, rowsum = absmax_quantize(X)
    acc1 = zero_gemm(Xq, q_up)
    H = dequant_f32(acc1, g_up, gA)
    A = relu2(H)
    gA2, Aq, rowsum2 = absmax_quantize(A)
    acc2 = zero_gemm(Aq, q_down)
    Y = dequant(acc2, g_down, gA2)
    return {"gamma_a": gA, "Xq": Xq, "acc1": acc1, "H": H, "A": A, "gamma_a2": gA2, "Aq": Aq,
            "rowsum2": rowsum2, "acc2": acc2, "Y": Y}


def ffn_forward(X: np.ndarray, W_up: np.ndarray, W_down: np.ndarray) -> Dict[str, np.ndarray]:
    """Y = BitLinear_down(ReLU^2(BitLinear_up(X))); W_up [F, D], W_down [D_out, F]."""
    g_up, q_up, _ = quantize_weights(W_up)
    g_dn, q_dn, _ = quantize_weights(W_down)
    out = ffn_from_codes(X, q_up, g_up, q_dn, g_dn)
    out.update({"gamma_up": g_up, "q_up": q_up, "gamma_down": g_dn, "q_down": q_dn})
    return out


# ---------------------------------------------------------------------------
# Backward with the straight-through estimator (STE)
# [PMV §2, STE paragraph: in the backward pass the gradient of the quantiser is
# taken as the identity, dW_q/dW = 1, for values inside the valid range;
# MBC bit_layers.py: BitLinear trains with a straight-through estimator]
#
# Reading: the forward is Y = A_hat W_hat^T with A_hat = (gamma_A / 127) A_q
# and W_hat = gamma W_q.  Both quantisers pass gradients straight through
# inside their clip ranges: the activation clip [-128, 127] never binds
# (|x * s| <= 127), and the weight passes where |fp32(W / fp32(gamma + eps))|
# <= 1 (inside RoundClip), so
#     dX = dY W_hat,        dW = (dY^T A_hat) * 1[|W / (gamma + eps)| <= 1].
# gamma and gamma_A are treated as constants.  Gradients and A_hat are in the
# training precision, bfloat16: dY is given in bfloat16 and A_hat is rounded
# to bfloat16 from fp32(fp32(gamma_A / 127) * A_q); the contractions here are
# exact (float64 on these integers-times-bfloat16 products), rounded once.
# ---------------------------------------------------------------------------

def _to_bf16_values(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 values."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def dequant_activations_bf16(Xq: np.ndarray, gamma_a: np.ndarray) -> np.ndarray:
    """A_hat = bf16(fp32(fp32(gamma_A / 127) * A_q)) as float32 values [M, K]."""
    c = (np.asarray(gamma_a, np.float32) / np.float32(127.0)).astype(np.float32)
    a = c[:, None] * np.asarray(Xq).astype(np.float32)
    assert a.dtype == np.float32
    return _to_bf16_values(a)


def ste_weight_mask(W: np.ndarray, gamma) -> np.ndarray:
    """1 where the weight lies inside RoundClip's range: |fp32(W / fp32(gamma + eps))| <= 1."""
    d = np.float32(np.float32(gamma) + EPS32)
    t = np.asarray(W, np.float32) / d
    assert t.dtype == np.float32
    return (np.abs(t) <= np.float32(1.0))


def pack_mask_bits(mask: np.ndarray) -> np.ndarray:
    """The range mask [N, K] as bits: uint32 [N, ceil(K / 32)], bit k % 32 of
    word k // 32 of row n is mask[n, k]; bits past K are 0.  (A storage format
    of this library: the mask depends only on W and gamma, so it is formed
    once per weight update next to the transposed codes.)"""
    mask = np.asarray(mask, dtype=bool)
    N, K = mask.shape
    Kw = -(-K // 32)
    bits = np.zeros((N, Kw * 32), dtype=np.uint64)
    bits[:, :K] = mask
    shifts = np.arange(32, dtype=np.uint64)
    words = (bits.reshape(N, Kw, 32) << shifts).sum(axis=2)
    return words.astype(np.uint32)


def unpack_mask_bits(words: np.ndarray, K: int) -> np.ndarray:
    """Inverse of pack_mask_bits: bool [N, K]."""
    words = np.asarray(words, dtype=np.uint32)
    N, Kw = words.shape
    bits = (words[:, :, None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)
    return bits.reshape(N, Kw * 32)[:, :K].astype(bool)


def ste_backward(dY: np.ndarray, q: np.ndarray, gamma, Xq: np.ndarray, gamma_a: np.ndarray,
                 W: np.ndarray) -> Dict[str, np.ndarray]:
    """dX [M, K] and dW [N, K] (float32) of the forward Y = A_hat W_hat^T under the STE.

    dY: [M, N] bfloat16 values (as float32); q: ternary codes [N, K]; gamma: the
    weight scale; Xq, gamma_a: the forward's activation codes and scales; W: the
    float32 weights (for the range mask).
    """
    dY = np.asarray(dY, np.float32).astype(np.float64)
    q64 = np.asarray(q).astype(np.float64)
    dX = (dY @ q64) * float(np.float32(gamma))
    A_hat = dequant_activations_bf16(Xq, gamma_a).astype(np.float64)
    mask = ste_weight_mask(W, gamma)
    dW = (dY.T @ A_hat) * mask
    return {"dX": dX.astype(np.float32), "dW": dW.astype(np.float32), "A_hat": A_hat.astype(np.float32),
            "mask": mask}


# ---------------------------------------------------------------------------
# LUT GEMV (the CPU prior art, as a comparison)  [PMV §4, LUT-GEMM figure]
# ---------------------------------------------------------------------------

LUT_GROUP = 4     # activations per table
LUT_ENTRIES = 81  # 3**4 sign patterns of four ternary weights


def lut_index(c4) -> int:
    """Table index of four weight codes c_t = q_t + 1: the base-3 number c_0 c_1 c_2 c_3.

    c_0 is the most significant digit, which puts all -1 at index 0, all 0 at
    40 and all +1 at 80, the three rows the LUT figure prints.
    """
    idx = 0
    for c in c4:
        c = int(c)
        if c not in (0, 1, 2):
            raise ValueError("lut_index: code outside {0, 1, 2}")
        idx = 3 * idx + c
    return idx


def lut_digits(idx: int):
    """The four base-3 digits (c_0 first) of a table index in [0, 81)."""
    if not 0 <= idx < LUT_ENTRIES:
        raise ValueError("lut_digits: index outside [0, 81)")
    out = []
    for _ in range(LUT_GROUP):
        out.append(idx % 3)
        idx //= 3
    return out[::-1]


def lut_table(a4) -> np.ndarray:
    """The 81 pre-sums of four INT8 activations: T[idx] = sum_t (c_t - 1) * a_t (int64 [81])."""
    a = [int(x) for x in a4]
    if len(a) != LUT_GROUP:
        raise ValueError("lut_table: needs four activations")
    T = np.empty(LUT_ENTRIES, np.int64)
    for idx in range(LUT_ENTRIES):
        T[idx] = sum((c - 1) * x for c, x in zip(lut_digits(idx), a))
    return T


def lut_gemv(Xq: np.ndarray, q: np.ndarray) -> np.ndarray:
    """acc = A_q x W_q^T formed the LUT way: one 81-entry table per token and block of 4 activations.

    K is split into blocks of 4 consecutive positions (the last one padded with
    zero activations and zero weights).  For every token and block the table
    of pre-sums is built once; every weight row then reads, per block, the
    entry its four codes index, and the entries are summed in INT32.
    """
    Xq = np.asarray(Xq, np.int64)
    q = np.asarray(q, np.int64)
    M, K = Xq.shape
    N = q.shape[0]
    Kg = -(-K // LUT_GROUP) * LUT_GROUP
    G = Kg // LUT_GROUP
    Xp = np.zeros((M, Kg), np.int64)
    Xp[:, :K] = Xq
    cp = np.ones((N, Kg), np.int64)  # code 1 = weight 0 in the padding
    cp[:, :K] = q + 1
    if cp.min(initial=1) < 0 or cp.max(initial=1) > 2:
        raise ValueError("lut_gemv: weights not ternary")
    idx = np.zeros((N, G), np.int64)
    for t in range(LUT_GROUP):  # base-3 number of the block's codes, c_0 first
        idx = 3 * idx + cp[:, t::LUT_GROUP]
    acc = np.zeros((M, N), np.int64)
    blocks = np.arange(G)
    for m in range(M):
        tables = np.stack([lut_table(Xp[m, LUT_GROUP * g:LUT_GROUP * (g + 1)]) for g in range(G)])
        acc[m] = tables[blocks[None, :], idx].sum(axis=1)
    if acc.size and (acc.min() < -(1 << 31) or acc.max() >= (1 << 31)):
        raise OverflowError("lut_gemv: INT32 accumulator overflow")
    return acc


def lut_forward(X: np.ndarray, q: np.ndarray, gamma) -> Dict[str, np.ndarray]:
    """Forward with the LUT contraction: quantise tokens, lut_gemv, dequantise."""
    gA, Xq, rowsum = absmax_quantize(X)
    acc = lut_gemv(Xq, q)
    return {"gamma_a": gA, "Xq": Xq, "rowsum": rowsum, "acc": acc, "Y": dequant(acc, gamma, gA)}
