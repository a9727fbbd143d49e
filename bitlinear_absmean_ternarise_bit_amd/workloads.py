"""Seeded synthetic inputs for the BitLinear forward.

This module holds no part of the method's arithmetic: it only draws weights and
activations (and casts fp32 activations to bfloat16 bit patterns) so that the
HIP path and the CPU oracle see byte-identical inputs.  It imports neither.

Recipe (one ``numpy.random.default_rng(seed)`` per workload, seed 0 unless
stated; draw order: W, then X, then any row/channel/token selections):

* W = float32(sigma * standard_normal(N, K)) drawn in float64, rounded once.
* FFN blocks (BitLinear up -> ReLU^2 -> BitLinear down) reuse a projection
  workload's X and W as X and W_up, and draw W_down [D, F] with the same sigma
  from a second generator, ``default_rng(seed + 1)``.
* X = float32 draws of shape (M, K); when the workload runs in bfloat16 the
  float32 values are rounded to bfloat16 with round-half-to-even.

Shapes follow the model sizes the BitNet b1.58 article (produtoramaxvision.com.br,
section on the memory wall, table of weight bytes per model size) reasons
about: a d_model-2048 projection, a 2048 -> 5632 FFN up-projection, a 7B-like
4096 -> 11008 FFN and a 70B-like 8192 -> 28672 FFN.  No public dataset is used;
these seeded draws stand in for real activations and trained weights.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_workload",
    "FfnWorkload",
    "FFN_WORKLOADS",
    "make_ffn_workload",
    "random_problem",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round half to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One seeded problem instance.

    ``X`` is always the float32 view the method quantises: for bfloat16
    workloads it is the exact widening of ``X_bf16_bits``.
    """

    name: str
    M: int
    K: int
    N: int
    W: np.ndarray  # float32 [N, K]
    X: np.ndarray  # float32 [M, K]
    x_dtype: str  # "f32" or "bf16"
    X_bf16_bits: Optional[np.ndarray] = None  # uint16 [M, K] when x_dtype == "bf16"
    notes: dict = field(default_factory=dict)


def _finish_x(x32: np.ndarray, x_dtype: str):
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if x_dtype == "f32":
        return x32, None
    if x_dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return bf16_bits_to_f32(bits), bits
    raise ValueError(f"unknown x_dtype {x_dtype!r}")


def _gauss_w(rng, N, K, sigma):
    return (sigma * rng.standard_normal((N, K))).astype(np.float32)


def _single_m4_k256_n128(seed=0):
    rng = np.random.default_rng(seed)
    M, K, N = 4, 256, 128
    W = _gauss_w(rng, N, K, 0.02)
    X, bits = _finish_x(rng.standard_normal((M, K)), "f32")
    return Workload("single_m4_k256_n128", M, K, N, W, X, "f32", bits)


def _decode_m1_k2048_n2048(seed=0):
    rng = np.random.default_rng(seed)
    M, K, N = 1, 2048, 2048
    W = _gauss_w(rng, N, K, 0.02)
    X, bits = _finish_x(rng.standard_normal((M, K)), "bf16")
    return Workload("decode_m1_k2048_n2048", M, K, N, W, X, "bf16", bits)


def _decode_ffn_up_m8_k2048_n5632(seed=0):
    rng = np.random.default_rng(seed)
    M, K, N = 8, 2048, 5632
    W = _gauss_w(rng, N, K, 0.02)
    x = rng.standard_normal((M, K))
    ch = rng.choice(K, size=K // 100, replace=False)  # 1% of channels
    x[:, ch] *= 20.0
    X, bits = _finish_x(x, "bf16")
    return Workload("decode_ffn_up_m8_k2048_n5632", M, K, N, W, X, "bf16", bits,
                    {"outlier_channels": np.sort(ch)})


def _prefill_ffn_m2048_k4096_n11008(seed=0):
    rng = np.random.default_rng(seed)
    M, K, N = 2048, 4096, 11008
    W = _gauss_w(rng, N, K, 0.015)
    X, bits = _finish_x(rng.standard_t(4, size=(M, K)), "bf16")
    return Workload("prefill_ffn_m2048_k4096_n11008", M, K, N, W, X, "bf16", bits)


def _prefill_ffn_m8192_k8192_n28672(seed=0):
    rng = np.random.default_rng(seed)
    M, K, N = 8192, 8192, 28672
    W = _gauss_w(rng, N, K, 0.01)
    x = rng.standard_normal((M, K))
    rows = rng.permutation(N)[: N // 2]
    W[rows, :] = 0.0
    tok = rng.choice(M, size=M // 100, replace=False)  # 1% outlier tokens
    x[tok, :] *= 100.0
    X, bits = _finish_x(x, "bf16")
    return Workload("prefill_ffn_m8192_k8192_n28672", M, K, N, W, X, "bf16", bits,
                    {"zero_rows": np.sort(rows), "outlier_tokens": np.sort(tok)})


WORKLOADS = {
    "single_m4_k256_n128": _single_m4_k256_n128,
    "decode_m1_k2048_n2048": _decode_m1_k2048_n2048,
    "decode_ffn_up_m8_k2048_n5632": _decode_ffn_up_m8_k2048_n5632,
    "prefill_ffn_m2048_k4096_n11008": _prefill_ffn_m2048_k4096_n11008,
    "prefill_ffn_m8192_k8192_n28672": _prefill_ffn_m8192_k8192_n28672,
}


def make_workload(name: str, seed: int = 0) -> Workload:
    """Build one of the named workloads (see module docstring for the recipe)."""
    try:
        fn = WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None
    return fn(seed)


def random_problem(M: int, K: int, N: int, seed: int, x_dtype: str = "f32",
                   sigma: float = 0.02, x_scale: float = 1.0) -> Workload:
    """A generic Gaussian problem of any shape (parity cases, ragged tails)."""
    rng = np.random.default_rng(seed)
    W = _gauss_w(rng, N, K, sigma)
    X, bits = _finish_x(x_scale * rng.standard_normal((M, K)), x_dtype)
    return Workload(f"gauss_m{M}_k{K}_n{N}_s{seed}", M, K, N, W, X, x_dtype, bits)


@dataclass
class FfnWorkload:
    name: str
    M: int
    D: int
    F: int
    D_out: int
    X: np.ndarray  # float32 [M, D]
    x_dtype: str
    X_bf16_bits: Optional[np.ndarray]
    W_up: np.ndarray  # float32 [F, D]
    W_down: np.ndarray  # float32 [D_out, F]
    notes: dict = field(default_factory=dict)


def _ffn_from(proj: str, sigma: float, name: str, seed: int) -> FfnWorkload:
    P = make_workload(proj, seed)
    rng = np.random.default_rng(seed + 1)
    W_down = _gauss_w(rng, P.K, P.N, sigma)
    return FfnWorkload(name, P.M, P.K, P.N, P.K, P.X, P.x_dtype, P.X_bf16_bits, P.W, W_down, dict(P.notes))


FFN_WORKLOADS = {
    # the small-batch decode FFN: d_model 2048, hidden 5632, 8 tokens
    "ffn_block_decode_m8_d2048_f5632": lambda seed=0: _ffn_from(
        "decode_ffn_up_m8_k2048_n5632", 0.02, "ffn_block_decode_m8_d2048_f5632", seed),
    # the 7B-like prefill FFN: d_model 4096, hidden 11008, 2048 tokens
    "ffn_block_prefill_m2048_d4096_f11008": lambda seed=0: _ffn_from(
        "prefill_ffn_m2048_k4096_n11008", 0.015, "ffn_block_prefill_m2048_d4096_f11008", seed),
}


def make_ffn_workload(name: str, seed: int = 0) -> FfnWorkload:
    try:
        fn = FFN_WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown FFN workload {name!r}; known: {sorted(FFN_WORKLOADS)}") from None
    return fn(seed)
