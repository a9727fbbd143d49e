"""The kernels decide ternary codes without a division (ternary_thresholds in
csrc/common.hpp): with d = fp32(gamma + eps), for float32 weights w,

    Round(Clip(fp32(w / d), -1, 1)) != 0   <=>   |w| > d/2
    |fp32(w / d)| <= 1                     <=>   |w| <= d

The exact boundaries are d (1/2 + 2^-25) and d (1 + 2^-24) (the ties above
1/2 and 1 round down to the even float32); no float32 lies between d/2 and
the first, or between d and the second, so their float32 round-downs are d/2
and d.  This checks that, and both identities against the literal IEEE
float32 division and round-half-to-even, for many scales d and for every
float32 weight in a window around each boundary, so a wrong constant or an
off-by-one-ulp threshold fails."""
import numpy as np


def f32_round_down(x: float) -> np.float32:
    f = np.float32(x)
    if float(f) > x:
        f = np.nextafter(f, np.float32(0))
    return f


def thresholds(d: np.float32):
    """What the kernels use: d/2 and d."""
    return np.float32(d) * np.float32(0.5), np.float32(d)


def exact_boundaries_rounded_down(d: np.float32):
    dd = float(d)
    return f32_round_down(dd * (0.5 + 2.0 ** -25)), f32_round_down(dd * (1.0 + 2.0 ** -24))


def window(center: np.float32, n: int) -> np.ndarray:
    """The 2n + 1 float32 values around `center` (consecutive ulps)."""
    bits = np.float32(center).view(np.int32)
    return (bits + np.arange(-n, n + 1, dtype=np.int32)).view(np.float32)


def test_threshold_identities_against_the_division():
    rng = np.random.default_rng(17)
    scales = np.concatenate([
        np.float32(1e-5) + np.zeros(1, np.float32),                       # gamma = 0
        (rng.uniform(1e-5, 1e-3, 300)).astype(np.float32),
        (rng.uniform(1e-3, 0.1, 300)).astype(np.float32),
        (10.0 ** rng.uniform(-1, 3, 200)).astype(np.float32),
    ])
    checked = 0
    for gamma in scales:
        d = np.float32(gamma) + np.float32(1e-5)                          # fp32(gamma + eps)
        t_nz, t_rng = thresholds(d)
        assert (t_nz, t_rng) == exact_boundaries_rounded_down(d)
        centers = [d * np.float32(0.5), d, np.float32(float(d) * 0.5), np.float32(float(d) * 1.5)]
        w = np.concatenate([window(c, 40) for c in centers])
        w = np.concatenate([w, -w, np.float32([0.0, -0.0])])
        with np.errstate(over="ignore", invalid="ignore"):
            t = w / d                                                     # IEEE float32 quotient
        q = np.rint(np.clip(t, np.float32(-1), np.float32(1)))
        assert np.array_equal(q != 0, np.abs(w) > t_nz), f"nonzero threshold wrong for d={d!r}"
        assert np.array_equal(np.abs(t) <= 1, np.abs(w) <= t_rng), f"range threshold wrong for d={d!r}"
        checked += w.size
    assert checked > 200_000


def test_ties_round_to_zero():
    """A quotient of exactly 1/2 is a tie that rounds to the even 0; the
    threshold keeps such weights at code 0 and the next float32 above them
    at +-1 (when that quotient exceeds 1/2)."""
    for d in (np.float32(0.25), np.float32(1e-5), np.float32(0.0123)):
        t_nz, _ = thresholds(d)
        half = np.float32(float(d) / 2)              # exact when d is a power of two
        if float(half) * 2 == float(d):
            assert not (abs(half) > t_nz)
            assert np.rint(half / d) == 0
        above = np.nextafter(t_nz, np.float32(np.inf))
        assert np.rint(np.clip(above / d, -1, 1)) != 0
        assert np.rint(np.clip(t_nz / d, -1, 1)) == 0
