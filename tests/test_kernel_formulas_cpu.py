"""Host checks of arithmetic shortcuts the gfx950 kernels take in place of
the oracle's plain operations (the kernels' own results are compared with
the oracle bit for bit by the GPU tests; these pin why that can hold)."""

from fractions import Fraction

import numpy as np

INV255_BITS = 0x3B808081  # the kernels' fl32(1/255)


def _f32(x: Fraction) -> np.float32:
    """x rounded to the nearest fp32 (ties to even), exactly."""
    c = np.float32(float(x))
    best = None
    for v in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        err = abs(Fraction(float(v)) - x)
        key = (err, int(np.float32(v).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, np.float32(v))
    return best[1]


def test_inv255_constant_is_the_rounded_reciprocal():
    assert int(_f32(Fraction(1, 255)).view(np.uint32)) == INV255_BITS


def test_reciprocal_with_one_fma_correction_equals_division_for_every_code():
    # r0 = fl(q c); e = fl(q - 255 r0) (one fma); ratio = fl(e c + r0) (one fma)
    c = Fraction(float(np.uint32(INV255_BITS).view(np.float32)))
    for q in range(256):
        r0 = _f32(Fraction(q) * c)
        e = _f32(Fraction(q) - 255 * Fraction(float(r0)))
        ratio = _f32(Fraction(float(e)) * c + Fraction(float(r0)))
        exact = _f32(Fraction(q, 255))
        assert ratio.view(np.uint32) == exact.view(np.uint32), q
        # and the oracle's numpy division gives the same value
        assert (np.float32(q) / np.float32(255)).view(np.uint32) == exact.view(np.uint32), q


# ---------------------------------------------------------------------------
# The quantizer's quotient: X = fl32(w / b), b = a / 16, from y = fl32(1 / b)
# and two fma corrections, must equal 16 fl32(w / a) -- the oracle's numpy
# division -- wherever the code can depend on it (|X| >= 1/2), and stay
# below 1/2 in magnitude elsewhere.  Every fma is rounded exactly here.

FAST_MIN, FAST_MAX = 2.0 ** -90, 2.0 ** 120


def _fma(a, b, c):
    return _f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def _kernel_quotient(w, a):
    b = np.float32(a) * np.float32(0.0625)
    y = _f32(Fraction(1) / Fraction(float(b)))
    q = _f32(Fraction(float(w)) * Fraction(float(y)))
    r = _fma(-b, q, w)
    q = _fma(r, y, q)
    r = _fma(-b, q, w)
    return _fma(r, y, q)


def _check(w, a):
    w, a = np.float32(w), np.float32(a)
    assert abs(w) <= a and FAST_MIN <= a <= FAST_MAX
    X = _kernel_quotient(w, a)
    x = np.float32(w) / np.float32(a)  # the oracle's fl32(w / a)
    if abs(x) >= np.float32(1 / 32):
        assert X.view(np.uint32) == (x * np.float32(16)).view(np.uint32), (w, a)
    else:
        assert abs(X) < 0.5, (w, a)


def _near(v, k):
    """The fp32 k ulps from v (k may be negative)."""
    bits = int(np.float32(v).view(np.int32)) + k
    return np.int32(bits).view(np.float32)


def test_quotient_equals_division_near_every_threshold():
    # w whose quotient falls within a few ulps of the midpoint that decides
    # each threshold comparison, for absmax values across the fast range
    thr = [np.float32(t) for t in _level_thresholds()]
    rng = np.random.default_rng(5)
    absmax = [np.float32(2.0) ** e * np.float32(m) for e, m in
              zip(rng.integers(-90, 120, 160), rng.uniform(1, 2, 160))]
    absmax += [np.float32(FAST_MIN), np.float32(FAST_MAX), np.float32(0.0371), np.float32(1.0),
               np.float32(np.nextafter(np.float32(2), np.float32(0)))]
    for a in absmax:
        a = np.float32(a)
        for t in thr:
            mid = (Fraction(float(t)) + Fraction(float(np.nextafter(t, np.float32(np.inf))))) / 2
            w0 = _f32(mid * Fraction(float(a)))
            for k in range(-3, 4):
                w = _near(w0, k)
                if abs(w) <= a:
                    _check(w, a)


def test_quotient_equals_division_on_random_and_extreme_weights():
    rng = np.random.default_rng(6)
    for _ in range(2000):
        a = np.float32(2.0 ** rng.integers(-90, 120) * rng.uniform(1, 2))
        for w in (a, -a, np.float32(0), np.float32(-0.0), _near(a, -1),
                  np.float32(a * np.float32(rng.uniform(-1, 1))),
                  np.float32(a * np.float32(rng.uniform(-1, 1) * 1e-3)),
                  np.float32(a * np.float32(1e-30)) if a > 1e-60 else np.float32(0)):
            _check(w, a)


def _level_thresholds():
    """The 15 decision points between neighbouring levels: the largest fp32
    x still nearest to the lower level (first-argmin ties), found by scanning
    the fp32 values between the two levels with the oracle's own rule."""
    from oracle import codebook as ocodebook
    from oracle import native as onative
    L = ocodebook.nf4_levels()
    out = []
    for j in range(15):
        lo = np.float32(L[j])
        hi = np.float32(L[j + 1])
        # bisection over ordered fp32 values in [lo, hi]
        def code(v):
            return int(onative.nearest_level_of_bits(int(np.float32(v).view(np.uint32)), 1, L)[0])
        a, b = lo, hi
        while True:
            mid = np.float32((np.float64(a) + np.float64(b)) / 2)
            if mid == a or mid == b:
                break
            if code(mid) <= j:
                a = mid
            else:
                b = mid
        while code(np.nextafter(a, np.float32(np.inf))) <= j:
            a = np.nextafter(a, np.float32(np.inf))
        out.append(a)
    return out
