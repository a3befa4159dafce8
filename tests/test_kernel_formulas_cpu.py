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
