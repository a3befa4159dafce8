"""Pins of oracle.nf4 (quantize / double quant / pack / dequant) against what
the pages print and what the mathematics fixes.  CPU only."""

import numpy as np
import pytest
import torch

from oracle import codebook
from oracle import native
from oracle import nf4 as onf4

L = codebook.nf4_levels()
MAX_HALF_GAP = float(np.max(np.diff(L.astype(np.float64))) / 2)


def _floats(s):
    return np.array([float(v) for v in s.split()], dtype=np.float32)


# ---------------------------------------------------------------- worked example

def test_absmax_worked_example(golden):
    # paperclase "QLoRA", Parte 1: absmax 0.5, codes, reconstruction, max error
    g = golden("paperclase_absmax_example.txt")
    w = _floats(g["weights"])
    a, c, w_hat = onf4.absmax_int4(w)
    assert f"{a:.1f}" == g["absmax"]
    assert c.tolist() == [int(v) for v in g["codes"].split()]
    assert " ".join(f"{v:.2f}" for v in w_hat) == g["restored_2dp"]
    err = np.abs(w - w_hat).max()
    assert f"{err:.3f}" == g["max_error_3dp"]
    # "absmax, en formulas": |w - w_hat| <= absmax / 14, printed as 0.036 here
    assert f"{a / 14:.3f}" == g["bound_3dp"]
    assert np.all(np.abs(w - w_hat) <= a / 14 + 1e-7)
    # "Un valor atipico arruina su bloque": w[3] = 4.0
    w2 = w.copy()
    w2[int(g["outlier_index"])] = float(g["outlier_value"])
    a2, c2, _ = onf4.absmax_int4(w2)
    assert c2.tolist() == [int(v) for v in g["outlier_codes"].split()]
    assert f"{a2 / 7:.2f}" == g["outlier_step_2dp"]


# ---------------------------------------------------------------- nearest level

def test_each_level_maps_to_itself():
    c = onf4.nearest_level(L, L)
    assert c.tolist() == list(range(16))


def test_exact_tie_takes_lower_index():
    # midpoint between the zero (code 7) and L[8]: halving is exact, so the two
    # fp32 distances are identical and the first minimum (code 7) must win
    x = np.float32(L[8] / np.float32(2))
    assert np.float32(x - L[7]) == np.float32(L[8] - x)
    assert onf4.nearest_level(np.array([x]), L)[0] == 7
    assert native.nearest_level(np.array([x], dtype=np.float32), L)[0] == 7
    # and just above the midpoint it is code 8
    x_up = np.nextafter(x, np.float32(1))
    assert onf4.nearest_level(np.array([x_up]), L)[0] == 8


def test_nearest_matches_fp64_nearest():
    # exact-arithmetic nearest level agrees except where the two best exact
    # distances are within an fp32 rounding of each other
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-1, 1, 200000), rng.normal(0, 0.3, 200000)]).astype(np.float32)
    x = np.clip(x, -1, 1)
    c = onf4.nearest_level(x, L)
    d = np.abs(x.astype(np.float64)[:, None] - L.astype(np.float64)[None, :])
    exact = d.argmin(axis=1)
    srt = np.sort(d, axis=1)
    clear = (srt[:, 1] - srt[:, 0]) > 1e-6
    assert np.all(c[clear] == exact[clear])
    assert clear.mean() > 0.999


def test_c_and_numpy_nearest_agree():
    rng = np.random.default_rng(2)
    x = rng.uniform(-1, 1, 1 << 20).astype(np.float32)
    # add every level, the fp32 midpoints and their neighbours
    mids = ((L[:-1].astype(np.float64) + L[1:]) / 2).astype(np.float32)
    extra = np.concatenate([L, mids, np.nextafter(mids, 2), np.nextafter(mids, -2)])
    x = np.concatenate([x, extra.astype(np.float32)])
    assert np.array_equal(onf4.nearest_level(x, L), native.nearest_level(x, L))


def test_c_bit_walk_matches_array_version():
    lo = int(np.float32(0.03).view(np.uint32))
    n = 1 << 16
    walk = native.nearest_level_of_bits(lo, n, L)
    xs = (np.arange(lo, lo + n, dtype=np.uint64).astype(np.uint32)).view(np.float32)
    assert np.array_equal(walk, onf4.nearest_level(xs, L))


# ---------------------------------------------------------------- quantize

def _w(seed, n, std=0.02):
    return (np.random.default_rng(seed).standard_normal(n).astype(np.float32) * np.float32(std))


def test_every_nonzero_block_holds_an_extreme_code():
    # the absmax element maps to exactly +-1, i.e. code 0 or 15
    w = _w(3, 64 * 512)
    packed, q, s = onf4.quantize(w)
    codes = onf4.unpack_nibbles(packed).reshape(-1, 64)
    assert np.all(np.any((codes == 0) | (codes == 15), axis=1))


def test_power_of_two_scaling_invariance():
    w = _w(4, 64 * 300)
    p1, q1, s1 = onf4.quantize(w)
    for k in (-3, 5):
        p2, q2, s2 = onf4.quantize(w * np.float32(2.0 ** k))
        assert np.array_equal(p1, p2) and np.array_equal(q1, q2)
        assert np.array_equal(s2, s1 * np.float32(2.0 ** k))


def test_zero_block_and_zero_group():
    w = _w(5, 64 * 256 * 3)
    w[64 * 10:64 * 11] = 0                     # one zero block
    w[64 * 256:64 * 512] = 0                   # one whole zero group
    packed, q, s = onf4.quantize(w)
    codes = onf4.unpack_nibbles(packed).reshape(-1, 64)
    assert np.all(codes[10] == 7) and np.all(codes[256:512] == 7)
    assert q[10] == 0 and np.all(q[256:512] == 0)
    assert s[1] == 0 and s[0] > 0 and s[2] > 0
    back = onf4.bf16_bits_to_f32(onf4.dequantize(packed, q, s)).reshape(-1, 64)
    assert np.all(back[10] == 0) and np.all(back[256:512] == 0)


def test_nf4_error_bound_before_double_quant():
    # |L[c] a - w| <= a * (largest half gap between neighbouring levels)
    w = _w(6, 64 * 1000)
    a = onf4.block_absmax(w)
    c = onf4.nf4_codes(w, a).reshape(-1, 64)
    restored = L[c] * a[:, None]
    err = np.abs(restored.astype(np.float64) - w.reshape(-1, 64))
    assert np.all(err <= a[:, None] * (MAX_HALF_GAP + 1e-6))
    assert abs(MAX_HALF_GAP - 0.15190) < 1e-4


def test_double_quant_properties():
    w = _w(7, 64 * 256 * 4 + 64 * 37)          # 4 full groups + a partial one
    a = onf4.block_absmax(w)
    q, s = onf4.double_quantize(a)
    assert s.size == 5 and q.size == a.size
    ahat = onf4.dequant_absmax(q, s)
    for g in range(5):
        blk = slice(256 * g, min(256 * (g + 1), a.size))
        j = np.argmax(a[blk])
        assert s[g] == a[blk].max()
        assert q[blk][j] == 255 and ahat[blk][j] == a[blk][j]
        # 8-bit analogue of absmax/14: at most half a step of s/255 (+ rounding)
        err = np.abs(ahat[blk].astype(np.float64) - a[blk])
        assert np.all(err <= s[g] / 510 * (1 + 1e-5))


def test_pack_order_and_roundtrip():
    codes = np.array([1, 2, 3, 4, 15, 0], dtype=np.uint8)
    packed = onf4.pack_nibbles(codes)
    assert packed.tolist() == [0x21, 0x43, 0x0F]
    rng = np.random.default_rng(8)
    c = rng.integers(0, 16, 4096).astype(np.uint8)
    assert np.array_equal(onf4.unpack_nibbles(onf4.pack_nibbles(c)), c)


def test_dequant_with_unit_scale_is_the_codebook():
    # q = 255 and s = 1 give a_hat = 1 exactly, so w_hat = bf16(L[c])
    codes = np.tile(np.arange(16, dtype=np.uint8), 4)
    packed = onf4.pack_nibbles(codes)
    back = onf4.dequantize(packed, np.array([255], dtype=np.uint8), np.array([1.0], dtype=np.float32))
    want = torch.from_numpy(L[codes]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(back, want)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.normal(0, 1, 100000), rng.normal(0, 1e-30, 1000),
                        rng.normal(0, 1e30, 1000)]).astype(np.float32)
    # exact ties: low half 0x8000, with even and odd kept bits
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32) + (0x3F80 << 16)
    x = np.concatenate([x, ties.view(np.float32), -ties.view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(onf4.bf16_rne_bits(x), want)


def test_full_roundtrip_error_budget():
    w = _w(10, 64 * 2048)
    packed, q, s = onf4.quantize(w)
    back = onf4.bf16_bits_to_f32(onf4.dequantize(packed, q, s)).astype(np.float64).reshape(-1, 64)
    a = onf4.block_absmax(w)[:, None].astype(np.float64)
    # nearest-level error + absmax error (s/510 times |L| <= 1) + bf16 half-ulp
    sg = np.repeat(s, 256)[: a.size][:, None]
    bound = a * MAX_HALF_GAP + sg / 510 + np.abs(back) * 2.0 ** -8 + 1e-12
    assert np.all(np.abs(back - w.reshape(-1, 64)) <= bound)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        onf4.block_absmax(np.zeros(65, dtype=np.float32))
    bad = np.zeros(64, dtype=np.float32)
    bad[3] = np.inf
    with pytest.raises(ValueError):
        onf4.block_absmax(bad)
