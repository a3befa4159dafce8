"""Pins of oracle.codebook against what the pages and mathematics fix."""

import numpy as np
import pytest

from oracle import codebook
from oracle import nf4 as onf4

mpmath = pytest.importorskip("mpmath")


def ulp_distance(a: np.float32, b: np.float32) -> int:
    """Distance in fp32 units in the last place (ordered-int trick)."""
    def key(v):
        i = int(np.float32(v).view(np.int32))
        return i if i >= 0 else -(i & 0x7FFFFFFF)
    return abs(key(a) - key(b))


def test_level_invariants():
    # ultralytics "QLoRA" NF4 bullet + paperclase Parte 2 "Cuantiles": 16 levels,
    # an exact shared zero (8 + 9 - 1), normalised to [-1, 1], sorted.
    L = codebook.nf4_levels()
    assert L.dtype == np.float32 and L.shape == (16,)
    assert np.all(np.diff(L) > 0)
    assert L.view(np.uint32)[7] == 0          # +0.0 exactly, at code 7
    assert L[0] == np.float32(-1.0) and L[15] == np.float32(1.0)
    assert int((L < 0).sum()) == 7 and int((L > 0).sum()) == 8


def test_levels_against_mpmath():
    # Independent evaluation: 50-digit inverse normal CDF at the exact decimal
    # probabilities, normalised by the largest quantile, rounded to fp32.
    mpmath.mp.dps = 50
    p_hi = mpmath.mpf("0.9677083")
    half = mpmath.mpf("0.5")
    pos = [mpmath.sqrt(2) * mpmath.erfinv(2 * (p_hi + (half - p_hi) * i / 8) - 1) for i in range(8)]
    neg = [-mpmath.sqrt(2) * mpmath.erfinv(2 * (p_hi + (half - p_hi) * i / 7) - 1) for i in range(7)]
    top = max(pos)
    exact = sorted([v / top for v in neg] + [mpmath.mpf(0)] + [v / top for v in pos])
    L = codebook.nf4_levels()
    dists = [ulp_distance(L[j], np.float32(float(exact[j]))) for j in range(16)]
    # the page's fp32 evaluation (fp32 probabilities, fp32 erfinv) differs from the
    # correctly rounded values by a few ulp; a wrong formula is off by millions
    assert max(dists) <= 8, dists


def test_levels_regression_fixture(golden):
    ref = golden("nf4_levels_fp32.txt")
    L = codebook.nf4_levels().view(np.uint32)
    for j in range(16):
        assert int(ref[str(j)].split()[0], 16) == int(L[j]), j


def test_toy_levels_print(golden):
    # paperclase Parte 2: the printed 2-decimal table of the toy NF4 (d = 0.03)
    g = golden("paperclase_toy_levels.txt")
    toy = codebook.toy_nf4_levels(float(g["d"]))
    assert len(toy) == 16
    printed = []
    for i in range(0, 16, 4):
        printed.append(" ".join(f"{v:+.2f}" for v in toy[i:i + 4]))
    assert printed == [g["row0"], g["row1"], g["row2"], g["row3"]]
    int4 = codebook.int4_levels()
    assert len(int4) == int(g["int4_levels"])
    assert f"{round(1 / 7, 3)}" == g["int4_step_3dp"]
    assert np.allclose(np.diff(int4), 1 / 7, atol=1e-6)


def test_uniform16_levels():
    u = codebook.uniform16_levels()
    assert u.shape == (16,) and u[0] == -1 and u[-1] == 1
    assert np.allclose(np.diff(u), 2 / 15, atol=1e-6)


def test_mse_experiment_reproduces_page(golden):
    # ultralytics "QLoRA": seed 0, randn(4096, 64) * 0.02, exact block absmax,
    # nearest level, MSE printed with ".3e".  Pins codebook, block absmax,
    # normalisation and the nearest-level rule together.
    import torch
    g = golden("ultralytics_mse.txt")
    torch.manual_seed(int(g["seed"]))
    rows, cols = (int(v) for v in g["shape"].split())
    w = (torch.randn(rows, cols) * float(g["std"])).numpy()
    out = {}
    for name, levels in (("nf4", codebook.nf4_levels()), ("uniform16", codebook.uniform16_levels())):
        restored = onf4.blockwise_restore(w, levels)
        mse = np.mean((restored.astype(np.float64) - w.astype(np.float64)) ** 2)
        out[name] = mse
        assert f"{mse:.3e}" == g[f"{name}_mse"], (name, mse)
    reduction = 100 * (1 - out["nf4"] / out["uniform16"])
    assert abs(reduction - float(g["reduction_percent_approx"])) < 1.0


def test_mse_experiment_through_the_stored_format_without_double_quant(golden):
    # the same experiment through the 4.5-bit storage (codes + fp32 block
    # absmax) and its fp32 reconstruction: identical to the page's print
    import torch
    g = golden("ultralytics_mse.txt")
    torch.manual_seed(int(g["seed"]))
    rows, cols = (int(v) for v in g["shape"].split())
    w = (torch.randn(rows, cols) * float(g["std"])).numpy()
    codes, absmax = onf4.quantize_nodq(w)
    assert codes.size * 8 + absmax.size * 32 == 4.5 * w.size  # 4 + 32/64 bits per weight
    restored = onf4.dequantize_nodq_f32(codes, absmax).reshape(w.shape)
    mse = np.mean((restored.astype(np.float64) - w.astype(np.float64)) ** 2)
    assert f"{mse:.3e}" == g["nf4_mse"]
