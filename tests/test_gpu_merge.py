"""GPU parity of qlora_merge (W_merged = bf16(W_hat + (alpha/r) B A)) against
the oracle.

The kernel rounds once from fp32 (the rank-r sum accumulated in fp32); the
oracle is exact in fp64.  Every element must lie within the error bound of
that arithmetic (fp32 roundings of the terms plus one bf16 rounding; where
the base and the adapter term cancel, the fp32 part dominates), the whole
within rel. Frobenius 2e-3 as for the linear, and where the result is a
single exact product or the base alone it must match bit for bit."""

import numpy as np
import pytest
import torch

import synth
from oracle import dense as odense
from oracle import native as onative
from oracle import nf4 as onf4

from gpu_util import TOL, banner, dev_bf16, dev_f32, host_bits, require_gpu

pytestmark = pytest.mark.gpu


def _allowed(w_hat, A, B, alpha, r, ref):
    """Per-element bound on |kernel - exact|: the fp32 rank-r sum and the
    fp32 addition (at most (r + 2) roundings of magnitude <= 2^-24 times the
    absolute terms), then one bf16 rounding (half a bf16 ulp of the result,
    taken as a whole ulp)."""
    s = float(alpha) / float(r)
    absterm = s * (np.abs(odense.widen(B)) @ np.abs(odense.widen(A))) + np.abs(odense.widen(w_hat))
    mag = np.abs(ref) + (r + 2) * 2.0 ** -24 * absterm
    ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 2.0 ** -126))) - 7)
    return ulp + (r + 2) * 2.0 ** -24 * absterm


def _run(q, w, A, B, r, alpha):
    W = q.nf4_quantize_weight(dev_f32(w))
    got = host_bits(q.qlora_merge(W, dev_bf16(A), dev_bf16(B), r, alpha))
    packed, aq, sc = onf4.quantize(w.reshape(-1), nearest=onative.nearest_level)
    w_hat = onf4.dequantize(packed, aq, sc).reshape(w.shape)
    return got, w_hat


@pytest.mark.parametrize("n_out,n_in,r,alpha", [
    (256, 256, 8, 16.0),       # the single-linear shape
    (192, 320, 12, 24.0),      # in not a multiple of the 256-column tile, r not of 16
    (64, 64, 256, 8.0),        # largest rank
    (320, 448, 24, 48.0),      # A and B read directly (r % 8 == 0), a partly live column strip
    (128, 512, 72, 144.0),     # padded factors, rank in two 64-wide chunks
    (14336, 4096, 64, 128.0),  # 8B MLP gate at full size
])
def test_merge_matches_oracle(n_out, n_in, r, alpha):
    q = require_gpu()
    banner(f"merge out={n_out} in={n_in} r={r}")
    w = synth.normal_f32(synth.seed_for(6, r % 10, "W"), (n_out, n_in), synth.W_STD)
    A = synth.bf16_bits(synth.normal_f32(synth.seed_for(6, r % 10, "A"), (r, n_in), 1.0 / n_in))
    # B larger than the workloads' 0.01 so the adapter term is visible in bf16
    B = synth.bf16_bits(synth.normal_f32(synth.seed_for(6, r % 10, "B"), (n_out, r), 1.0))
    got, w_hat = _run(q, w, A, B, r, alpha)
    ref = odense.merge(w_hat, A, B, alpha, r)
    gotf = onf4.bf16_bits_to_f32(got).reshape(ref.shape).astype(np.float64)
    err = odense.rel_frobenius(gotf, ref)
    excess = np.abs(gotf - ref) / _allowed(w_hat, A, B, alpha, r, ref)
    ref_bits = onf4.bf16_rne_bits(ref.astype(np.float32)).reshape(ref.shape)
    frac = float(np.mean(got.reshape(ref.shape) != ref_bits))
    print(f"  rel_frobenius={err:.3e} max |err|/bound={excess.max():.3f} "
          f"bf16 patterns differing from the rounded oracle={frac:.2e}", flush=True)
    assert err <= TOL
    assert excess.max() <= 1.0
    assert frac < 0.01


def test_merge_without_adapter_is_the_dequantized_base():
    q = require_gpu()
    banner("merge B = 0")
    w = synth.normal_f32(71, (320, 512), synth.W_STD)
    A = synth.bf16_bits(synth.normal_f32(72, (16, 512), 1.0))
    B = np.zeros((320, 16), dtype=np.uint16)
    got, w_hat = _run(q, w, A, B, 16, 32.0)
    assert np.array_equal(got.reshape(w_hat.shape), w_hat)


def test_merge_rank_one_on_zero_weight_is_exact():
    # W = 0 (codes 7, absmax 0) and r = 1 with s = 2: every element is the
    # single product 2 b a, exact in fp32, rounded once to bf16
    q = require_gpu()
    banner("merge W = 0, r = 1")
    w = np.zeros((128, 256), dtype=np.float32)
    A = synth.bf16_bits(synth.normal_f32(73, (1, 256), 1.0))
    B = synth.bf16_bits(synth.normal_f32(74, (128, 1), 1.0))
    got, w_hat = _run(q, w, A, B, 1, 2.0)
    ref = odense.merge(w_hat, A, B, 2.0, 1)
    assert np.array_equal(got.reshape(ref.shape), onf4.bf16_rne_bits(ref.astype(np.float32)).reshape(ref.shape))
