"""GPU parity of the large-token QLoRA linear at the full workload sizes.

Forward and backward of the 8B MLP (gate 4096->14336, down 14336->4096,
T = 4096, r = 64), the 8B attention projections (q 4096x4096, k 4096->1024,
T = 8192, r = 16) and the 70B MLP (gate 8192->28672, down 28672->8192,
T = 4096, r = 64, alpha = 16), each through the same calls and launch
configuration the benchmark times, plus a ragged token count on the
256 x 256-tile GEMM.

The oracle quantizes the same fp32 weight itself and evaluates, in fp64, the
outputs it can afford one by one: sampled token rows of Y and dX (every
output feature of those rows) and the full dA and dB (their reductions over
all tokens).  Acceptance: relative Frobenius error <= 2e-3 for each of Y, dX,
dA and dB over what is compared."""

import numpy as np
import pytest

import synth
from oracle import dense as odense
from oracle import native as onative
from oracle import nf4 as onf4

from gpu_util import TOL, banner, dev_bf16, dev_f32, host, host_bits, require_gpu

pytestmark = pytest.mark.gpu


def _rows(T, n=24, seed=11):
    """Sampled token rows: the first and last of the first tiles, the last
    row, and random rows in between."""
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = [0, 1, 127, 128, 255, 256, T - 1]
    pick = rng.choice(T, size=n, replace=False)
    return np.unique(np.concatenate([np.array([t for t in fixed if t < T]), pick]))


def _case(wid, proj, T=None):
    wl = synth.WORKLOADS[wid]
    p = wl.projections[proj]
    T = wl.tokens[0] if T is None else T
    r, alpha = wl.r, wl.alpha
    w = synth.weight(wid, proj, p.out_features, p.in_features)
    X = synth.activations(wid, proj, T, p.in_features)
    dY = synth.activations(wid, proj, T, p.out_features, "dY")
    A = synth.lora_A(wid, proj, r, p.in_features)
    B = synth.lora_B(wid, proj, p.out_features, r)
    return w, X, dY, A, B, r, alpha


def _check(wid, proj, T=None):
    q = require_gpu()
    w, X, dY, A, B, r, alpha = _case(wid, proj, T)
    T = X.shape[0]
    n_out, n_in = w.shape
    banner(f"large linear workload {wid} projection {proj}: T={T} out={n_out} in={n_in} r={r}")

    W = q.nf4_quantize_weight(dev_f32(w))
    Xd, dYd, Ad, Bd = dev_bf16(X), dev_bf16(dY), dev_bf16(A), dev_bf16(B)
    Y = q.qlora_linear_fwd(W, Xd, Ad, Bd, r, alpha)
    dX, dA, dB = q.qlora_linear_bwd(W, Xd, dYd, Ad, Bd, r, alpha)
    Yh = onf4.bf16_bits_to_f32(host_bits(Y)).astype(np.float64)
    dXh = onf4.bf16_bits_to_f32(host_bits(dX)).astype(np.float64)
    dAh, dBh = host(dA).astype(np.float64), host(dB).astype(np.float64)
    del Y, dX, dA, dB, W, Xd, dYd

    # oracle: its own quantization of the same weight, then fp64
    packed, aq, sc = onf4.quantize(w.reshape(-1), nearest=onative.nearest_level)
    del w
    w_hat = odense.widen(onf4.dequantize(packed, aq, sc).reshape(n_out, n_in))
    del packed, aq, sc
    s = float(alpha) / float(r)
    Xw, Gw, Aw, Bw = odense.widen(X), odense.widen(dY), odense.widen(A), odense.widen(B)
    rows = _rows(T)
    U = Xw @ Aw.T                              # [T, r]
    V = Gw @ Bw                                # [T, r]
    Y_ref = Xw[rows] @ w_hat.T + s * (U[rows] @ Bw.T)
    dX_ref = Gw[rows] @ w_hat + s * (V[rows] @ Aw)
    dA_ref = s * (V.T @ Xw)
    dB_ref = s * (Gw.T @ U)
    errs = {
        "Y": odense.rel_frobenius(Yh[rows], Y_ref),
        "dX": odense.rel_frobenius(dXh[rows], dX_ref),
        "dA": odense.rel_frobenius(dAh, dA_ref),
        "dB": odense.rel_frobenius(dBh, dB_ref),
    }
    print("  rel_frobenius " + " ".join(f"{k}={v:.3e}" for k, v in errs.items())
          + f" ({len(rows)} sampled rows)", flush=True)
    assert all(v <= TOL for v in errs.values()), errs


@pytest.mark.parametrize("wid,proj", [
    (3, 0),   # 8B MLP gate 4096 -> 14336 (fused NF4 forward on 256 x 256 tiles, 896 tiles)
    (3, 2),   # 8B MLP down 14336 -> 4096 (dX over 14336 input features)
    (4, 0),   # 8B attention q 4096 x 4096, T = 8192
    (4, 1),   # 8B attention k 4096 -> 1024 (128 x 128 tiles)
    (5, 0),   # 70B MLP gate 8192 -> 28672, alpha / r = 0.25
    (5, 2),   # 70B MLP down 28672 -> 8192
])
def test_workload_projection_fwd_bwd(wid, proj):
    _check(wid, proj)


def test_ragged_tokens_on_large_tiles():
    # q-shaped 4096 x 4096 with T = 4136: 17 x 16 tiles of 256, the last row of
    # tiles 40 tokens tall (rows past T read as zero and are not stored)
    _check(4, 0, T=4136)


def test_fused_dequant_gemm_below_materialize_threshold():
    # 8B MLP gate at T = 1536 (6 x 56 tiles of 256): the forward takes the fused
    # NF4 GEMM (codes dequantized while staged into LDS); from T = 2048 on it
    # dequantizes the weight once into the workspace instead
    _check(3, 0, T=1536)
