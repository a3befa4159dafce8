"""GPU parity of the multi-projection calls (projections sharing X, e.g.
q|k|v and gate|up) against the fp64 oracle, projection by projection:
Y_i = X W_hat_i^T + s (X A_i^T) B_i^T side by side; dX = sum_i of the
single-projection input gradients (one rounding); dA_i, dB_i per projection.
Acceptance as for the single linear: rel. Frobenius <= 2e-3 for each of Y,
dX, dA_i, dB_i; n = 1 must be bit-identical to the single-projection call."""

import numpy as np
import pytest
import torch

import synth
from oracle import dense as odense
from oracle import native as onative
from oracle import nf4 as onf4

from gpu_util import TOL, banner, dev_bf16, dev_f32, host, host_bits, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(seed, T, n_in, outs, r):
    ws, As, Bs = [], [], []
    for i, o in enumerate(outs):
        ws.append(synth.normal_f32(seed + 10 * i, (o, n_in), synth.W_STD))
        As.append(synth.bf16_bits(synth.normal_f32(seed + 10 * i + 1, (r, n_in), 1.0 / n_in)))
        Bs.append(synth.bf16_bits(synth.normal_f32(seed + 10 * i + 2, (o, r), 0.05)))
    X = synth.bf16_bits(synth.normal_f32(seed + 7, (T, n_in), 1.0))
    dY = synth.bf16_bits(synth.normal_f32(seed + 8, (T, sum(outs)), 1.0))
    return ws, As, Bs, X, dY


def _w_hat(w):
    packed, aq, sc = onf4.quantize(w.reshape(-1), nearest=onative.nearest_level)
    return onf4.dequantize(packed, aq, sc).reshape(w.shape)


def _rows(T, n=24):
    rng = np.random.Generator(np.random.PCG64(5))
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=min(n, T), replace=False)]))


@pytest.mark.parametrize("T,n_in,outs,r,alpha", [
    (300, 256, [512, 256], 16, 32.0),              # gate|up-like, ragged T, 128-tiles
    (9, 512, [256, 64, 64], 16, 32.0),             # q|k|v-like at a small-token count
    (1, 4096, [4096, 1024, 1024], 16, 32.0),       # 8B q|k|v decode: U up front, one launch
    (16, 4096, [4096, 1024, 1024], 16, 32.0),      # the same at T = 16
    (7, 1024, [128, 64, 192], 24, 48.0),           # r > 16: U computed up front, one launch
    (5, 1024, [2048, 1024, 1024], 16, 32.0),       # 4096 rows: one fused launch
    (4096, 4096, [4096, 1024, 1024], 16, 32.0),    # 8B q|k|v at T = 4096 (256-tiles)
    (4096, 1024, [4160, 4032], 8, 16.0),           # outputs not multiples of the tile
])
def test_multi_projection_matches_oracle(T, n_in, outs, r, alpha):
    q = require_gpu()
    banner(f"multi T={T} in={n_in} outs={outs} r={r}")
    ws, As, Bs, X, dY = _inputs(900 + T % 97, T, n_in, outs, r)
    Ws = [q.nf4_quantize_weight(dev_f32(w)) for w in ws]
    Xd, dYd = dev_bf16(X), dev_bf16(dY)
    Ad, Bd = [dev_bf16(a) for a in As], [dev_bf16(b) for b in Bs]
    Y = host_bits(q.qlora_linear_fwd_multi(Ws, Xd, Ad, Bd, r, alpha))
    dX, dAs, dBs = q.qlora_linear_bwd_multi(Ws, Xd, dYd, Ad, Bd, r, alpha)
    dX = host_bits(dX)
    dAs, dBs = [host(t) for t in dAs], [host(t) for t in dBs]

    rows = _rows(T)
    s = float(alpha) / float(r)
    Xw = odense.widen(X)
    Gw = odense.widen(dY)
    dX_ref = np.zeros((len(rows), n_in))
    off = 0
    errs = {}
    for i, (w, A, B) in enumerate(zip(ws, As, Bs)):
        o = w.shape[0]
        wh = odense.widen(_w_hat(w))
        Aw, Bw = odense.widen(A), odense.widen(B)
        U = Xw @ Aw.T
        Gi = Gw[:, off:off + o]
        V = Gi @ Bw
        Y_ref = Xw[rows] @ wh.T + s * (U[rows] @ Bw.T)
        got = onf4.bf16_bits_to_f32(Y[rows, off:off + o]).astype(np.float64)
        errs[f"Y{i}"] = odense.rel_frobenius(got, Y_ref)
        dX_ref += Gi[rows] @ wh + s * (V[rows] @ Aw)
        errs[f"dA{i}"] = odense.rel_frobenius(dAs[i], s * (V.T @ Xw))
        errs[f"dB{i}"] = odense.rel_frobenius(dBs[i], s * (Gi.T @ U))
        off += o
    errs["dX"] = odense.rel_frobenius(onf4.bf16_bits_to_f32(dX[rows]).astype(np.float64), dX_ref)
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= TOL for v in errs.values()), errs


@pytest.mark.parametrize("T", [5, 600])
def test_one_projection_equals_single_call(T):
    q = require_gpu()
    banner(f"multi n=1 vs single call T={T}")
    ws, As, Bs, X, dY = _inputs(950, T, 320, [192], 12)
    W = q.nf4_quantize_weight(dev_f32(ws[0]))
    Xd, dYd, Ad, Bd = dev_bf16(X), dev_bf16(dY), dev_bf16(As[0]), dev_bf16(Bs[0])
    Y1 = q.qlora_linear_fwd(W, Xd, Ad, Bd, 12, 24.0)
    Ym = q.qlora_linear_fwd_multi([W], Xd, [Ad], [Bd], 12, 24.0)
    assert torch.equal(Y1.view(torch.int16), Ym.view(torch.int16))
    dX1, dA1, dB1 = q.qlora_linear_bwd(W, Xd, dYd, Ad, Bd, 12, 24.0)
    dXm, dAm, dBm = q.qlora_linear_bwd_multi([W], Xd, dYd, [Ad], [Bd], 12, 24.0)
    assert torch.equal(dX1.view(torch.int16), dXm.view(torch.int16))
    # dA, dB: the same token slices added in the same order, bit for bit
    assert torch.equal(dAm[0].view(torch.int32), dA1.view(torch.int32))
    assert torch.equal(dBm[0].view(torch.int32), dB1.view(torch.int32))
