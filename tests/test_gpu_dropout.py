"""GPU parity of the LoRA-dropout calls (qlora_linear_fwd_dropout /
qlora_linear_bwd_dropout) against the fp64 oracle (oracle.dense.*_dropout),
on the same seeded inputs and the same packed keep mask.

Acceptance as for the plain linear: relative Frobenius error <= 2e-3 for each
of Y, dX, dA and dB.  Reductions the method has: p = 0 with every element
kept equals the plain call (Y bit for bit above 16 tokens, where both take
the same kernels; dX, dA, dB up to summation order); nothing kept leaves the
base alone (Y and dX equal the plain call with a zero adapter, dA = dB = 0)."""

import numpy as np
import pytest
import torch

import synth
from oracle import dense as odense
from oracle import native as onative
from oracle import nf4 as onf4

from gpu_util import TOL, banner, dev_bf16, dev_f32, host, host_bits, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(seed, T, n_in, n_out, r):
    w = synth.normal_f32(seed, (n_out, n_in), synth.W_STD)
    X = synth.bf16_bits(synth.normal_f32(seed + 1, (T, n_in), 1.0))
    A = synth.bf16_bits(synth.normal_f32(seed + 2, (r, n_in), 1.0 / n_in))
    # B larger than the workloads' 0.01 so the adapter term is well above rounding
    B = synth.bf16_bits(synth.normal_f32(seed + 3, (n_out, r), 0.05))
    dY = synth.bf16_bits(synth.normal_f32(seed + 4, (T, n_out), 1.0))
    return w, X, A, B, dY


def _w_hat(w):
    packed, aq, sc = onf4.quantize(w.reshape(-1), nearest=onative.nearest_level)
    return onf4.dequantize(packed, aq, sc).reshape(w.shape)


def _rows(T, n=24):
    rng = np.random.Generator(np.random.PCG64(9))
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=min(n, T), replace=False)]))


def _run(q, w, X, A, B, dY, keep_bytes, p, r, alpha):
    W = q.nf4_quantize_weight(dev_f32(w))
    Xd, Ad, Bd, Gd = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    K = torch.from_numpy(np.ascontiguousarray(keep_bytes)).cuda()
    Y = q.qlora_linear_fwd_dropout(W, Xd, K, p, Ad, Bd, r, alpha)
    dX, dA, dB = q.qlora_linear_bwd_dropout(W, Xd, Gd, K, p, Ad, Bd, r, alpha)
    return W, host_bits(Y), host_bits(dX), host(dA), host(dB)


@pytest.mark.parametrize("T,n_in,n_out,r,alpha,p", [
    (1, 256, 192, 12, 24.0, 0.05),        # one token: general path, not the small-token kernel
    (16, 4096, 4096, 16, 32.0, 0.05),     # decode-shaped q_proj
    (300, 512, 256, 16, 32.0, 0.1),       # ragged T, 128-tiles
    (1000, 1024, 640, 64, 128.0, 0.3),    # heavier dropout, r = 64
    (4096, 4096, 14336, 64, 128.0, 0.05), # 8B MLP gate shape (256-tiles, dX over 14336)
])
def test_dropout_matches_oracle(T, n_in, n_out, r, alpha, p):
    q = require_gpu()
    banner(f"dropout T={T} in={n_in} out={n_out} r={r} p={p}")
    w, X, A, B, dY = _inputs(7000 + T % 1000, T, n_in, n_out, r)
    kb = synth.keep_mask(7100 + T % 1000, T, n_in, p)
    _, Y, dX, dA, dB = _run(q, w, X, A, B, dY, kb, p, r, alpha)
    keep = odense.unpack_keep(kb, T, n_in)
    wh = odense.widen(_w_hat(w))
    s = alpha / r
    Xw, Aw, Bw, Gw = odense.widen(X), odense.widen(A), odense.widen(B), odense.widen(dY)
    Xt = odense.dropped_input(X, keep, p)
    U = Xt @ Aw.T
    V = Gw @ Bw
    rows = _rows(T)
    Y_ref = Xw[rows] @ wh.T + s * (U[rows] @ Bw.T)
    dX_ref = Gw[rows] @ wh + np.where(keep[rows], s * (V[rows] @ Aw), 0.0) / (1 - p)
    errs = {
        "Y": odense.rel_frobenius(onf4.bf16_bits_to_f32(Y[rows]).astype(np.float64), Y_ref),
        "dX": odense.rel_frobenius(onf4.bf16_bits_to_f32(dX[rows]).astype(np.float64), dX_ref),
        "dA": odense.rel_frobenius(dA, s * (V.T @ Xt)),
        "dB": odense.rel_frobenius(dB, s * (Gw.T @ U)),
    }
    if T <= 300:  # the whole-tensor oracle too (its own code path)
        Yf = odense.linear_fwd_dropout(wh, X, A, B, alpha, r, keep, p)
        dXf, dAf, dBf = odense.linear_bwd_dropout(wh, X, dY, A, B, alpha, r, keep, p)
        errs["Y_all"] = odense.rel_frobenius(onf4.bf16_bits_to_f32(Y).astype(np.float64), Yf)
        errs["dX_all"] = odense.rel_frobenius(onf4.bf16_bits_to_f32(dX).astype(np.float64), dXf)
        errs["dA_all"] = odense.rel_frobenius(dA, dAf)
        errs["dB_all"] = odense.rel_frobenius(dB, dBf)
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= TOL for v in errs.values()), errs


@pytest.mark.parametrize("T", [40, 600])
def test_everything_kept_at_p0_is_the_plain_call(T):
    q = require_gpu()
    banner(f"dropout p=0 all kept vs plain T={T}")
    n_in, n_out, r, alpha = 320, 192, 12, 24.0
    w, X, A, B, dY = _inputs(7300, T, n_in, n_out, r)
    kb = np.full((T, n_in // 8), 0xff, dtype=np.uint8)
    W, Y, dX, dA, dB = _run(q, w, X, A, B, dY, kb, 0.0, r, alpha)
    Xd, Ad, Bd, Gd = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    Y1 = host_bits(q.qlora_linear_fwd(W, Xd, Ad, Bd, r, alpha))
    dX1, dA1, dB1 = q.qlora_linear_bwd(W, Xd, Gd, Ad, Bd, r, alpha)
    assert np.array_equal(Y, Y1)
    # the masked dX adds the adapter term first, the plain one last
    f = lambda b: onf4.bf16_bits_to_f32(b).astype(np.float64)
    assert odense.rel_frobenius(f(dX), f(host_bits(dX1))) < 1e-4
    assert odense.rel_frobenius(dA, host(dA1).astype(np.float64)) < 1e-6
    assert odense.rel_frobenius(dB, host(dB1).astype(np.float64)) < 1e-6


def test_nothing_kept_leaves_the_base():
    q = require_gpu()
    banner("dropout nothing kept")
    T, n_in, n_out, r, alpha = 200, 256, 128, 8, 16.0
    w, X, A, B, dY = _inputs(7400, T, n_in, n_out, r)
    kb = np.zeros((T, n_in // 8), dtype=np.uint8)
    W, Y, dX, dA, dB = _run(q, w, X, A, B, dY, kb, 0.5, r, alpha)
    assert not dA.any() and not dB.any()
    Xd, Gd = dev_bf16(X), dev_bf16(dY)
    zA = torch.zeros(r, n_in, dtype=torch.bfloat16, device="cuda")
    zB = torch.zeros(n_out, r, dtype=torch.bfloat16, device="cuda")
    assert np.array_equal(Y, host_bits(q.qlora_linear_fwd(W, Xd, zA, zB, r, alpha)))
    dX0, _, _ = q.qlora_linear_bwd(W, Xd, Gd, zA, zB, r, alpha)
    assert np.array_equal(dX, host_bits(dX0))
