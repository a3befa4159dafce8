"""Pins of oracle.dense: explicit loops on tiny shapes, torch autograd for the
backward (an independent derivation of the gradients of the forward), and
the special cases the formulas reduce to."""

import numpy as np
import torch

from oracle import dense
from oracle.nf4 import bf16_bits_to_f32
from synth import bf16_bits


def _bf16(rng, shape, std=1.0):
    return bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(std))


def _problem(seed, T=3, n_in=5, n_out=4, r=2):
    rng = np.random.default_rng(seed)
    return (_bf16(rng, (n_out, n_in), 0.05), _bf16(rng, (T, n_in)), _bf16(rng, (r, n_in), 0.3),
            _bf16(rng, (n_out, r), 0.3), _bf16(rng, (T, n_out)))


def _f(b):
    return bf16_bits_to_f32(b).astype(np.float64)


def test_forward_against_loops():
    W, X, A, B, _ = _problem(0)
    alpha, r = 6.0, 2
    Wd, Xd, Ad, Bd = _f(W), _f(X), _f(A), _f(B)
    T, n_in = Xd.shape
    n_out = Wd.shape[0]
    Y = dense.linear_fwd(W, X, A, B, alpha, r)
    for t in range(T):
        u = [sum(Xd[t, k] * Ad[j, k] for k in range(n_in)) for j in range(r)]
        for o in range(n_out):
            base = sum(Xd[t, k] * Wd[o, k] for k in range(n_in))
            lora = sum(u[j] * Bd[o, j] for j in range(r))
            assert abs(Y[t, o] - (base + alpha / r * lora)) < 1e-12


def test_backward_against_autograd():
    W, X, A, B, dY = _problem(1, T=4, n_in=6, n_out=5, r=3)
    alpha, r = 9.0, 3
    Xt = torch.tensor(_f(X), requires_grad=True)
    At = torch.tensor(_f(A), requires_grad=True)
    Bt = torch.tensor(_f(B), requires_grad=True)
    Wt = torch.tensor(_f(W))
    Y = Xt @ Wt.T + (alpha / r) * (Xt @ At.T) @ Bt.T
    Y.backward(torch.tensor(_f(dY)))
    dX, dA, dB = dense.linear_bwd(W, X, dY, A, B, alpha, r)
    assert np.allclose(dX, Xt.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(dA, At.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(dB, Bt.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_backward_against_loops():
    W, X, A, B, dY = _problem(2)
    alpha, r = 4.0, 2
    s = alpha / r
    Wd, Xd, Ad, Bd, Gd = _f(W), _f(X), _f(A), _f(B), _f(dY)
    T, n_in = Xd.shape
    n_out = Wd.shape[0]
    dX, dA, dB = dense.linear_bwd(W, X, dY, A, B, alpha, r)
    # dL/dx = (W_hat + s B A)^T dL/dh, row by row
    for t in range(T):
        for k in range(n_in):
            ref = sum(Gd[t, o] * (Wd[o, k] + s * sum(Bd[o, j] * Ad[j, k] for j in range(r)))
                      for o in range(n_out))
            assert abs(dX[t, k] - ref) < 1e-12
    for j in range(r):
        for k in range(n_in):
            ref = s * sum(sum(Gd[t, o] * Bd[o, j] for o in range(n_out)) * Xd[t, k] for t in range(T))
            assert abs(dA[j, k] - ref) < 1e-12
    for o in range(n_out):
        for j in range(r):
            ref = s * sum(Gd[t, o] * sum(Xd[t, k] * Ad[j, k] for k in range(n_in)) for t in range(T))
            assert abs(dB[o, j] - ref) < 1e-12


def test_special_cases():
    W, X, A, B, dY = _problem(3, T=6, n_in=8, n_out=7, r=2)
    zero_W = np.zeros_like(W)
    Y = dense.linear_fwd(zero_W, X, A, B, 2.0, 2)
    assert np.allclose(Y, (_f(X) @ _f(A).T) @ _f(B).T)
    # one-hot rows with B = 0 select columns of W_hat exactly
    Xo = np.zeros((3, 8), dtype=np.uint16)
    Xo[0, 5] = Xo[1, 0] = Xo[2, 7] = 0x3F80       # bf16 1.0
    Y = dense.linear_fwd(W, Xo, A, np.zeros_like(B), 2.0, 2)
    assert np.array_equal(Y, _f(W)[:, [5, 0, 7]].T)
    _, dA, _ = dense.linear_bwd(W, X, dY, A, np.zeros_like(B), 2.0, 2)
    assert np.all(dA == 0)
    _, _, dB = dense.linear_bwd(W, X, dY, np.zeros_like(A), B, 2.0, 2)
    assert np.all(dB == 0)


def test_rel_frobenius():
    assert dense.rel_frobenius([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert abs(dense.rel_frobenius([3.0, 4.0], [0.0, 5.0]) - np.sqrt(10) / 5) < 1e-15


def test_merge_against_loops():
    W, _, A, B, _ = _problem(3, n_in=6, n_out=5, r=3)
    alpha, r = 6.0, 3
    Wd, Ad, Bd = _f(W), _f(A), _f(B)
    M = dense.merge(W, A, B, alpha, r)
    for o in range(Wd.shape[0]):
        for k in range(Wd.shape[1]):
            ref = Wd[o, k] + alpha / r * sum(Bd[o, j] * Ad[j, k] for j in range(r))
            assert abs(M[o, k] - ref) < 1e-12


def test_merged_weight_serves_the_same_linear():
    # (W_hat + s B A) x = W_hat x + s B (A x): the merged weight reproduces
    # the QLoRA forward for any input
    W, X, A, B, _ = _problem(4, T=6, n_in=7, n_out=5, r=2)
    alpha, r = 3.0, 2
    Y = dense.linear_fwd(W, X, A, B, alpha, r)
    Ym = _f(X) @ dense.merge(W, A, B, alpha, r).T
    assert np.max(np.abs(Y - Ym)) < 1e-12 * max(1.0, np.max(np.abs(Y)))


def test_merge_special_cases():
    W, _, A, B, _ = _problem(5)
    # B = 0: the base alone; W = 0: the adapter alone
    assert np.array_equal(dense.merge(W, A, np.zeros_like(B), 4.0, 2), _f(W))
    assert np.array_equal(dense.merge(np.zeros_like(W), A, B, 4.0, 2), 2.0 * (_f(B) @ _f(A)))
