"""Pins of the LoRA-dropout oracle (oracle.dense.*_dropout): the mask layout,
explicit loops, torch autograd through the dropped forward (an independent
derivation of its gradients), the cases dropout reduces to (p = 0 with
everything kept is the plain linear; nothing kept leaves only the base), and
the inverted-dropout scaling checked as an expectation over many masks."""

import numpy as np
import torch

import synth
from oracle import dense
from oracle.nf4 import bf16_bits_to_f32
from synth import bf16_bits


def _bf16(rng, shape, std=1.0):
    return bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(std))


def _problem(seed, T=3, n_in=16, n_out=4, r=2):
    rng = np.random.default_rng(seed)
    return (_bf16(rng, (n_out, n_in), 0.05), _bf16(rng, (T, n_in)), _bf16(rng, (r, n_in), 0.3),
            _bf16(rng, (n_out, r), 0.3), _bf16(rng, (T, n_out)))


def _f(b):
    return bf16_bits_to_f32(b).astype(np.float64)


def test_mask_layout_is_bit_k_mod_8_of_byte_k_div_8():
    packed = np.array([[0b00000101, 0b10000000]], dtype=np.uint8)  # one row, 16 elements
    keep = dense.unpack_keep(packed, 1, 16)
    expect = np.zeros(16, dtype=bool)
    expect[[0, 2, 15]] = True
    assert np.array_equal(keep[0], expect)
    # the generator packs the same way and keeps about 1 - p
    m = synth.keep_mask(7, 64, 256, 0.25)
    k = dense.unpack_keep(m, 64, 256)
    assert m.shape == (64, 32) and abs(k.mean() - 0.75) < 0.02


def test_forward_and_backward_against_loops():
    W, X, A, B, dY = _problem(1)
    alpha, r, p = 6.0, 2, 0.3
    T, n_in = X.shape
    n_out = W.shape[0]
    keep = dense.unpack_keep(synth.keep_mask(3, T, n_in, p), T, n_in)
    Wd, Xd, Ad, Bd, Gd = _f(W), _f(X), _f(A), _f(B), _f(dY)
    s = alpha / r
    Y = dense.linear_fwd_dropout(W, X, A, B, alpha, r, keep, p)
    dX, dA, dB = dense.linear_bwd_dropout(W, X, dY, A, B, alpha, r, keep, p)
    xt = [[Xd[t, k] / (1 - p) if keep[t, k] else 0.0 for k in range(n_in)] for t in range(T)]
    u = [[sum(xt[t][k] * Ad[j, k] for k in range(n_in)) for j in range(r)] for t in range(T)]
    v = [[sum(Gd[t, o] * Bd[o, j] for o in range(n_out)) for j in range(r)] for t in range(T)]
    for t in range(T):
        for o in range(n_out):
            base = sum(Xd[t, k] * Wd[o, k] for k in range(n_in))
            assert abs(Y[t, o] - (base + s * sum(u[t][j] * Bd[o, j] for j in range(r)))) < 1e-12
        for k in range(n_in):
            g = sum(Gd[t, o] * Wd[o, k] for o in range(n_out))
            lora = s * sum(v[t][j] * Ad[j, k] for j in range(r))
            assert abs(dX[t, k] - (g + (lora / (1 - p) if keep[t, k] else 0.0))) < 1e-12
    for j in range(r):
        for k in range(n_in):
            assert abs(dA[j, k] - s * sum(v[t][j] * xt[t][k] for t in range(T))) < 1e-12
    for o in range(n_out):
        for j in range(r):
            assert abs(dB[o, j] - s * sum(Gd[t, o] * u[t][j] for t in range(T))) < 1e-12


def test_backward_matches_autograd():
    W, X, A, B, dY = _problem(2, T=5, n_in=32, n_out=6, r=3)
    alpha, r, p = 12.0, 3, 0.05
    keep = dense.unpack_keep(synth.keep_mask(4, 5, 32, p), 5, 32)
    Wt = torch.tensor(_f(W))
    Xt = torch.tensor(_f(X), requires_grad=True)
    At = torch.tensor(_f(A), requires_grad=True)
    Bt = torch.tensor(_f(B), requires_grad=True)
    Kt = torch.tensor(keep.astype(np.float64))
    drop = Xt * Kt / (1 - p)
    Yt = Xt @ Wt.T + (alpha / r) * (drop @ At.T) @ Bt.T
    Yt.backward(torch.tensor(_f(dY)))
    Y = dense.linear_fwd_dropout(W, X, A, B, alpha, r, keep, p)
    dX, dA, dB = dense.linear_bwd_dropout(W, X, dY, A, B, alpha, r, keep, p)
    assert np.allclose(Y, Yt.detach().numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(dX, Xt.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(dA, At.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(dB, Bt.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_no_dropout_and_all_dropped():
    W, X, A, B, dY = _problem(3, T=4, n_in=24, n_out=5, r=2)
    alpha, r = 4.0, 2
    ones = np.ones((4, 24), dtype=bool)
    assert np.array_equal(dense.linear_fwd_dropout(W, X, A, B, alpha, r, ones, 0.0),
                          dense.linear_fwd(W, X, A, B, alpha, r))
    for a, b in zip(dense.linear_bwd_dropout(W, X, dY, A, B, alpha, r, ones, 0.0),
                    dense.linear_bwd(W, X, dY, A, B, alpha, r)):
        assert np.array_equal(a, b)
    zeros = np.zeros((4, 24), dtype=bool)
    Y = dense.linear_fwd_dropout(W, X, A, B, alpha, r, zeros, 0.5)
    assert np.array_equal(Y, _f(X) @ _f(W).T)
    dX, dA, dB = dense.linear_bwd_dropout(W, X, dY, A, B, alpha, r, zeros, 0.5)
    assert np.array_equal(dX, _f(dY) @ _f(W)) and not dA.any() and not dB.any()


def test_inverted_scaling_keeps_the_expectation():
    # E[keep / (1 - p)] = 1: the adapter term averaged over many masks tends
    # to the undropped one (a missing or doubled 1/(1-p) fails by ~40%)
    W, X, A, B, _ = _problem(4, T=2, n_in=8, n_out=3, r=2)
    alpha, r, p = 2.0, 2, 0.3
    base = _f(X) @ _f(W).T
    full = dense.linear_fwd(W, X, A, B, alpha, r) - base
    rng = np.random.Generator(np.random.PCG64(11))
    acc = np.zeros_like(full)
    n = 20000
    for _ in range(n):
        keep = rng.random((2, 8)) >= p
        acc += dense.linear_fwd_dropout(W, X, A, B, alpha, r, keep, p) - base
    assert np.abs(acc / n - full).max() < 0.03 * np.abs(full).max()
