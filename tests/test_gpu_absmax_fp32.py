"""GPU parity of the linear calls on the 4.5-bit format (qlora_nf4_weight
flags = QLORA_NF4_ABSMAX_FP32: codes plus the exact fp32 absmax of each
64-weight block, no double quantization; paperclase "QLoRA", Parte 3, "Bits
por parametro") against the fp64 oracle, whose W_hat comes from the oracle's
own 4.5-bit quantize and dequantize.

Acceptance as for the double-quantized format: relative Frobenius error
<= 2e-3 for Y, dX, dA, dB; bit-exact where a one-hot operand selects a
column (forward) or a row (backward) of W_hat, which pins the fp32-absmax
dequantization on both the expanded forward weight and the backward's
transposed one."""

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
    B = synth.bf16_bits(synth.normal_f32(seed + 3, (n_out, r), synth.B_STD))
    dY = synth.bf16_bits(synth.normal_f32(seed + 4, (T, n_out), 1.0))
    return w, X, A, B, dY


def _weight(q, w):
    """Device 4.5-bit weight and the oracle's W_hat of the same tensor."""
    W = q.nf4_quantize_weight_nodq(dev_f32(w))
    assert W.flags == q.QLORA_NF4_ABSMAX_FP32 and W.absmax_q is None
    packed, absmax = onf4.quantize_nodq(w.reshape(-1), nearest=onative.nearest_level)
    w_hat = onf4.dequantize_nodq(packed, absmax).reshape(w.shape)
    return W, w_hat


def _f(bits):
    return onf4.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("T,n_in,n_out,r,alpha", [
    (1, 512, 768, 16, 32.0),       # one token (the double-quant format would take the small-token kernel)
    (16, 4096, 4096, 16, 32.0),    # decode-shaped q_proj
    (300, 512, 256, 8, 16.0),      # ragged T
    (2048, 1024, 640, 64, 128.0),  # large-token range
])
def test_fwd_bwd_match_oracle(T, n_in, n_out, r, alpha):
    q = require_gpu()
    banner(f"4.5-bit fwd+bwd T={T} in={n_in} out={n_out} r={r}")
    w, X, A, B, dY = _inputs(9000 + T, T, n_in, n_out, r)
    W, w_hat = _weight(q, w)
    Xd, Ad, Bd = dev_bf16(X), dev_bf16(A), dev_bf16(B)
    Y = q.qlora_linear_fwd(W, Xd, Ad, Bd, r, alpha)
    dX, dA, dB = q.qlora_linear_bwd(W, Xd, dev_bf16(dY), Ad, Bd, r, alpha)
    ref = odense.linear_fwd(w_hat, X, A, B, alpha, r)
    rdX, rdA, rdB = odense.linear_bwd(w_hat, X, dY, A, B, alpha, r)
    errs = {"Y": odense.rel_frobenius(_f(host_bits(Y)), ref),
            "dX": odense.rel_frobenius(_f(host_bits(dX)), rdX),
            "dA": odense.rel_frobenius(host(dA).astype(np.float64), rdA),
            "dB": odense.rel_frobenius(host(dB).astype(np.float64), rdB)}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= TOL for v in errs.values()), errs


@pytest.mark.parametrize("T", [1, 5, 40])
def test_one_hot_pins_both_directions(T):
    # X one-hot, B = 0: Y[t, :] = W_hat[:, i_t]; dY one-hot, A = 0:
    # dX[t, :] = W_hat[n_t, :], bit for bit
    q = require_gpu()
    banner(f"4.5-bit one-hot T={T}")
    n_in, n_out, r = 320, 192, 8
    w, _, A, B, _ = _inputs(9100 + T, T, n_in, n_out, r)
    W, w_hat = _weight(q, w)
    rng = np.random.default_rng(91 + T)
    ic, ir = rng.integers(0, n_in, T), rng.integers(0, n_out, T)
    X = np.zeros((T, n_in), dtype=np.uint16)
    X[np.arange(T), ic] = 0x3F80
    dY = np.zeros((T, n_out), dtype=np.uint16)
    dY[np.arange(T), ir] = 0x3F80
    Y = q.qlora_linear_fwd(W, dev_bf16(X), dev_bf16(A), dev_bf16(np.zeros_like(B)), r, 16.0)
    assert np.array_equal(host_bits(Y), w_hat[:, ic].T)
    dX, _, dB = q.qlora_linear_bwd(W, dev_bf16(X), dev_bf16(dY), dev_bf16(np.zeros_like(A)), dev_bf16(B), r,
                                   16.0)
    assert np.array_equal(host_bits(dX), w_hat[ir, :])
    assert np.all(host(dB) == 0)


def test_multi_projection_and_mixed_formats():
    q = require_gpu()
    banner("4.5-bit multi-projection")
    T, n_in, outs, r, alpha = 16, 512, [512, 128], 16, 32.0
    X = synth.bf16_bits(synth.normal_f32(9201, (T, n_in), 1.0))
    Ws, whs, As, Bs = [], [], [], []
    for i, o in enumerate(outs):
        w, _, A, B, _ = _inputs(9210 + 10 * i, T, n_in, o, r)
        W, wh = _weight(q, w)
        Ws.append(W), whs.append(wh), As.append(A), Bs.append(B)
    Y = q.qlora_linear_fwd_multi(Ws, dev_bf16(X), [dev_bf16(a) for a in As], [dev_bf16(b) for b in Bs], r, alpha)
    ref = np.concatenate([odense.linear_fwd(wh, X, A, B, alpha, r) for wh, A, B in zip(whs, As, Bs)], axis=1)
    err = odense.rel_frobenius(_f(host_bits(Y)), ref)
    print(f"  Y rel_frob={err:.3e}", flush=True)
    assert err <= TOL
    # the projections of one call must share the format
    Wdq = q.nf4_quantize_weight(dev_f32(_inputs(9210, T, n_in, outs[0], r)[0]))
    with pytest.raises(q.QloraError) as e:
        q.qlora_linear_fwd_multi([Wdq, Ws[1]], dev_bf16(X), [dev_bf16(a) for a in As], [dev_bf16(b) for b in Bs],
                                 r, alpha)
    assert q.STATUS[e.value.status] == "ERR_VALUE"


def test_dropout_and_merge_refusal():
    q = require_gpu()
    banner("4.5-bit dropout")
    T, n_in, n_out, r, alpha, p = 64, 512, 256, 16, 32.0, 0.1
    w, X, A, B, dY = _inputs(9300, T, n_in, n_out, r)
    W, w_hat = _weight(q, w)
    kb = synth.keep_mask(9301, T, n_in, p)
    kd = torch.from_numpy(kb).cuda()
    Y = q.qlora_linear_fwd_dropout(W, dev_bf16(X), kd, p, dev_bf16(A), dev_bf16(B), r, alpha)
    dX, dA, dB = q.qlora_linear_bwd_dropout(W, dev_bf16(X), dev_bf16(dY), kd, p, dev_bf16(A), dev_bf16(B), r,
                                            alpha)
    keep = odense.unpack_keep(kb, T, n_in)
    wh = odense.widen(w_hat)
    Yr = odense.linear_fwd_dropout(wh, X, A, B, alpha, r, keep, p)
    dXr, dAr, dBr = odense.linear_bwd_dropout(wh, X, dY, A, B, alpha, r, keep, p)
    errs = [odense.rel_frobenius(_f(host_bits(Y)), Yr), odense.rel_frobenius(_f(host_bits(dX)), dXr),
            odense.rel_frobenius(host(dA).astype(np.float64), dAr),
            odense.rel_frobenius(host(dB).astype(np.float64), dBr)]
    print("  " + " ".join(f"{v:.2e}" for v in errs), flush=True)
    assert all(v <= TOL for v in errs)
    with pytest.raises(q.QloraError) as e:
        q.qlora_merge(W, dev_bf16(A), dev_bf16(B), r, alpha)
    assert q.STATUS[e.value.status] == "ERR_VALUE"
