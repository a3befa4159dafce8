"""GPU parity of the small-token backward (T <= 16, no dropout), three
launches: the dX row splits stream the NF4 codes once (W_hat only in LDS)
next to the chunked rank-r reductions U = X A^T and V = dY B; then sU and
sV; then dX (the splits added in order plus the adapter term, one rounding),
dA and dB (each element written once) -- against the fp64 oracle at the 8B
MLP shapes and for a multi-projection call, plus bit-exact one-hot pins
through the row splits and a repeat-call reproducibility check.

Acceptance: relative Frobenius error <= 2e-3 on dX, dA, dB (full tensors);
one-hot dY rows with A = 0 select rows of W_hat bit for bit; a repeated call
gives the same dX, dA and dB bits."""

import numpy as np
import pytest

import synth
from oracle import dense as odense
from oracle import native as onative
from oracle import nf4 as onf4

from gpu_util import TOL, banner, dev_bf16, dev_f32, host, host_bits, require_gpu

pytestmark = pytest.mark.gpu


def _case(seed, T, n_in, outs, r):
    ws = [synth.normal_f32(seed + 10 * i, (o, n_in), synth.W_STD) for i, o in enumerate(outs)]
    As = [synth.bf16_bits(synth.normal_f32(seed + 10 * i + 2, (r, n_in), 1.0 / n_in)) for i in range(len(outs))]
    Bs = [synth.bf16_bits(synth.normal_f32(seed + 10 * i + 3, (o, r), synth.B_STD)) for i, o in enumerate(outs)]
    X = synth.bf16_bits(synth.normal_f32(seed + 1, (T, n_in), 1.0))
    dY = synth.bf16_bits(synth.normal_f32(seed + 4, (T, sum(outs)), 1.0))
    return ws, As, Bs, X, dY


def _w_hat(w):
    packed, aq, sc = onf4.quantize(w.reshape(-1), nearest=onative.nearest_level)
    return onf4.dequantize(packed, aq, sc).reshape(w.shape)


@pytest.mark.parametrize("T,n_in,n_out,r", [
    (1, 4096, 14336, 64),    # 8B gate: 224 row chunks per column strip
    (16, 4096, 14336, 64),
    (7, 14336, 4096, 64),    # 8B down: 224 column strips
    (16, 4096, 4096, 16),    # decode-shaped q_proj
])
def test_small_token_bwd_matches_oracle(T, n_in, n_out, r):
    q = require_gpu()
    banner(f"small-token bwd T={T} in={n_in} out={n_out} r={r}")
    alpha = 2.0 * r
    ws, As, Bs, X, dY = _case(12000 + T + n_out % 97, T, n_in, [n_out], r)
    W = q.nf4_quantize_weight(dev_f32(ws[0]))
    Xd, dYd, Ad, Bd = dev_bf16(X), dev_bf16(dY), dev_bf16(As[0]), dev_bf16(Bs[0])
    dX, dA, dB = q.qlora_linear_bwd(W, Xd, dYd, Ad, Bd, r, alpha)
    rdX, rdA, rdB = odense.linear_bwd(_w_hat(ws[0]), X, dY, As[0], Bs[0], alpha, r)
    errs = [odense.rel_frobenius(onf4.bf16_bits_to_f32(host_bits(dX)).astype(np.float64), rdX),
            odense.rel_frobenius(host(dA).astype(np.float64), rdA),
            odense.rel_frobenius(host(dB).astype(np.float64), rdB)]
    print(f"  dX={errs[0]:.2e} dA={errs[1]:.2e} dB={errs[2]:.2e}", flush=True)
    assert all(e <= TOL for e in errs), errs
    dX2, dA2, dB2 = q.qlora_linear_bwd(W, Xd, dYd, Ad, Bd, r, alpha)
    assert np.array_equal(host_bits(dX2), host_bits(dX))
    # each element of dA and dB is written once (no atomics): reproducible too
    assert np.array_equal(host(dA2), host(dA)) and np.array_equal(host(dB2), host(dB))


def test_small_token_bwd_multi_projection():
    # q|k|v stacked: dY's columns are the three projections' side by side
    q = require_gpu()
    banner("small-token bwd multi")
    T, n_in, outs, r, alpha = 11, 4096, [4096, 1024, 1024], 16, 32.0
    ws, As, Bs, X, dY = _case(12500, T, n_in, outs, r)
    Ws = [q.nf4_quantize_weight(dev_f32(w)) for w in ws]
    dX, dAs, dBs = q.qlora_linear_bwd_multi(Ws, dev_bf16(X), dev_bf16(dY), [dev_bf16(a) for a in As],
                                            [dev_bf16(b) for b in Bs], r, alpha)
    rdX = np.zeros((T, n_in))
    off = 0
    for i, (w, A, B) in enumerate(zip(ws, As, Bs)):
        g = dY[:, off:off + outs[i]]
        rX, rA, rB = odense.linear_bwd(_w_hat(w), X, g, A, B, alpha, r)
        rdX += rX
        assert odense.rel_frobenius(host(dAs[i]).astype(np.float64), rA) <= TOL
        assert odense.rel_frobenius(host(dBs[i]).astype(np.float64), rB) <= TOL
        off += outs[i]
    err = odense.rel_frobenius(onf4.bf16_bits_to_f32(host_bits(dX)).astype(np.float64), rdX)
    print(f"  dX={err:.2e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("T,n_in,outs,r", [
    (5, 320, [192], 200),       # ranks in a 64 + 64 + 64 + 8 loop, a 64-wide last U chunk, a 64-row V chunk
    (1, 64, [64], 1),           # one strip, one 64-row chunk, rank 1
    (13, 320, [192, 64], 24),   # two projections: V chunks and dB rows per projection
    (16, 1024, [128, 1024, 64], 256),  # the largest rank
])
def test_small_token_bwd_edge_shapes(T, n_in, outs, r):
    q = require_gpu()
    banner(f"small-token bwd edges T={T} in={n_in} outs={outs} r={r}")
    alpha = 1.5 * r
    ws, As, Bs, X, dY = _case(13000 + T + r, T, n_in, outs, r)
    Ws = [q.nf4_quantize_weight(dev_f32(w)) for w in ws]
    if len(outs) == 1:
        dX, dA, dB = q.qlora_linear_bwd(Ws[0], dev_bf16(X), dev_bf16(dY), dev_bf16(As[0]), dev_bf16(Bs[0]), r,
                                        alpha)
        dAs, dBs = [dA], [dB]
    else:
        dX, dAs, dBs = q.qlora_linear_bwd_multi(Ws, dev_bf16(X), dev_bf16(dY), [dev_bf16(a) for a in As],
                                                [dev_bf16(b) for b in Bs], r, alpha)
    rdX = np.zeros((T, n_in))
    off = 0
    for i, (w, A, B) in enumerate(zip(ws, As, Bs)):
        rX, rA, rB = odense.linear_bwd(_w_hat(w), X, dY[:, off:off + outs[i]], A, B, alpha, r)
        rdX += rX
        ea = odense.rel_frobenius(host(dAs[i]).astype(np.float64), rA)
        eb = odense.rel_frobenius(host(dBs[i]).astype(np.float64), rB)
        assert ea <= TOL and eb <= TOL, (i, ea, eb)
        off += outs[i]
    err = odense.rel_frobenius(onf4.bf16_bits_to_f32(host_bits(dX)).astype(np.float64), rdX)
    print(f"  dX={err:.2e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("T,n_out", [(3, 14336), (16, 2048)])
def test_small_token_bwd_one_hot_bit_exact(T, n_out):
    # dY rows one-hot, A = 0: dX[t] = W_hat[row_t] exactly, whichever row
    # split holds the row
    q = require_gpu()
    banner(f"small-token bwd one-hot T={T} out={n_out}")
    n_in, r = 4096, 16
    ws, As, Bs, X, _ = _case(12700 + T, T, n_in, [n_out], r)
    W = q.nf4_quantize_weight(dev_f32(ws[0]))
    rng = np.random.default_rng(127 + T)
    rows = rng.integers(0, n_out, T)
    dY = np.zeros((T, n_out), dtype=np.uint16)
    dY[np.arange(T), rows] = 0x3F80
    dX, _, dB = q.qlora_linear_bwd(W, dev_bf16(X), dev_bf16(dY), dev_bf16(np.zeros_like(As[0])),
                                   dev_bf16(Bs[0]), r, 32.0)
    assert np.array_equal(host_bits(dX), _w_hat(ws[0])[rows, :])
    assert np.all(host(dB) == 0)
