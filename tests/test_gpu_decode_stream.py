"""GPU parity of the weight-stream form of the small-token forward
(k_decode_stream: persistent workgroups over ranges of 16-row blocks, the
reduction dimension split over 8 waves, U = X A^T computed up front) against
the fp64 oracle, over the shapes that select its variants: the number of
chunk steps per row block (in / 2048), row blocks per workgroup (1 to 8),
token counts 1..16 up to the X capacity (T * in <= 65536), ranks 1..64, and
multi-projection calls whose workgroups straddle a projection boundary.

Acceptance: relative Frobenius error <= 2e-3 on the full Y; a repeated call is
bit-identical (the partial sums meet in a fixed order).  The calls take this
kernel from 2 row blocks per CU (512 of 16 rows) on."""

import numpy as np
import pytest
import torch

import synth
from oracle import dense as odense
from oracle import native as onative
from oracle import nf4 as onf4

from gpu_util import TOL, banner, dev_bf16, dev_f32, host_bits, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(seed, T, n_in, outs, r):
    ws = [synth.normal_f32(seed + 10 * i, (o, n_in), synth.W_STD) for i, o in enumerate(outs)]
    As = [synth.bf16_bits(synth.normal_f32(seed + 10 * i + 2, (r, n_in), 1.0 / n_in)) for i in range(len(outs))]
    Bs = [synth.bf16_bits(synth.normal_f32(seed + 10 * i + 3, (o, r), synth.B_STD)) for i, o in enumerate(outs)]
    X = synth.bf16_bits(synth.normal_f32(seed + 1, (T, n_in), 1.0))
    return ws, As, Bs, X


def _reference(ws, As, Bs, X, r, alpha):
    s = float(alpha) / float(r)
    Xw = odense.widen(X)
    cols = []
    for w, A, B in zip(ws, As, Bs):
        packed, aq, sc = onf4.quantize(w.reshape(-1), nearest=onative.nearest_level)
        wh = odense.widen(onf4.dequantize(packed, aq, sc).reshape(w.shape))
        cols.append(Xw @ wh.T + s * ((Xw @ odense.widen(A).T) @ odense.widen(B).T))
    return np.concatenate(cols, axis=1)


def _run(q, ws, As, Bs, X, r, alpha):
    Ws = [q.nf4_quantize_weight(dev_f32(w)) for w in ws]
    Xd = dev_bf16(X)
    Ad, Bd = [dev_bf16(a) for a in As], [dev_bf16(b) for b in Bs]
    if len(Ws) == 1:
        return Ws, Xd, Ad, Bd, q.qlora_linear_fwd(Ws[0], Xd, Ad[0], Bd[0], r, alpha)
    return Ws, Xd, Ad, Bd, q.qlora_linear_fwd_multi(Ws, Xd, Ad, Bd, r, alpha)


@pytest.mark.parametrize("T,n_in,outs,r", [
    (1, 4096, [8192], 16),           # 512 row blocks: 2 per workgroup, 2 chunk steps each
    (16, 4096, [8192], 16),          # X at full capacity (16 x 4096)
    (2, 8192, [8192], 1),            # 4 chunk steps per row block (4 in flight), rank 1
    (7, 4096, [16384], 64),          # 4 row blocks per workgroup, r = 64
    (3, 12288, [8192], 32),          # 6 chunk steps per row block (2 in flight)
    (16, 4096, [14336], 64),         # 8B gate: 896 row blocks, 3 or 4 per workgroup
    (1, 4096, [32768], 16),          # 2048 row blocks: 8 per workgroup
    (8, 8192, [28672], 64),          # 70B gate at T = 8: 7 row blocks per workgroup, full X
    (5, 4096, [4160, 4096], 16),     # workgroups straddling the projection boundary
    (11, 4096, [4096, 2048, 1024, 1024], 24),  # four projections
    (16, 4096, [8192, 4096, 4096], 16),        # three projections, 4 row blocks per workgroup
])
def test_stream_matches_oracle(T, n_in, outs, r):
    q = require_gpu()
    banner(f"stream T={T} in={n_in} outs={outs} r={r}")
    alpha = 2.0 * r
    ws, As, Bs, X = _inputs(4000 + T + n_in % 97, T, n_in, outs, r)
    Ws, Xd, Ad, Bd, Y = _run(q, ws, As, Bs, X, r, alpha)
    got = onf4.bf16_bits_to_f32(host_bits(Y)).astype(np.float64)
    err = odense.rel_frobenius(got, _reference(ws, As, Bs, X, r, alpha))
    print(f"  Y rel_frob={err:.3e}", flush=True)
    assert err <= TOL
    # a repeat call gives the same bits
    if len(Ws) == 1:
        Y2 = q.qlora_linear_fwd(Ws[0], Xd, Ad[0], Bd[0], r, alpha)
    else:
        Y2 = q.qlora_linear_fwd_multi(Ws, Xd, Ad, Bd, r, alpha)
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))


def test_stream_zero_weight_is_lora_only():
    # W = 0: Y = s U B^T exactly through the stream's epilogue
    q = require_gpu()
    banner("stream W=0")
    T, n_in, outs, r = 16, 4096, [8192], 16
    ws, As, Bs, X = _inputs(4200, T, n_in, outs, r)
    ws = [np.zeros_like(ws[0])]
    _, _, _, _, Y = _run(q, ws, As, Bs, X, r, 32.0)
    got = onf4.bf16_bits_to_f32(host_bits(Y)).astype(np.float64)
    assert odense.rel_frobenius(got, _reference(ws, As, Bs, X, r, 32.0)) <= TOL


def test_stream_one_hot_selects_columns_bit_exact():
    # X rows one-hot, B = 0: Y[t, :] = W_hat[:, i_t] bit for bit (the
    # dequantization inside the stream, in the lookup's element order)
    q = require_gpu()
    banner("stream one-hot")
    T, n_in, n_out, r = 16, 4096, 8192, 16
    w = synth.normal_f32(4300, (n_out, n_in), synth.W_STD)
    rng = np.random.default_rng(43)
    idx = rng.integers(0, n_in, T)
    X = np.zeros((T, n_in), dtype=np.uint16)
    X[np.arange(T), idx] = 0x3F80
    A = synth.bf16_bits(synth.normal_f32(4301, (r, n_in), 1.0 / n_in))
    W = q.nf4_quantize_weight(dev_f32(w))
    Y = q.qlora_linear_fwd(W, dev_bf16(X), dev_bf16(A), dev_bf16(np.zeros((n_out, r), np.uint16)), r, 32.0)
    packed, aq, sc = onf4.quantize(w, nearest=onative.nearest_level)
    w_hat = onf4.dequantize(packed, aq, sc).reshape(n_out, n_in)
    assert np.array_equal(host_bits(Y), w_hat[:, idx].T)


def test_stream_under_graph_replay():
    # the two launches (U, then the stream) captured in a graph, replayed with
    # eager calls on the same workspace in between: every replay bit-equal to
    # the eager result
    q = require_gpu()
    banner("stream graph replay")
    n_in, outs, r, alpha = 4096, [8192], 32, 64.0
    cases = [_inputs(4400 + T, T, n_in, outs, r) for T in (1, 9, 16)]
    W = q.nf4_quantize_weight(dev_f32(cases[0][0][0]))
    ins = [(dev_bf16(c[3]), dev_bf16(c[1][0]), dev_bf16(c[2][0])) for c in cases]
    wsb = q.make_workspace(max(q.qlora_workspace_bytes(T, n_in, outs[0], r, False) for T in (1, 9, 16)), "cuda")
    Ys = [torch.empty(X.shape[0], outs[0], dtype=torch.bfloat16, device="cuda") for X, _, _ in ins]
    eager = [host_bits(q.qlora_linear_fwd(W, X, A, B, r, alpha, Y=Y, ws=wsb)).copy()
             for (X, A, B), Y in zip(ins, Ys)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (X, A, B), Y in zip(ins, Ys):
            q.qlora_linear_fwd(W, X, A, B, r, alpha, Y=Y, ws=wsb)
    for rep in range(3):
        for Y in Ys:
            Y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, Y in enumerate(Ys):
            assert np.array_equal(host_bits(Y), eager[i]), (rep, i)
        X, A, B = ins[1]
        q.qlora_linear_fwd(W, X, A, B, r, alpha, Y=torch.empty_like(Ys[1]), ws=wsb)
        torch.cuda.synchronize()
