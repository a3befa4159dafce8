"""GPU parity of the backward's fused dX route: given a workspace of
qlora_workspace_bytes_bwd_min (no room for the expanded W_hat^T), the dX GEMM
reads the NF4 codes and dequantizes each weight tile, transposed, while it
stages it into LDS (paperclase "QLoRA", Parte 4: dX = (W_hat + s B A)^T dY,
with W_hat built, used and discarded).

Checks:
- against the fp64 oracle (relative Frobenius <= 2e-3 for dX, dA, dB) at
  small ragged shapes, full tensors;
- against the expanded route on the same inputs: dX bit for bit (both routes
  feed the same bf16 W_hat values to the same MFMA sequence), dA and dB bit for
  bit too (token-slice sums added in a fixed order), at shapes that run every
  kernel form (the 128 x 128 kernel with a partial column tile, the 256-column
  kernel with 128- and 256-row tiles), several projections, and dropout;
- one-hot dY rows select rows of W_hat bit for bit through the fused route;
- split-K (grids below one workgroup per CU, forward and backward, both
  routes): oracle parity, repeated calls bit for bit, one-hot pins, several
  projections, dropout;
- dA and dB repeated bit for bit, and the large-token forward / backward
  replayed from a captured graph bit for bit."""

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
    ws = [synth.normal_f32(seed + 10 * i, (o, n_in), synth.W_STD) for i, o in enumerate(outs)]
    As = [synth.bf16_bits(synth.normal_f32(seed + 10 * i + 2, (r, n_in), 1.0 / n_in)) for i in range(len(outs))]
    Bs = [synth.bf16_bits(synth.normal_f32(seed + 10 * i + 3, (o, r), 0.05)) for i, o in enumerate(outs)]
    X = synth.bf16_bits(synth.normal_f32(seed + 1, (T, n_in), 1.0))
    dY = synth.bf16_bits(synth.normal_f32(seed + 4, (T, sum(outs)), 1.0))
    return ws, As, Bs, X, dY


def _w_hat(w):
    packed, aq, sc = onf4.quantize(w, nearest=onative.nearest_level)
    return onf4.dequantize(packed, aq, sc).reshape(w.shape)


def _min_ws(q, T, n_in, outs, r, dropout=False):
    need = q.qlora_workspace_bytes_bwd_min(T, n_in, outs, r, dropout)
    full = q.qlora_workspace_bytes_flags(T, n_in, outs, r, True, dropout)
    assert 0 < need < full, (need, full)
    return q.make_workspace(need, "cuda")


def _both(q, T, n_in, outs, r, alpha, seed):
    """dX, dA, dB of the multi call through the fused route and the expanded one."""
    ws, As, Bs, X, dY = _inputs(seed, T, n_in, outs, r)
    Ws = [q.nf4_quantize_weight(dev_f32(w)) for w in ws]
    Xd, dYd = dev_bf16(X), dev_bf16(dY)
    Ad, Bd = [dev_bf16(a) for a in As], [dev_bf16(b) for b in Bs]
    fused = q.qlora_linear_bwd_multi(Ws, Xd, dYd, Ad, Bd, r, alpha, ws=_min_ws(q, T, n_in, outs, r))
    fused = (host_bits(fused[0]), [host(a) for a in fused[1]], [host(b) for b in fused[2]])
    full = q.qlora_linear_bwd_multi(Ws, Xd, dYd, Ad, Bd, r, alpha)
    full = (host_bits(full[0]), [host(a) for a in full[1]], [host(b) for b in full[2]])
    return (ws, As, Bs, X, dY), fused, full


def _same_route_result(fused, full):
    assert np.array_equal(fused[0], full[0]), "dX differs between the fused and the expanded route"
    for a, b in zip(fused[1] + fused[2], full[1] + full[2]):
        # the same gradient kernels, their token slices added in a fixed order
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "dA / dB differ between the routes"


@pytest.mark.parametrize("T,n_in,outs,r,alpha", [
    (37, 192, [320], 12, 24.0),       # ragged T, 128 x 128 kernel, 192 columns: half a tile past `in`
    (200, 512, [128], 64, 16.0),      # ragged tail of a 128-row tile, r = 64
    (300, 320, [512, 256], 16, 32.0), # two projections: a K-step switches weight mid-call
])
def test_fused_route_matches_oracle(T, n_in, outs, r, alpha):
    q = require_gpu()
    banner(f"fused dX vs oracle T={T} in={n_in} outs={outs} r={r}")
    (ws, As, Bs, X, dY), fused, full = _both(q, T, n_in, outs, r, alpha, 1300 + T)
    _same_route_result(fused, full)
    w_hats = [_w_hat(w) for w in ws]
    rdX = np.zeros((T, n_in))
    col = 0
    for i, (w_hat, o) in enumerate(zip(w_hats, outs)):
        g = np.ascontiguousarray(dY[:, col:col + o])
        dXi, rdA, rdB = odense.linear_bwd(w_hat, X, g, As[i], Bs[i], alpha, r)
        rdX += dXi
        assert odense.rel_frobenius(fused[1][i].astype(np.float64), rdA) <= TOL
        assert odense.rel_frobenius(fused[2][i].astype(np.float64), rdB) <= TOL
        col += o
    err = odense.rel_frobenius(onf4.bf16_bits_to_f32(fused[0]).astype(np.float64), rdX)
    print(f"  dX rel_frob={err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("T,n_in,outs,r,alpha", [
    (4096, 4096, [14336], 64, 128.0),          # 8B MLP gate: 256 x 256 tiles, K = 14336
    (1024, 8192, [1024], 16, 32.0),            # 128 x 256 tiles (8 x 32 of them)
    (4096, 4096, [4096, 1024, 1024], 16, 32.0),  # 8B q|k|v: 256 x 256 tiles over three projections
    (8192, 4096, [1024], 16, 32.0),            # 8B attention k: 32 x 16 tiles, K = 1024
    (4096, 8192, [28672], 64, 16.0),           # 70B MLP gate: K = 28672
    (4096, 28672, [8192], 64, 16.0),           # 70B MLP down: 16 x 112 tiles
])
def test_fused_route_equals_expanded_route(T, n_in, outs, r, alpha):
    q = require_gpu()
    banner(f"fused dX vs expanded T={T} in={n_in} outs={outs} r={r}")
    _, fused, full = _both(q, T, n_in, outs, r, alpha, 1400 + T % 97)
    _same_route_result(fused, full)


@pytest.mark.parametrize("T,n_in,n_out,r,p", [(600, 1024, 512, 16, 0.1), (4096, 4096, 4096, 16, 0.05)])
def test_fused_route_with_dropout(T, n_in, n_out, r, p):
    q = require_gpu()
    banner(f"fused dX with dropout T={T} in={n_in} out={n_out} p={p}")
    (w,), (A,), (B,), X, dY = _inputs(1500 + T % 89, T, n_in, [n_out], r)
    rng = np.random.Generator(np.random.PCG64(1501))
    keep = np.packbits(rng.random((T, n_in)) >= p, axis=1, bitorder="little")
    W = q.nf4_quantize_weight(dev_f32(w))
    Xd, dYd, Ad, Bd = dev_bf16(X), dev_bf16(dY), dev_bf16(A), dev_bf16(B)
    K = torch.from_numpy(np.ascontiguousarray(keep)).cuda()
    f = q.qlora_linear_bwd_dropout(W, Xd, dYd, K, p, Ad, Bd, r, 2.0 * r,
                                   ws=_min_ws(q, T, n_in, [n_out], r, dropout=True))
    f = (host_bits(f[0]), [host(f[1])], [host(f[2])])
    e = q.qlora_linear_bwd_dropout(W, Xd, dYd, K, p, Ad, Bd, r, 2.0 * r)
    e = (host_bits(e[0]), [host(e[1])], [host(e[2])])
    _same_route_result(f, e)


def _one_hot(n, idx):
    m = np.zeros((len(idx), n), dtype=np.uint16)
    m[np.arange(len(idx)), idx] = 0x3F80  # bf16 1.0
    return m


@pytest.mark.parametrize("T,n_out,n_in", [
    (70, 192, 320),      # 128 x 128 kernel, partial column tile
    (2048, 512, 8192),   # 256 x 256 tiles (8 x 32)
    (1024, 512, 8192),   # 128 x 256 tiles (8 x 32)
])
def test_fused_route_one_hot_rows_bit_exact(T, n_out, n_in):
    # dY rows one-hot and A = 0: dX[t, :] = W_hat[n_t, :] exactly
    q = require_gpu()
    banner(f"fused dX one-hot T={T} out={n_out} in={n_in}")
    r = 16
    w = synth.normal_f32(78_000 + n_out + n_in, (n_out, n_in), synth.W_STD)
    rng = np.random.default_rng(T + n_in)
    gi = rng.integers(0, n_out, T)
    X = synth.bf16_bits(synth.normal_f32(7, (T, n_in), 1.0))
    B = synth.bf16_bits(synth.normal_f32(6, (n_out, r), synth.B_STD))
    W = q.nf4_quantize_weight(dev_f32(w))
    dX, dA, dB = q.qlora_linear_bwd(W, dev_bf16(X), dev_bf16(_one_hot(n_out, gi)),
                                    dev_bf16(np.zeros((r, n_in), np.uint16)), dev_bf16(B), r, 32.0,
                                    ws=_min_ws(q, T, n_in, [n_out], r))
    assert np.array_equal(host_bits(dX), _w_hat(w)[gi, :])
    assert np.all(host(dB) == 0)  # U = X A^T = 0


# ------------------------------------------------------------------ split-K
# Grids of 128 x 128 tiles below one workgroup per CU (e.g. 64 tokens against
# 4096 output columns: 32 tiles) split K into up to 8 ranges of fp32 partials,
# summed in order and rounded once.

def _single(seed, T, n_out, n_in, r):
    (w,), (A,), (B,), X, dY = _inputs(seed, T, n_in, [n_out], r)
    return w, A, B, X, dY


@pytest.mark.parametrize("T,n_out,n_in,r", [
    (64, 4096, 4096, 16),    # fwd: 32 tiles, 8 splits of 8 K-steps; dX: 32 tiles, 8 splits
    (64, 14336, 4096, 64),   # dX over K = 14336: 8 splits of 28 K-steps
    (100, 1024, 640, 16),    # ragged T, partial column tile, 2 splits of 8 K-steps (dX)
])
def test_split_k_matches_oracle_and_repeats(T, n_out, n_in, r):
    q = require_gpu()
    banner(f"split-K T={T} out={n_out} in={n_in} r={r}")
    alpha = 2.0 * r
    w, A, B, X, dY = _single(1600 + T, T, n_out, n_in, r)
    W = q.nf4_quantize_weight(dev_f32(w))
    Xd, dYd, Ad, Bd = dev_bf16(X), dev_bf16(dY), dev_bf16(A), dev_bf16(B)
    w_hat = _w_hat(w)
    Y = host_bits(q.qlora_linear_fwd(W, Xd, Ad, Bd, r, alpha))
    ref = odense.linear_fwd(w_hat, X, A, B, alpha, r)
    ey = odense.rel_frobenius(onf4.bf16_bits_to_f32(Y).astype(np.float64), ref)
    rdX, rdA, rdB = odense.linear_bwd(w_hat, X, dY, A, B, alpha, r)
    for ws in (None, _min_ws(q, T, n_in, [n_out], r)):
        dX, dA, dB = q.qlora_linear_bwd(W, Xd, dYd, Ad, Bd, r, alpha, ws=ws)
        ex = odense.rel_frobenius(onf4.bf16_bits_to_f32(host_bits(dX)).astype(np.float64), rdX)
        ea = odense.rel_frobenius(host(dA).astype(np.float64), rdA)
        eb = odense.rel_frobenius(host(dB).astype(np.float64), rdB)
        print(f"  {'min' if ws is not None else 'full'} ws: Y={ey:.3e} dX={ex:.3e} dA={ea:.3e} dB={eb:.3e}",
              flush=True)
        assert max(ey, ex, ea, eb) <= TOL
        # the partial sums are added in a fixed order: a second call repeats dX bit for bit
        dX2 = q.qlora_linear_bwd(W, Xd, dYd, Ad, Bd, r, alpha, ws=ws)[0]
        assert np.array_equal(host_bits(dX2), host_bits(dX))
    assert np.array_equal(host_bits(q.qlora_linear_fwd(W, Xd, Ad, Bd, r, alpha)), Y)


def test_split_k_routes_equal():
    # 8B gate dX at 64 tokens: both routes split K the same way, dX bit for bit
    q = require_gpu()
    banner("split-K fused vs expanded T=64 in=4096 out=14336")
    _, fused, full = _both(q, 64, 4096, [14336], 64, 128.0, 1700)
    _same_route_result(fused, full)


@pytest.mark.parametrize("T,n_in,outs", [(64, 4096, [4096, 1024, 1024]), (64, 1024, [4160, 4032])])
def test_split_k_multi_forward(T, n_in, outs):
    # one launch over q|k|v-like stacked projections, and one launch per
    # projection where a 128-column tile would straddle two
    q = require_gpu()
    banner(f"split-K multi fwd T={T} in={n_in} outs={outs}")
    r, alpha = 16, 32.0
    ws, As, Bs, X, _ = _inputs(1800 + len(outs), T, n_in, outs, r)
    Ws = [q.nf4_quantize_weight(dev_f32(w)) for w in ws]
    Y = host_bits(q.qlora_linear_fwd_multi(Ws, dev_bf16(X), [dev_bf16(a) for a in As],
                                           [dev_bf16(b) for b in Bs], r, alpha))
    col = 0
    for w, A, B, o in zip(ws, As, Bs, outs):
        ref = odense.linear_fwd(_w_hat(w), X, A, B, alpha, r)
        got = onf4.bf16_bits_to_f32(np.ascontiguousarray(Y[:, col:col + o])).astype(np.float64)
        assert odense.rel_frobenius(got, ref) <= TOL
        col += o


@pytest.mark.parametrize("T,n_out,n_in", [(64, 512, 8192), (64, 8192, 512)])
def test_split_k_one_hot_bit_exact(T, n_out, n_in):
    # one-hot X (B = 0): Y[t] = W_hat[:, i_t]; one-hot dY (A = 0): dX[t] = W_hat[n_t]
    # -- the one nonzero product lands in one split, the others add exact zeros
    q = require_gpu()
    banner(f"split-K one-hot T={T} out={n_out} in={n_in}")
    r = 16
    w = synth.normal_f32(79_000 + n_out, (n_out, n_in), synth.W_STD)
    rng = np.random.default_rng(T + n_out)
    xi, gi = rng.integers(0, n_in, T), rng.integers(0, n_out, T)
    A = synth.bf16_bits(synth.normal_f32(5, (r, n_in), 1.0 / n_in))
    B = synth.bf16_bits(synth.normal_f32(6, (n_out, r), synth.B_STD))
    W = q.nf4_quantize_weight(dev_f32(w))
    w_hat = _w_hat(w)
    Y = q.qlora_linear_fwd(W, dev_bf16(_one_hot(n_in, xi)), dev_bf16(A), dev_bf16(np.zeros_like(B)), r, 32.0)
    assert np.array_equal(host_bits(Y), w_hat[:, xi].T)
    Xr = synth.bf16_bits(synth.normal_f32(7, (T, n_in), 1.0))
    for ws in (None, _min_ws(q, T, n_in, [n_out], r)):
        dX = q.qlora_linear_bwd(W, dev_bf16(Xr), dev_bf16(_one_hot(n_out, gi)), dev_bf16(np.zeros_like(A)),
                                dev_bf16(B), r, 32.0, ws=ws)[0]
        assert np.array_equal(host_bits(dX), w_hat[gi, :])


def test_split_k_with_dropout():
    q = require_gpu()
    T, n_in, n_out, r, p = 64, 1024, 4096, 16, 0.1
    banner(f"split-K dropout T={T} in={n_in} out={n_out}")
    w, A, B, X, dY = _single(1900, T, n_out, n_in, r)
    rng = np.random.Generator(np.random.PCG64(1901))
    keep_bool = rng.random((T, n_in)) >= p
    keep = np.packbits(keep_bool, axis=1, bitorder="little")
    W = q.nf4_quantize_weight(dev_f32(w))
    K = torch.from_numpy(np.ascontiguousarray(keep)).cuda()
    args = (dev_bf16(X), dev_bf16(dY), K, p, dev_bf16(A), dev_bf16(B), r, 32.0)
    rdX, rdA, rdB = odense.linear_bwd_dropout(_w_hat(w), X, dY, A, B, 32.0, r, keep_bool, p)
    for ws in (None, _min_ws(q, T, n_in, [n_out], r, dropout=True)):
        dX, dA, dB = q.qlora_linear_bwd_dropout(W, *args, ws=ws)
        ex = odense.rel_frobenius(onf4.bf16_bits_to_f32(host_bits(dX)).astype(np.float64), rdX)
        assert ex <= TOL, ex
        assert odense.rel_frobenius(host(dA).astype(np.float64), rdA) <= TOL
        assert odense.rel_frobenius(host(dB).astype(np.float64), rdB) <= TOL


@pytest.mark.parametrize("T,n_in,outs,r", [(300, 1024, [640], 16), (4096, 4096, [14336], 64),
                                           (4096, 4096, [4096, 1024, 1024], 16)])
def test_gradients_reproducible(T, n_in, outs, r):
    # from 17 tokens on dA and dB are token-slice sums written to the workspace
    # and added in a fixed order: two identical calls agree bit for bit
    q = require_gpu()
    banner(f"dA/dB repeat T={T} in={n_in} outs={outs} r={r}")
    ws, As, Bs, X, dY = _inputs(2000 + T % 91, T, n_in, outs, r)
    Ws = [q.nf4_quantize_weight(dev_f32(w)) for w in ws]
    args = (Ws, dev_bf16(X), dev_bf16(dY), [dev_bf16(a) for a in As], [dev_bf16(b) for b in Bs], r, 2.0 * r)
    first = q.qlora_linear_bwd_multi(*args)
    first = [host(t).copy() for t in first[1] + first[2]]
    again = q.qlora_linear_bwd_multi(*args)
    for a, b in zip(first, [host(t) for t in again[1] + again[2]]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_gradients_reproducible_with_dropout():
    q = require_gpu()
    T, n_in, n_out, r, p = 600, 1024, 512, 16, 0.1
    banner(f"dA/dB repeat with dropout T={T}")
    (w,), (A,), (B,), X, dY = _inputs(2100, T, n_in, [n_out], r)
    keep = np.packbits(np.random.Generator(np.random.PCG64(2101)).random((T, n_in)) >= p, axis=1,
                       bitorder="little")
    W = q.nf4_quantize_weight(dev_f32(w))
    K = torch.from_numpy(np.ascontiguousarray(keep)).cuda()
    args = (W, dev_bf16(X), dev_bf16(dY), K, p, dev_bf16(A), dev_bf16(B), r, 32.0)
    a1 = [host(t).copy() for t in q.qlora_linear_bwd_dropout(*args)[1:]]
    a2 = [host(t) for t in q.qlora_linear_bwd_dropout(*args)[1:]]
    for a, b in zip(a1, a2):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_large_token_paths_under_graph_replay():
    # A captured graph replays forwards and backwards that use the split-K
    # partials, the fused dX route and the gradients' slice sums (every launch a
    # kernel, no memory-set nodes), sharing workspaces with eager calls made
    # between the replays; every replay must equal the eager results bit for bit.
    q = require_gpu()
    banner("graph replay of the large-token forward / backward")
    n_out, n_in, r, alpha = 4096, 4096, 16, 32.0
    (w,), (A,), (B,), X, dY = _inputs(2200, 300, n_in, [n_out], r)
    W = q.nf4_quantize_weight(dev_f32(w))
    Ad, Bd = dev_bf16(A), dev_bf16(B)
    Xs = {T: dev_bf16(X[:T]) for T in (64, 300)}
    dYs = {T: dev_bf16(dY[:T]) for T in (64, 300)}
    wsf = q.make_workspace(max(q.qlora_workspace_bytes(T, n_in, n_out, r, False) for T in (64, 300)), "cuda")
    wsb = q.make_workspace(max(q.qlora_workspace_bytes(T, n_in, n_out, r, True) for T in (64, 300)), "cuda")
    wsm = q.make_workspace(max(q.qlora_workspace_bytes_bwd_min(T, n_in, [n_out], r) for T in (64, 300)), "cuda")
    calls = []  # (outputs, launcher)
    for T in (64, 300):
        Y = torch.empty(T, n_out, dtype=torch.bfloat16, device="cuda")
        calls.append(([Y], lambda T=T, Y=Y: q.qlora_linear_fwd(W, Xs[T], Ad, Bd, r, alpha, Y=Y, ws=wsf)))
        for ws in (wsb, wsm):
            o = [torch.empty(T, n_in, dtype=torch.bfloat16, device="cuda"),
                 torch.empty(r, n_in, dtype=torch.float32, device="cuda"),
                 torch.empty(n_out, r, dtype=torch.float32, device="cuda")]
            calls.append((o, lambda T=T, o=o, ws=ws: q.qlora_linear_bwd(W, Xs[T], dYs[T], Ad, Bd, r, alpha, *o, ws=ws)))
    bits = lambda t: host(t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)).copy()
    eager = []
    for o, f in calls:
        f()
        eager.append([bits(t) for t in o])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, f in calls:
            f()
    for rep in range(3):
        for o, _ in calls:
            for t in o:
                t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, _) in enumerate(calls):
            for t, ref in zip(o, eager[k]):
                assert np.array_equal(bits(t), ref), (rep, k)
        calls[2][1]()  # eager work on the shared workspaces between replays
        calls[4][1]()
        torch.cuda.synchronize()


@pytest.mark.parametrize("T,n_in,outs,r", [
    (1536, 4096, [14336], 64),             # 6 x 56 tiles of 256
    (4096, 14336, [4096], 64),             # 8B down, K = 14336
    (4096, 4096, [4096, 1024, 1024], 16),  # q|k|v stacked in one launch
    (600, 1024, [4160, 4032], 8),          # 128 x 128 tiles, one launch per projection, split-K
])
def test_forward_routes_equal(T, n_in, outs, r):
    # from 512 tokens on the forward expands W_hat when the workspace holds it
    # and dequantizes in the GEMM's staging otherwise: same bf16 W_hat, same
    # MFMA sequence, so Y is the same bit for bit
    q = require_gpu()
    banner(f"forward routes T={T} in={n_in} outs={outs} r={r}")
    ws, As, Bs, X, _ = _inputs(2300 + T % 83, T, n_in, outs, r)
    Ws = [q.nf4_quantize_weight(dev_f32(w)) for w in ws]
    args = (Ws, dev_bf16(X), [dev_bf16(a) for a in As], [dev_bf16(b) for b in Bs], r, 2.0 * r)
    need = q.qlora_workspace_bytes_fwd_min(T, n_in, outs, r)
    full = q.qlora_workspace_bytes_multi(T, n_in, outs, r, False)
    assert 0 < need < full and full - need >= sum(outs) * n_in * 2
    Yf = host_bits(q.qlora_linear_fwd_multi(*args, ws=q.make_workspace(need, "cuda")))
    Ye = host_bits(q.qlora_linear_fwd_multi(*args, ws=q.make_workspace(full, "cuda")))
    assert np.array_equal(Yf, Ye)
