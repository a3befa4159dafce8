"""GPU parity of qlora_linear_fwd / qlora_linear_bwd against the fp64 oracle.

Acceptance: relative Frobenius error <= 2e-3 for Y, dX, dA, dB separately;
bit-exact where the result is a single product (one-hot activations select a
column of W_hat, which pins the dequantization inside the fused kernels)."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import dense as odense
from oracle import native as onative
from oracle import nf4 as onf4

from gpu_util import TOL, banner, dev_bf16, dev_f32, host, host_bits, require_gpu

pytestmark = pytest.mark.gpu


def _make(wid, proj, T, n_out, n_in, r, seed_shift=0, w_scale=None):
    """Seeded inputs of one projection; returns host arrays and device tensors."""
    w = synth.normal_f32(synth.seed_for(wid, proj, "W") + seed_shift, (n_out, n_in), synth.W_STD)
    if w_scale is not None:
        w = w * np.float32(w_scale)
    X = synth.bf16_bits(synth.normal_f32(synth.seed_for(wid, proj, "X") + seed_shift, (T, n_in), 1.0))
    A = synth.bf16_bits(synth.normal_f32(synth.seed_for(wid, proj, "A") + seed_shift, (r, n_in), 1.0 / n_in))
    B = synth.bf16_bits(synth.normal_f32(synth.seed_for(wid, proj, "B") + seed_shift, (n_out, r), synth.B_STD))
    dY = synth.bf16_bits(synth.normal_f32(synth.seed_for(wid, proj, "dY") + seed_shift, (T, n_out), 1.0))
    return dict(w=w, X=X, A=A, B=B, dY=dY)


def _quantize(q, w_host):
    W = q.nf4_quantize_weight(dev_f32(w_host))
    packed, aq, sc = onf4.quantize(w_host, nearest=onative.nearest_level)
    w_hat = onf4.dequantize(packed, aq, sc).reshape(w_host.shape)
    return W, w_hat


def _fwd(q, W, h, r, alpha):
    return q.qlora_linear_fwd(W, dev_bf16(h["X"]), dev_bf16(h["A"]), dev_bf16(h["B"]), r, alpha)


def _bwd(q, W, h, r, alpha):
    return q.qlora_linear_bwd(W, dev_bf16(h["X"]), dev_bf16(h["dY"]), dev_bf16(h["A"]),
                              dev_bf16(h["B"]), r, alpha)


def _check_fwd(Y, w_hat, h, r, alpha, what):
    ref = odense.linear_fwd(w_hat, h["X"], h["A"], h["B"], alpha, r)
    got = onf4.bf16_bits_to_f32(host_bits(Y)).astype(np.float64)
    err = odense.rel_frobenius(got, ref)
    print(f"  {what}: Y rel_frob={err:.3e}", flush=True)
    assert err <= TOL, (what, err)


def _check_bwd(res, w_hat, h, r, alpha, what):
    dX, dA, dB = res
    rdX, rdA, rdB = odense.linear_bwd(w_hat, h["X"], h["dY"], h["A"], h["B"], alpha, r)
    e1 = odense.rel_frobenius(onf4.bf16_bits_to_f32(host_bits(dX)).astype(np.float64), rdX)
    e2 = odense.rel_frobenius(host(dA).astype(np.float64), rdA)
    e3 = odense.rel_frobenius(host(dB).astype(np.float64), rdB)
    print(f"  {what}: dX={e1:.3e} dA={e2:.3e} dB={e3:.3e}", flush=True)
    assert e1 <= TOL and e2 <= TOL and e3 <= TOL, (what, e1, e2, e3)


# ------------------------------------------------------------------ configs

def test_single_linear_256_T16_r8():
    # single QLoRA linear: W 256x256, 16 tokens, r = 8, alpha = 16, fwd + bwd
    q = require_gpu()
    wl = synth.WORKLOADS[1]
    banner("linear 256x256 T=16 r=8")
    h = _make(1, 0, 16, 256, 256, wl.r)
    W, w_hat = _quantize(q, h["w"])
    _check_fwd(_fwd(q, W, h, wl.r, wl.alpha), w_hat, h, wl.r, wl.alpha, "cfg1")
    _check_bwd(_bwd(q, W, h, wl.r, wl.alpha), w_hat, h, wl.r, wl.alpha, "cfg1")


@pytest.mark.parametrize("T", [1, 16])
def test_decode_q_proj_4096(T):
    # decode-shaped q_proj 4096x4096, r = 16, alpha = 32, forward
    q = require_gpu()
    wl = synth.WORKLOADS[2]
    banner(f"q_proj 4096x4096 fwd T={T}")
    h = _make(2, 0, T, 4096, 4096, wl.r)
    W, w_hat = _quantize(q, h["w"])
    _check_fwd(_fwd(q, W, h, wl.r, wl.alpha), w_hat, h, wl.r, wl.alpha, f"q_proj T={T}")


@pytest.mark.parametrize("T,n_out,n_in,r,alpha", [
    (37, 320, 192, 12, 24.0),     # ragged T, r not a multiple of 8, several tiles
    (200, 128, 512, 64, 16.0),    # ragged tail of a 128-row tile, r = 64
    (129, 64, 64, 1, 1.0),        # smallest shapes, rank 1
    (5, 192, 256, 256, 8.0),      # largest rank
    (16, 512, 320, 16, 32.0),     # T at the small-token boundary
    (17, 512, 320, 16, 32.0),     # just above it
    (2, 256, 192, 24, 48.0),      # small-token path, two rank tiles
    (9, 128, 448, 40, 10.0),      # small-token path, four rank tiles, K not a multiple of 256
    (1, 64, 64, 64, 64.0),        # small-token path, largest rank it takes
])
def test_shapes_fwd_bwd(T, n_out, n_in, r, alpha):
    q = require_gpu()
    banner(f"shape T={T} out={n_out} in={n_in} r={r}")
    h = _make(7, T % 10, T, n_out, n_in, r)
    W, w_hat = _quantize(q, h["w"])
    _check_fwd(_fwd(q, W, h, r, alpha), w_hat, h, r, alpha, "fwd")
    _check_bwd(_bwd(q, W, h, r, alpha), w_hat, h, r, alpha, "bwd")


# ------------------------------------------------------------------ exact pins

@pytest.mark.parametrize("T", [3, 16, 40, 300])
def test_one_hot_rows_select_columns_bit_exact(T):
    # X rows one-hot (value 1) and B = 0: Y[t, :] = W_hat[:, i_t] exactly
    q = require_gpu()
    banner(f"one-hot fwd T={T}")
    n_out, n_in, r = 192, 320, 8
    h = _make(8, 1, T, n_out, n_in, r)
    W, w_hat = _quantize(q, h["w"])
    rng = np.random.default_rng(T)
    idx = rng.integers(0, n_in, T)
    X = np.zeros((T, n_in), dtype=np.uint16)
    X[np.arange(T), idx] = 0x3F80
    h["X"] = X
    h["B"] = np.zeros_like(h["B"])
    Y = host_bits(_fwd(q, W, h, r, 16.0))
    assert np.array_equal(Y, w_hat[:, idx].T)


@pytest.mark.parametrize("T", [4, 16, 70])
def test_one_hot_grad_rows_select_weight_rows_bit_exact(T):
    # dY rows one-hot and A = 0: dX[t, :] = W_hat[n_t, :] exactly; U = X A^T = 0
    # so dB = s dY^T U = 0
    q = require_gpu()
    banner(f"one-hot bwd T={T}")
    n_out, n_in, r = 192, 320, 8
    h = _make(8, 2, T, n_out, n_in, r)
    W, w_hat = _quantize(q, h["w"])
    rng = np.random.default_rng(100 + T)
    idx = rng.integers(0, n_out, T)
    dY = np.zeros((T, n_out), dtype=np.uint16)
    dY[np.arange(T), idx] = 0x3F80
    h["dY"] = dY
    h["A"] = np.zeros_like(h["A"])
    dX, dA, dB = _bwd(q, W, h, r, 16.0)
    assert np.array_equal(host_bits(dX), w_hat[idx, :])
    assert np.all(host(dB) == 0)


def test_zero_weight_isolates_lora():
    # W = 0 (all codes 7): Y = s U B^T and dX = s V A
    q = require_gpu()
    banner("zero weight")
    T, n_out, n_in, r, alpha = 48, 256, 192, 16, 32.0
    h = _make(9, 0, T, n_out, n_in, r)
    h["w"] = np.zeros_like(h["w"])
    W, w_hat = _quantize(q, h["w"])
    assert np.all(w_hat == 0)
    _check_fwd(_fwd(q, W, h, r, alpha), w_hat, h, r, alpha, "W=0 fwd")
    _check_bwd(_bwd(q, W, h, r, alpha), w_hat, h, r, alpha, "W=0 bwd")


def test_zero_tokens():
    q = require_gpu()
    banner("T = 0")
    n_out, n_in, r = 128, 128, 8
    h = _make(9, 1, 1, n_out, n_in, r)
    W, _ = _quantize(q, h["w"])
    X = torch.empty(0, n_in, dtype=torch.bfloat16, device="cuda")
    dY = torch.empty(0, n_out, dtype=torch.bfloat16, device="cuda")
    Y = q.qlora_linear_fwd(W, X, dev_bf16(h["A"]), dev_bf16(h["B"]), r, 16.0)
    assert Y.shape == (0, n_out)
    dA = torch.full((r, n_in), 7.0, device="cuda")
    dB = torch.full((n_out, r), 7.0, device="cuda")
    q.qlora_linear_bwd(W, X, dY, dev_bf16(h["A"]), dev_bf16(h["B"]), r, 16.0, dA=dA, dB=dB)
    torch.cuda.synchronize()
    assert torch.all(dA == 0) and torch.all(dB == 0)


def test_gradients_overwrite_not_accumulate():
    q = require_gpu()
    banner("overwrite semantics")
    T, n_out, n_in, r, alpha = 33, 128, 192, 8, 16.0
    h = _make(9, 2, T, n_out, n_in, r)
    W, w_hat = _quantize(q, h["w"])
    dA = torch.full((r, n_in), 123.0, device="cuda")
    dB = torch.full((n_out, r), -5.0, device="cuda")
    res = q.qlora_linear_bwd(W, dev_bf16(h["X"]), dev_bf16(h["dY"]), dev_bf16(h["A"]),
                             dev_bf16(h["B"]), r, alpha, dA=dA, dB=dB)
    _check_bwd(res, w_hat, h, r, alpha, "overwrite")


@pytest.mark.parametrize("r", [16, 24])
def test_small_token_forward_under_graph_replay(r):
    # A captured graph replays small-token forwards sharing one workspace
    # (r = 24: U = X A^T goes through it; r = 16: one launch, no workspace),
    # with eager calls on the same workspace in between; every replay must
    # equal the eager result bit for bit.
    q = require_gpu()
    banner(f"graph replay of the small-token forward r={r}")
    n_out, n_in, alpha = 512, 768, 2.0 * r
    hs = [_make(10, p, T, n_out, n_in, r) for p, T in ((0, 1), (1, 16), (2, 7))]
    W, w_hat = _quantize(q, hs[0]["w"])
    ins = [(dev_bf16(h["X"]), dev_bf16(h["A"]), dev_bf16(h["B"])) for h in hs]
    ws = q.make_workspace(max(q.qlora_workspace_bytes(T, n_in, n_out, r, False) for T in (1, 7, 16)),
                          "cuda")
    outs = [torch.empty(X.shape[0], n_out, dtype=torch.bfloat16, device="cuda") for X, _, _ in ins]
    eager = []
    for (X, A, B), Y in zip(ins, outs):
        eager.append(host_bits(q.qlora_linear_fwd(W, X, A, B, r, alpha, Y=Y, ws=ws)).copy())
    for h, ref_bits in zip(hs, eager):
        ref = odense.linear_fwd(w_hat, h["X"], h["A"], h["B"], alpha, r)
        assert odense.rel_frobenius(onf4.bf16_bits_to_f32(ref_bits), ref) <= TOL
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (X, A, B), Y in zip(ins, outs):
            q.qlora_linear_fwd(W, X, A, B, r, alpha, Y=Y, ws=ws)
    for rep in range(4):
        for Y in outs:
            Y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, Y in enumerate(outs):
            assert np.array_equal(host_bits(Y), eager[i]), (rep, i)
        # eager work on the same workspace between replays
        scratch = torch.empty_like(outs[1])
        X, A, B = ins[1]
        q.qlora_linear_fwd(W, X, A, B, r, alpha, Y=scratch, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(scratch), eager[1])


def test_workspace_needs_no_initialisation():
    # the workspace is plain scratch: a buffer full of 0xff bytes gives the
    # same results, bit for bit, as a zeroed one, for small- and large-token
    # forwards and backwards sharing one buffer
    q = require_gpu()
    banner("workspace contents do not matter")
    n_out, n_in, r, alpha = 384, 512, 16, 32.0
    hs = {T: _make(11, T % 7, T, n_out, n_in, r) for T in (3, 16, 40)}
    W, w_hat = _quantize(q, hs[3]["w"])
    need = max(q.qlora_workspace_bytes(T, n_in, n_out, r, b) for T in hs for b in (False, True))
    results = []
    for fill in (0x00, 0xFF):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        got = []
        for T, h in hs.items():
            Y = q.qlora_linear_fwd(W, dev_bf16(h["X"]), dev_bf16(h["A"]), dev_bf16(h["B"]), r, alpha, ws=ws)
            _check_fwd(Y, w_hat, h, r, alpha, f"T={T} fill={fill:#x}")
            res = q.qlora_linear_bwd(W, dev_bf16(h["X"]), dev_bf16(h["dY"]), dev_bf16(h["A"]),
                                     dev_bf16(h["B"]), r, alpha, ws=ws)
            _check_bwd(res, w_hat, h, r, alpha, f"T={T} fill={fill:#x}")
            got.append([host_bits(Y).copy(), host_bits(res[0]).copy(), host(res[1]).copy(),
                        host(res[2]).copy()])
        results.append(got)
    for a, b in zip(results[0], results[1]):
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_small_token_forward_needs_no_workspace():
    q = require_gpu()
    banner("small-token forward with ws = NULL")
    n_out, n_in, r, alpha = 256, 512, 16, 32.0
    h = _make(11, 9, 4, n_out, n_in, r)
    W, w_hat = _quantize(q, h["w"])
    X, A, B = dev_bf16(h["X"]), dev_bf16(h["A"]), dev_bf16(h["B"])  # alive across the call
    Y = torch.empty(4, n_out, dtype=torch.bfloat16, device="cuda")
    wc = W._c()
    st = q._lib.qlora_linear_fwd(ctypes.byref(wc), X.data_ptr(), 4, A.data_ptr(), B.data_ptr(), r,
                                 ctypes.c_float(alpha), Y.data_ptr(), None, 0,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    _check_fwd(Y, w_hat, h, r, alpha, "ws=NULL")
    # r > 16 computes U into the workspace first: NULL is refused, nothing runs
    r2 = 32
    h2 = _make(11, 8, 4, n_out, n_in, r2)
    A2, B2 = dev_bf16(h2["A"]), dev_bf16(h2["B"])
    st = q._lib.qlora_linear_fwd(ctypes.byref(wc), X.data_ptr(), 4, A2.data_ptr(), B2.data_ptr(), r2,
                                 ctypes.c_float(64.0), Y.data_ptr(), None, 0,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == -4  # QLORA_ERR_WORKSPACE


# ------------------------------------------------------------------ small-token path

@pytest.mark.parametrize("T,r", [(1, 1), (1, 16), (5, 17), (16, 32), (3, 33), (16, 64)])
def test_small_token_ranks(T, r):
    # every rank-tile variant of the small-token kernel and both ends of T
    q = require_gpu()
    banner(f"small-token T={T} r={r}")
    n_out, n_in, alpha = 1024, 1536, 2.0 * r
    h = _make(12, r % 10, T, n_out, n_in, r)
    W, w_hat = _quantize(q, h["w"])
    _check_fwd(_fwd(q, W, h, r, alpha), w_hat, h, r, alpha, f"T={T} r={r}")


@pytest.mark.parametrize("T", [1, 16])
def test_small_token_lora_only(T):
    # W = 0: Y = s U B^T, so the U each workgroup computes for itself (r <= 16)
    # is all of Y
    q = require_gpu()
    banner(f"small-token W=0 T={T}")
    n_out, n_in, r, alpha = 2048, 4096, 16, 32.0
    h = _make(13, T, T, n_out, n_in, r)
    h["w"] = np.zeros_like(h["w"])
    W, w_hat = _quantize(q, h["w"])
    _check_fwd(_fwd(q, W, h, r, alpha), w_hat, h, r, alpha, f"W=0 T={T}")


@pytest.mark.parametrize("T,n_out,n_in,r", [
    (3, 256, 4096, 16),    # two token-row pairs, four unrolled chunk steps, whole chunks
    (6, 256, 4096, 8),     # four token-row pairs
    (11, 128, 8192, 16),   # eight token-row pairs, eight unrolled steps
    (2, 192, 3136, 16),    # four unrolled steps, a partial last chunk in every wave
    (13, 64, 2048, 12),    # the step loop, whole chunks
    (7, 64, 1600, 5),      # the step loop, a partial last chunk
])
def test_small_token_split_variants(T, n_out, n_in, r):
    # the r <= 16 kernel's variants: token-row pairs, unrolled or looped chunk
    # steps, whole or partial chunks per wave
    q = require_gpu()
    banner(f"small-token split T={T} out={n_out} in={n_in} r={r}")
    alpha = 2.0 * r
    h = _make(14, T, T, n_out, n_in, r)
    W, w_hat = _quantize(q, h["w"])
    _check_fwd(_fwd(q, W, h, r, alpha), w_hat, h, r, alpha, f"T={T} in={n_in}")


@pytest.mark.parametrize("T", [1, 16])
def test_small_token_u_up_front_eight_steps(T):
    # r = 64 with 16 row blocks: U computed up front, then the split kernel
    # with eight unrolled chunk steps per wave (4096 < in <= 8192), the
    # variant the 70B gate takes at 16 tokens
    q = require_gpu()
    banner(f"small-token U up front, eight steps, T={T}")
    n_out, n_in, r, alpha = 256, 8192, 64, 128.0
    h = _make(15, T, T, n_out, n_in, r)
    W, w_hat = _quantize(q, h["w"])
    _check_fwd(_fwd(q, W, h, r, alpha), w_hat, h, r, alpha, f"pre-U ns=8 T={T}")


@pytest.mark.parametrize("T,r", [(1, 16), (16, 16), (1, 64), (16, 64)])
def test_small_token_more_workgroups_than_cus(T, r):
    # 8B MLP gate shape at decode size: 896 workgroups of 16 rows, more than
    # can be resident at once (U computed up front); also checks a repeat
    # call is bit-identical
    q = require_gpu()
    banner(f"small-token 14336x4096 T={T} r={r}")
    h = _make(3, 0, T, 14336, 4096, r)
    W, w_hat = _quantize(q, h["w"])
    Y1 = _fwd(q, W, h, r, 2.0 * r)
    _check_fwd(Y1, w_hat, h, r, 2.0 * r, f"gate T={T} r={r}")
    Y2 = _fwd(q, W, h, r, 2.0 * r)
    assert torch.equal(Y1, Y2)


@pytest.mark.parametrize("T", [1, 16])
def test_small_token_down_shape(T):
    # 8B MLP down shape (4096 x 14336, r = 64) at decode size: the chunk-step
    # loop with U computed up front
    q = require_gpu()
    banner(f"small-token 4096x14336 T={T} r=64")
    h = _make(3, 2, T, 4096, 14336, 64)
    W, w_hat = _quantize(q, h["w"])
    _check_fwd(_fwd(q, W, h, 64, 128.0), w_hat, h, 64, 128.0, f"down T={T}")
