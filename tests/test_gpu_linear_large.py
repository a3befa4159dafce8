"""GPU parity of the large-token QLoRA linear at the full workload sizes.

Forward and backward of every projection of the 8B MLP (gate, up
4096->14336, down 14336->4096, T = 4096, r = 64), the 8B attention
projections (q, o 4096x4096, k, v 4096->1024, T = 8192, r = 16) and the 70B
MLP (gate, up 8192->28672, down 28672->8192, T = 4096, r = 64, alpha = 16),
each through the same calls and launch
configuration the benchmark times, plus a ragged token count on the
256 x 256-tile GEMM.

The oracle quantizes the same fp32 weight itself and evaluates the full Y,
dX, dA and dB in fp64 (every output element of every call).  Acceptance:
relative Frobenius error <= 2e-3 for each of Y, dX, dA and dB.

Also here: bit-exact one-hot pins through the paths that only run at large
token counts (the forward's weight expansion from 512 tokens on, the fused
NF4 GEMM given the smallest forward workspace, and the large-tile GEMMs of
both directions)."""

import numpy as np
import pytest

import synth
from oracle import dense as odense
from oracle import native as onative
from oracle import nf4 as onf4

from gpu_util import TOL, banner, dev_bf16, dev_f32, host, host_bits, require_gpu

pytestmark = pytest.mark.gpu


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


def _check(wid, proj, T=None, fwd_min_ws=False):
    q = require_gpu()
    w, X, dY, A, B, r, alpha = _case(wid, proj, T)
    T = X.shape[0]
    n_out, n_in = w.shape
    banner(f"large linear workload {wid} projection {proj}: T={T} out={n_out} in={n_in} r={r}")

    W = q.nf4_quantize_weight(dev_f32(w))
    Xd, dYd, Ad, Bd = dev_bf16(X), dev_bf16(dY), dev_bf16(A), dev_bf16(B)
    wsf = q.make_workspace(q.qlora_workspace_bytes_fwd_min(T, n_in, [n_out], r), "cuda") if fwd_min_ws else None
    Y = q.qlora_linear_fwd(W, Xd, Ad, Bd, r, alpha, ws=wsf)
    dX, dA, dB = q.qlora_linear_bwd(W, Xd, dYd, Ad, Bd, r, alpha)
    Yh = onf4.bf16_bits_to_f32(host_bits(Y)).astype(np.float64)
    dXh = onf4.bf16_bits_to_f32(host_bits(dX)).astype(np.float64)
    dAh, dBh = host(dA).astype(np.float64), host(dB).astype(np.float64)
    del Y, dX, dA, dB, W, Xd, dYd

    # oracle: its own quantization of the same weight, then fp64 over every
    # output element
    packed, aq, sc = onf4.quantize(w.reshape(-1), nearest=onative.nearest_level)
    del w
    w_hat = odense.widen(onf4.dequantize(packed, aq, sc).reshape(n_out, n_in))
    del packed, aq, sc
    s = float(alpha) / float(r)
    Xw, Gw, Aw, Bw = odense.widen(X), odense.widen(dY), odense.widen(A), odense.widen(B)
    U = Xw @ Aw.T                              # [T, r]
    V = Gw @ Bw                                # [T, r]
    errs = {
        "Y": odense.rel_frobenius(Yh, Xw @ w_hat.T + s * (U @ Bw.T)),
        "dX": odense.rel_frobenius(dXh, Gw @ w_hat + s * (V @ Aw)),
        "dA": odense.rel_frobenius(dAh, s * (V.T @ Xw)),
        "dB": odense.rel_frobenius(dBh, s * (Gw.T @ U)),
    }
    print("  rel_frobenius " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()) + " (full tensors)",
          flush=True)
    assert all(v <= TOL for v in errs.values()), errs


@pytest.mark.parametrize("wid,proj", [
    (3, 0),   # 8B MLP gate 4096 -> 14336 (896 tiles of 256 x 256)
    (3, 1),   # 8B MLP up 4096 -> 14336
    (3, 2),   # 8B MLP down 14336 -> 4096 (dX over 14336 input features)
    (4, 0),   # 8B attention q 4096 x 4096, T = 8192
    (4, 1),   # 8B attention k 4096 -> 1024 (128 x 128 tiles)
    (4, 2),   # 8B attention v 4096 -> 1024
    (4, 3),   # 8B attention o 4096 x 4096
    (5, 0),   # 70B MLP gate 8192 -> 28672, alpha / r = 0.25
    (5, 1),   # 70B MLP up 8192 -> 28672
    (5, 2),   # 70B MLP down 28672 -> 8192
])
def test_workload_projection_fwd_bwd(wid, proj):
    _check(wid, proj)


def test_ragged_tokens_on_large_tiles():
    # q-shaped 4096 x 4096 with T = 4136: 17 x 16 tiles of 256, the last row of
    # tiles 40 tokens tall (rows past T read as zero and are not stored)
    _check(4, 0, T=4136)


def test_fused_dequant_gemm_in_the_smallest_workspace():
    # 8B MLP gate at T = 1536 (6 x 56 tiles of 256) with the smallest forward
    # workspace: the forward takes the fused NF4 GEMM (codes dequantized while
    # staged into LDS) instead of expanding the weight
    _check(3, 0, T=1536, fwd_min_ws=True)


# ------------------------------------------------------------ one-hot pins

def _one_hot(n, idx):
    m = np.zeros((len(idx), n), dtype=np.uint16)
    m[np.arange(len(idx)), idx] = 0x3F80  # bf16 1.0
    return m


@pytest.mark.parametrize("T,n_out,n_in", [
    (2048, 512, 320),    # weight expanded once into the workspace, 128 x 128 tiles
    (2048, 8192, 512),   # the same on 256 x 256 tiles (8 x 32 = 256 tiles)
    (1792, 8192, 512),   # 7 x 32 tiles of 256; with the smallest workspace the fused NF4 GEMM on 14 x 32 of 128 x 256
    (2048, 512, 8192),   # the expanded-weight dX GEMM on 256 x 256 tiles (8 x 32)
    (1024, 512, 8192),   # the same on 128 x 256 tiles (8 x 32)
])
def test_one_hot_large_token_paths_bit_exact(T, n_out, n_in):
    # X rows one-hot and B = 0: Y[t, :] = W_hat[:, i_t] exactly (one non-zero
    # product per output, exact in fp32 and in bf16).  dY rows one-hot and
    # A = 0: dX[t, :] = W_hat[n_t, :] exactly, through the backward's dX GEMM.
    q = require_gpu()
    banner(f"one-hot large-token T={T} out={n_out} in={n_in}")
    r, alpha = 16, 32.0
    w = synth.normal_f32(77_000 + n_out, (n_out, n_in), synth.W_STD)
    rng = np.random.default_rng(T + n_out)
    xi = rng.integers(0, n_in, T)
    gi = rng.integers(0, n_out, T)
    X = _one_hot(n_in, xi)
    dY = _one_hot(n_out, gi)
    A = synth.bf16_bits(synth.normal_f32(5, (r, n_in), 1.0 / n_in))
    B = synth.bf16_bits(synth.normal_f32(6, (n_out, r), synth.B_STD))
    W = q.nf4_quantize_weight(dev_f32(w))
    Y = q.qlora_linear_fwd(W, dev_bf16(X), dev_bf16(A), dev_bf16(np.zeros_like(B)), r, alpha)
    dX, dA, dB = q.qlora_linear_bwd(W, dev_bf16(X), dev_bf16(dY), dev_bf16(np.zeros_like(A)),
                                    dev_bf16(B), r, alpha)
    packed, aq, sc = onf4.quantize(w, nearest=onative.nearest_level)
    w_hat = onf4.dequantize(packed, aq, sc).reshape(n_out, n_in)
    assert np.array_equal(host_bits(Y), w_hat[:, xi].T)
    assert np.array_equal(host_bits(dX), w_hat[gi, :])
    assert np.all(host(dB) == 0)  # U = X A^T = 0
    # the forward in its smallest workspace (the fused NF4 GEMM from 512 tokens on)
    wsm = q.make_workspace(q.qlora_workspace_bytes_fwd_min(T, n_in, [n_out], r), "cuda")
    Ym = q.qlora_linear_fwd(W, dev_bf16(X), dev_bf16(A), dev_bf16(np.zeros_like(B)), r, alpha, ws=wsm)
    assert np.array_equal(host_bits(Ym), w_hat[:, xi].T)
