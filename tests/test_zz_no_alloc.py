"""GPU test of qlora_linear_fwd_noalloc, the forward for callers that cannot
allocate: it runs on the library's static scratch and must give the same bits
as qlora_linear_fwd with a caller workspace, call after call on the shared
scratch, and refuse a call whose smallest workspace exceeds the scratch.

Each sequence makes two calls in a row on one weight, the second with fewer
tokens, through the paths that use the scratch: the LDS-staged fused GEMM
(T = 300, U and the padded B in the scratch) then the weight stream (T = 16,
U computed up front); the dequantize-then-GEMM path (T = 2048, the weight
dequantized into the scratch) then the single-token forward at r = 64; and
T = 2048 on a 4096 x 4096 weight, whose expanded weight (32 MiB) does not fit:
the scratch call takes the fused GEMM where the workspace call expands, and Y
is still the same bit for bit."""

import numpy as np
import pytest
import torch

import synth

from gpu_util import banner, dev_bf16, dev_f32, host_bits, require_gpu

pytestmark = pytest.mark.gpu


def _factors(seed, n_in, n_out, r):
    A = synth.bf16_bits(synth.normal_f32(seed + 2, (r, n_in), 1.0 / n_in))
    B = synth.bf16_bits(synth.normal_f32(seed + 3, (n_out, r), synth.B_STD))
    return dev_bf16(A), dev_bf16(B)


@pytest.mark.parametrize("n_in,n_out,r,tokens", [
    (4096, 8192, 16, (300, 16)),   # fused GEMM, then the weight stream
    (1024, 1024, 64, (2048, 1)),   # dequantize + GEMM, then one token
    (4096, 4096, 16, (2048, 16)),  # fused GEMM in the scratch (the workspace call expands), then T = 16
])
def test_noalloc_matches_workspace_forward(n_in, n_out, r, tokens):
    q = require_gpu()
    seed = 5000 + n_out + r
    W = q.nf4_quantize_weight(dev_f32(synth.normal_f32(seed, (n_out, n_in), synth.W_STD)))
    A, B = _factors(seed, n_in, n_out, r)
    alpha = 2.0 * r
    for i, T in enumerate(tokens):
        banner(f"noalloc call {i}: T={T} in={n_in} out={n_out} r={r}")
        assert q.qlora_workspace_bytes_fwd_min(T, n_in, [n_out], r) <= q.qlora_noalloc_scratch_bytes()
        X = dev_bf16(synth.bf16_bits(synth.normal_f32(seed + 10 + T, (T, n_in), 1.0)))
        ws = q.make_workspace(q.qlora_workspace_bytes(T, n_in, n_out, r, False), "cuda")
        want = host_bits(q.qlora_linear_fwd(W, X, A, B, r, alpha, ws=ws))
        Y = torch.full((T, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
        got = host_bits(q.qlora_linear_fwd_noalloc(W, X, A, B, r, alpha, Y))
        assert np.array_equal(got, want), (i, T)


def test_noalloc_refuses_oversized_workspace():
    # T = 16384 tokens at rank 256: the rank-r product alone (T x 256 fp32 in
    # its padded bf16 hi / lo form) takes 16 MiB, so even the smallest
    # workspace exceeds the scratch; refused before any launch, Y untouched
    q = require_gpu()
    banner("noalloc oversized")
    T, n_in, n_out, r = 16384, 64, 64, 256
    assert q.qlora_workspace_bytes_fwd_min(T, n_in, [n_out], r) > q.qlora_noalloc_scratch_bytes()
    W = q.nf4_quantize_weight(dev_f32(synth.normal_f32(5200, (n_out, n_in), synth.W_STD)))
    A, B = _factors(5200, n_in, n_out, r)
    X = torch.zeros(T, n_in, dtype=torch.bfloat16, device="cuda")
    Y = torch.full((T, n_out), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(q.QloraError) as err:
        q.qlora_linear_fwd_noalloc(W, X, A, B, r, 2.0 * r, Y)
    assert q.STATUS[err.value.status] == "ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())
