"""GPU parity of nf4_quantize / nf4_dequantize against the oracle: codes,
8-bit absmax codes, group scales and the dequantized bf16 weight must match
bit for bit."""

import os

import numpy as np
import pytest
import torch

import synth
from oracle import native as onative
from oracle import nf4 as onf4
from oracle.codebook import nf4_levels

from gpu_util import banner, dev_f32, host, host_bits, require_gpu

pytestmark = pytest.mark.gpu


def _quant_both(q, w_host: np.ndarray):
    w = dev_f32(w_host)
    codes, aq, sc = q.nf4_quantize(w)
    torch.cuda.synchronize()
    ref = onf4.quantize(w_host, nearest=onative.nearest_level)
    return (host(codes), host(aq), host(sc)), ref, (codes, aq, sc)


def _assert_bits_equal(got, ref, what):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.dtype == np.float32:
        got, ref = got.view(np.uint32), ref.view(np.uint32)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: {got[bad[:5]]} vs {ref[bad[:5]]}"


@pytest.mark.parametrize("shape", [(256, 256), (4096, 4096), (64,), (64 * (256 * 3 + 37),)])
def test_quantize_dequantize_bit_exact(shape):
    q = require_gpu()
    banner(f"quantize/dequantize shape={shape}")
    w_host = synth.normal_f32(11, shape, synth.W_STD)
    (codes, aq, sc), (rc, raq, rsc), dev = _quant_both(q, w_host)
    _assert_bits_equal(codes, rc, "codes")
    _assert_bits_equal(aq, raq, "absmax_q")
    _assert_bits_equal(sc, rsc, "scale")
    n = int(np.prod(shape))
    back = q.nf4_dequantize(*dev, n)
    torch.cuda.synchronize()
    _assert_bits_equal(host_bits(back), onf4.dequantize(rc, raq, rsc), "dequant")


def test_dequantize_every_absmax_code():
    # 3 groups of 256 blocks whose absmax codes run through 0..255 and whose
    # 64 codes cycle through the 16 levels, with an ordinary, a tiny and a
    # huge group scale: the dequantized bf16 must match bit for bit
    q = require_gpu()
    banner("dequantize all 256 absmax codes x 16 levels")
    nblk = 3 * 256
    n = nblk * 64
    levels = (np.arange(n) % 16).astype(np.uint8)
    packed = (levels[0::2] | (levels[1::2] << 4)).astype(np.uint8)
    aq = (np.arange(nblk) % 256).astype(np.uint8)
    sc = np.array([0.0371, 1.0e-38, 3.0e38], dtype=np.float32)
    back = q.nf4_dequantize(torch.from_numpy(packed).cuda(), torch.from_numpy(aq).cuda(),
                            torch.from_numpy(sc).cuda(), n)
    torch.cuda.synchronize()
    _assert_bits_equal(host_bits(back), onf4.dequantize(packed, aq, sc), "dequant")


def test_edge_blocks():
    # zero blocks, a zero group, tiny (subnormal) blocks, huge and exact-level values
    q = require_gpu()
    banner("quantize edge blocks")
    w = synth.normal_f32(12, (64 * 256 * 4,), synth.W_STD)
    w[0:64] = 0.0                                        # zero block
    w[64 * 256:64 * 512] = 0.0                           # zero group
    w[64 * 5:64 * 6] *= np.float32(1e-37)                # subnormal-range values
    w[64 * 7:64 * 8] = np.float32(3e37) * np.sign(w[64 * 7:64 * 8])  # huge, equal magnitude
    w[64 * 9:64 * 9 + 16] = nf4_levels() * np.float32(0.37)  # exact levels * a
    w[64 * 9 + 16] = np.float32(0.37)
    w[64 * 600 + 3] = -np.float32(5.0)                   # one large outlier in group 2
    (codes, aq, sc), (rc, raq, rsc), dev = _quant_both(q, w)
    _assert_bits_equal(codes, rc, "codes")
    _assert_bits_equal(aq, raq, "absmax_q")
    _assert_bits_equal(sc, rsc, "scale")
    back = q.nf4_dequantize(*dev, w.size)
    torch.cuda.synchronize()
    _assert_bits_equal(host_bits(back), onf4.dequantize(rc, raq, rsc), "dequant")


def _near_threshold_blocks(seed, absmax):
    """One 64-weight block per absmax value: w[0] = a (the block maximum), the
    rest within 3 ulps of fl32(m * a), m the exact midpoint between a code
    threshold and the next fp32 -- the quotients where fl32(w / a) decides
    the code -- with random signs of the offsets."""
    rng = np.random.default_rng(seed)
    import bit_nf4_quantized_20_amd as q
    thr = np.array(q.nf4_code_thresholds(), dtype=np.float32)
    mids = (thr.astype(np.float64) + np.nextafter(thr, np.float32(np.inf)).astype(np.float64)) / 2
    out = np.zeros((len(absmax), 64), dtype=np.float32)
    for b, a in enumerate(absmax):
        a = np.float32(a)
        j = rng.integers(0, 15, 63)
        w = (mids[j] * np.float64(a)).astype(np.float32)  # m a exact in fp64, one rounding
        w = (w.view(np.int32) + rng.integers(-3, 4, 63).astype(np.int32)).view(np.float32)
        w = np.where(np.abs(w) <= a, w, np.float32(0))
        out[b, 0] = a
        out[b, 1:] = w
    return out.reshape(-1)


def test_quantize_near_thresholds_bit_exact():
    # quotients at the code decision points, absmax across the range the
    # kernel takes with its reciprocal (2^-90 .. 2^120, both ends) and beyond
    # it (direct division): 3 full groups plus a ragged one, the out-of-range
    # blocks in the second group only, so the first group runs the
    # whole-wave reciprocal path
    q = require_gpu()
    banner("quantize near thresholds")
    rng = np.random.default_rng(21)
    nblk = 3 * 256 + 37
    e = rng.integers(-89, 120, nblk).astype(np.float64)
    absmax = (2.0 ** e * rng.uniform(1, 2, nblk)).astype(np.float32)
    absmax[0], absmax[1] = np.float32(2.0 ** -90), np.float32(2.0 ** 120)
    edge = [2.0 ** -91, 2.0 ** -126, 1e-40, 2.0 ** 121, 3e38, 0.0, 0.037, 1.0]
    absmax[256:256 + len(edge)] = np.array(edge, dtype=np.float32)
    w = _near_threshold_blocks(22, absmax)  # absmax 0.0: a zero block
    (codes, aq, sc), (rc, raq, rsc), dev = _quant_both(q, w)
    _assert_bits_equal(codes, rc, "codes")
    _assert_bits_equal(aq, raq, "absmax_q")
    _assert_bits_equal(sc, rsc, "scale")
    codes2, absmax2 = q.nf4_quantize_nodq(dev_f32(w))
    torch.cuda.synchronize()
    rc2, ra2 = onf4.quantize_nodq(w, nearest=onative.nearest_level)
    _assert_bits_equal(host(codes2), rc2, "nodq codes")
    _assert_bits_equal(host(absmax2), ra2, "nodq absmax")


def test_tiny_absmax_block_gives_signed_zero():
    # a block whose 8-bit absmax code rounds to 0 dequantizes to +-0 (sign of
    # the level), bit-exactly as IEEE multiplication gives it
    q = require_gpu()
    banner("tiny absmax block")
    w = synth.normal_f32(13, (64 * 256,), synth.W_STD)
    w[0:64] *= np.float32(1e-4)
    (codes, aq, sc), (rc, raq, rsc), dev = _quant_both(q, w)
    assert raq[0] == 0
    _assert_bits_equal(codes, rc, "codes")
    back = host_bits(q.nf4_dequantize(*dev, w.size))
    ref = onf4.dequantize(rc, raq, rsc)
    assert np.any(ref[:64] == 0x8000)
    _assert_bits_equal(back, ref, "dequant")


def test_empty_is_noop():
    q = require_gpu()
    w = torch.empty(0, dtype=torch.float32, device="cuda")
    c, a, s = q.nf4_quantize(w)
    assert c.numel() == 0 and a.numel() == 0 and s.numel() == 0


@pytest.mark.parametrize("proj", [0, 2])
def test_mlp_weight_full_buffers(proj):
    # 8B-MLP-shaped weights (gate 14336x4096 / down 4096x14336), full buffers
    q = require_gpu()
    p = synth.WORKLOADS[3].projections[proj]
    banner(f"quantize {p.name} {p.out_features}x{p.in_features}")
    w_host = synth.weight(3, proj, p.out_features, p.in_features)
    (codes, aq, sc), (rc, raq, rsc), dev = _quant_both(q, w_host)
    _assert_bits_equal(codes, rc, "codes")
    _assert_bits_equal(aq, raq, "absmax_q")
    _assert_bits_equal(sc, rsc, "scale")
    back = host_bits(q.nf4_dequantize(*dev, w_host.size))
    _assert_bits_equal(back, onf4.dequantize(rc, raq, rsc), "dequant")


@pytest.mark.timeout(900)
def test_flat_2pow30_full_buffers():
    # the 2^30-element flat quantize workload, every output buffer compared
    # bit for bit: codes, absmax codes, group scales and the dequantized bf16
    # weights.  The oracle runs on independent slices of whole double-quant
    # groups (each group's codes and scale depend on that group alone), a few
    # slices at a time on host threads.
    q = require_gpu()
    n = synth.FLAT_QUANTIZE_NUMEL
    banner(f"quantize flat n={n}")
    w_host = synth.normal_f32(synth.FLAT_QUANTIZE_SEED, (n,), synth.W_STD)
    w = dev_f32(w_host)
    codes, aq, sc = q.nf4_quantize(w)
    torch.cuda.synchronize()
    del w
    codes_h, aq_h, sc_h = host(codes), host(aq), host(sc)
    back = q.nf4_dequantize(codes, aq, sc, n)
    torch.cuda.synchronize()
    del codes, aq, sc
    back_h = host_bits(back)
    del back
    torch.cuda.empty_cache()

    G = 16384
    chunk = 1024 * G  # 1024 groups per slice

    def check(start):
        stop = min(start + chunk, n)
        rc, raq, rsc = onf4.quantize(w_host[start:stop], nearest=onative.nearest_level)
        g0, g1 = start // G, (stop + G - 1) // G
        bad = []
        if not np.array_equal(codes_h[start // 2:stop // 2], rc):
            bad.append("codes")
        if not np.array_equal(aq_h[start // 64:stop // 64], raq):
            bad.append("absmax_q")
        if not np.array_equal(sc_h[g0:g1].view(np.uint32), rsc.view(np.uint32)):
            bad.append("scale")
        if not np.array_equal(back_h[start:stop], onf4.dequantize(rc, raq, rsc)):
            bad.append("dequant")
        return start, bad

    from concurrent.futures import ThreadPoolExecutor
    workers = max(1, min(8, len(os.sched_getaffinity(0)) // 2))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(check, range(0, n, chunk)))
    failed = [(s0, b) for s0, b in results if b]
    assert not failed, failed[:4]
    assert len(results) == n // chunk


# ------------------------------------------ format without double quantization

@pytest.mark.parametrize("shape", [(256, 256), (4096, 4096), (64 * (256 * 3 + 37),)])
def test_nodq_quantize_dequantize_bit_exact(shape):
    q = require_gpu()
    banner(f"no-double-quant quantize/dequantize shape={shape}")
    w_host = synth.normal_f32(13, shape, synth.W_STD)
    w_host.reshape(-1)[0:64] = 0.0  # a zero block
    codes, absmax = q.nf4_quantize_nodq(dev_f32(w_host))
    torch.cuda.synchronize()
    rc, ra = onf4.quantize_nodq(w_host, nearest=onative.nearest_level)
    _assert_bits_equal(host(codes), rc, "codes")
    _assert_bits_equal(host(absmax), ra, "absmax")
    n = int(np.prod(shape))
    back = q.nf4_dequantize_nodq(codes, absmax, n)
    torch.cuda.synchronize()
    _assert_bits_equal(host_bits(back), onf4.dequantize_nodq(rc, ra), "dequant")


def test_nodq_gpu_codes_replay_the_mse_experiment():
    # ultralytics glossary "QLoRA": seed 0, randn(4096, 64) * 0.02, exact block
    # absmax, nearest NF4 level: the printed MSE is 3.395e-06.  The GPU's
    # codes and absmax, reconstructed in fp32 as on the page, give it again.
    q = require_gpu()
    banner("MSE experiment from GPU codes")
    torch.manual_seed(0)
    w = (torch.randn(4096, 64) * 0.02).numpy()
    codes, absmax = q.nf4_quantize_nodq(dev_f32(w))
    torch.cuda.synchronize()
    restored = onf4.dequantize_nodq_f32(host(codes), host(absmax)).reshape(w.shape)
    mse = np.mean((restored.astype(np.float64) - w.astype(np.float64)) ** 2)
    assert f"{mse:.3e}" == "3.395e-06", mse
