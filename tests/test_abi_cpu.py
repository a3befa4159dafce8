"""Boundary tests that need no GPU: the C-ABI library loads, exports what
include/qlora.h declares, sizes its buffers as the format fixes, rejects bad
arguments on the host before touching HIP, and its compiled-in codebook and
code thresholds agree with the oracle's definitions."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import codebook as ocodebook
from oracle import native as onative
from oracle import storage as ostorage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")
# QLORA_ABI_LIB selects another build of the library (the sanitized one)
LIB = os.environ.get("QLORA_ABI_LIB") or os.path.join(ROOT, "bit_nf4_quantized_20_amd", "libqlora.so")


def _lib():
    if not os.path.exists(LIB):
        pytest.skip("libqlora.so not built")
    return ctypes.CDLL(LIB)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("nf4_quantize", "nf4_dequantize", "qlora_linear_fwd", "qlora_linear_bwd",
              "nf4_storage_bytes", "qlora_workspace_bytes", "nf4_codebook",
              "nf4_code_thresholds", "qlora_status_string"):
        assert n in names, names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_storage_bytes_match_format():
    lib = _lib()
    f = lib.nf4_storage_bytes
    f.argtypes = [ctypes.c_int64] + [ctypes.POINTER(ctypes.c_size_t)] * 3
    f.restype = ctypes.c_int
    for n in (0, 64, 64 * 255, 16384, 16384 * 3 + 64, 1 << 30):
        c, q, s = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        assert f(n, ctypes.byref(c), ctypes.byref(q), ctypes.byref(s)) == 0
        assert (c.value, q.value, s.value) == ostorage.buffer_bytes(n)
    assert f(65, None, None, None) == -2
    assert f(-64, None, None, None) == -2


def test_codebook_matches_oracle_bit_for_bit():
    lib = _lib()
    out = (ctypes.c_float * 16)()
    lib.nf4_codebook(out)
    got = np.frombuffer(out, dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ocodebook.nf4_levels().view(np.uint32))


def _thresholds():
    lib = _lib()
    out = (ctypes.c_float * 15)()
    lib.nf4_code_thresholds(out)
    return np.frombuffer(out, dtype=np.float32).copy()


@pytest.mark.slow
def test_threshold_rule_equals_argmin_on_every_fp32_in_unit_interval():
    # Exhaustive: every fp32 x in [-1, 1] (both signs, ~2.1e9 values).  The
    # library's rule code = #{j : x > t_j}, and the quantize kernel's bucket
    # lookup on X = 16 x, must both equal the oracle's first-argmin of
    # |fl32(x - L_j)|.
    thr = _thresholds()
    assert np.all(np.diff(thr) > 0)
    L = ocodebook.nf4_levels()
    one = int(np.float32(1.0).view(np.uint32))
    chunk = 1 << 26
    for sign in (0x00000000, 0x80000000):
        start = 0
        while start <= one:
            n = min(chunk, one + 1 - start)
            ref = onative.nearest_level_of_bits(sign | start, n, L)
            bits = (np.arange(start, start + n, dtype=np.uint64) | sign).astype(np.uint32)
            x = bits.view(np.float32)
            got = np.searchsorted(thr, x, side="left").astype(np.uint8)
            bad = np.nonzero(got != ref)[0]
            assert bad.size == 0, (hex(int(bits[bad[0]])), int(got[bad[0]]), int(ref[bad[0]]))
            got = _bucket_codes(x)
            bad = np.nonzero(got != ref)[0]
            assert bad.size == 0, ("bucket", hex(int(bits[bad[0]])), int(got[bad[0]]), int(ref[bad[0]]))
            start += n


def test_threshold_rule_near_every_boundary():
    # fast version of the exhaustive test: +-65536 ulps around every threshold
    thr = _thresholds()
    L = ocodebook.nf4_levels()
    for t in thr:
        b = int(np.float32(t).view(np.uint32))
        lo = b - 65536
        ref = onative.nearest_level_of_bits(lo, 131072, L)
        x = np.arange(lo, lo + 131072, dtype=np.uint64).astype(np.uint32).view(np.float32)
        got = np.searchsorted(thr, x, side="left")
        assert np.array_equal(got, ref)


def _buckets():
    lib = _lib()
    thr, base = (ctypes.c_float * 33)(), (ctypes.c_uint32 * 33)()
    lib.nf4_code_buckets(thr, base)
    return np.frombuffer(thr, dtype=np.float32).copy(), np.frombuffer(base, dtype=np.uint32).copy()


def _bucket_codes(x):
    # the kernel's lookup on X = 16 x (exact: a power-of-two scaling of |x| <= 1)
    thr, base = _buckets()
    X = x.astype(np.float32) * np.float32(16)
    k = np.floor(X).astype(np.int64) + 16
    return (base[k] + (X > thr[k])).astype(np.uint8)


def test_bucket_table_holds_each_threshold_once():
    thr, base = _buckets()
    t16 = _thresholds() * np.float32(16)
    inside = np.isfinite(thr)
    assert np.array_equal(np.sort(thr[inside]), t16)
    for i in range(33):
        lo = i - 16
        assert base[i] == np.count_nonzero(t16 < lo)
        if inside[i]:
            assert lo <= thr[i] < lo + 1


def test_bucket_rule_near_every_threshold_and_bucket_edge():
    # fast version: +-65536 ulps around every threshold and every bucket
    # edge k / 16
    L = ocodebook.nf4_levels()
    points = list(_thresholds()) + [np.float32(k / 16) for k in range(-16, 17)]
    starts = []
    for p in points:
        b = int(np.float32(p).view(np.uint32))
        starts += [0, 0x80000000] if p == 0 else [b - 65536]
    for lo in starts:
        ref = onative.nearest_level_of_bits(lo, 131072, L)
        x = np.arange(lo, lo + 131072, dtype=np.uint64).astype(np.uint32).view(np.float32)
        keep = np.abs(x) <= 1
        assert np.array_equal(_bucket_codes(x[keep]), ref[keep]), hex(lo)


# ---------------------------------------------------------------- host validation

_FAKE = 0x10000  # 16-byte aligned address that is never dereferenced
_MISALIGNED = 0x10008


class _W(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("absmax_q", ctypes.c_void_p),
                ("absmax_scale", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("flags", ctypes.c_uint32)]


def _api(lib):
    p, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.nf4_quantize.argtypes = [p, i64, p, p, p, p]
    lib.nf4_dequantize.argtypes = [p, p, p, i64, p, p]
    lib.qlora_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.qlora_workspace_bytes.restype = sz
    lib.qlora_linear_fwd.argtypes = [ctypes.POINTER(_W), p, i64, p, p, i64, ctypes.c_float, p, p, sz, p]
    lib.qlora_linear_bwd.argtypes = [ctypes.POINTER(_W), p, p, i64, p, p, i64, ctypes.c_float,
                                     p, p, p, p, sz, p]
    lib.qlora_status_string.restype = ctypes.c_char_p
    return lib


def test_quantize_dequantize_validation():
    lib = _api(_lib())
    F = _FAKE
    assert lib.nf4_quantize(F, 100, F, F, F, None) == -2          # numel % 64
    assert lib.nf4_quantize(F, -64, F, F, F, None) == -2
    assert lib.nf4_quantize(None, 64, F, F, F, None) == -1
    assert lib.nf4_quantize(F, 64, None, F, F, None) == -1
    assert lib.nf4_quantize(_MISALIGNED, 64, F, F, F, None) == -3
    assert lib.nf4_quantize(F, 0, None, None, None, None) == 0    # empty: no-op, no HIP call
    assert lib.nf4_dequantize(F, F, F, 63, F, None) == -2
    assert lib.nf4_dequantize(F, F, None, 64, F, None) == -1
    assert lib.nf4_dequantize(F, F, F, 64, _MISALIGNED, None) == -3
    assert lib.nf4_dequantize(F, F, F, 0, F, None) == 0


def test_linear_validation():
    lib = _api(_lib())
    F = _FAKE
    W = _W(F, F, F, 128, 256)
    # the large-token forward needs a workspace (LoRA factors, split-K
    # partials of the rank-r product); the small-token one none, but every
    # valid shape reports at least 256 bytes, T = 0 included
    assert lib.qlora_workspace_bytes(16, 256, 128, 8, 0) > 0
    assert lib.qlora_workspace_bytes(0, 256, 128, 8, 0) >= 256
    assert lib.qlora_workspace_bytes(0, 256, 128, 8, 1) >= 256
    assert lib.qlora_workspace_bytes(4096, 4096, 14336, 64, 1) > 4096 * 14336 * 2
    assert lib.qlora_workspace_bytes(16, 256, 128, 65, 0) > 0
    ws = lib.qlora_workspace_bytes(32, 256, 128, 8, 0)
    wsb = lib.qlora_workspace_bytes(16, 256, 128, 8, 1)
    assert ws > 0 and wsb > 0
    fwd = lambda **k: lib.qlora_linear_fwd(ctypes.byref(k.get("W", W)), k.get("X", F), k.get("T", 32),
                                           F, F, k.get("r", 8), k.get("alpha", 16.0), k.get("Y", F),
                                           k.get("ws", F), k.get("wsb", ws), None)
    assert fwd(W=_W(F, F, F, 128, 100)) == -2      # in % 64
    assert fwd(W=_W(F, F, F, 100, 256)) == -2      # out % 64
    assert fwd(r=0) == -2 and fwd(r=257) == -2
    assert fwd(T=-1) == -2
    assert fwd(X=None) == -1
    assert fwd(W=_W(None, F, F, 128, 256)) == -1
    assert fwd(Y=_MISALIGNED) == -3
    assert fwd(alpha=float("nan")) == -7 and fwd(alpha=float("inf")) == -7
    assert fwd(ws=None) == -4
    assert fwd(wsb=ws - 1) == -4
    assert fwd(T=0) == 0                           # no-op, no HIP call
    bwd = lambda **k: lib.qlora_linear_bwd(ctypes.byref(W), F, k.get("dY", F), k.get("T", 16), F, F, 8,
                                           16.0, F, k.get("dA", F), F, k.get("ws", F),
                                           k.get("wsb", wsb), None)
    assert bwd(dY=None) == -1
    assert bwd(dA=_MISALIGNED) == -3
    assert bwd(wsb=wsb - 1) == -4
    assert lib.qlora_workspace_bytes(16, 100, 128, 8, 0) == 0
    assert lib.qlora_workspace_bytes(-1, 256, 128, 8, 1) == 0
    for s in (0, -1, -2, -3, -4, -5, -6, -7, 42):
        assert len(lib.qlora_status_string(s)) > 0


def test_small_token_backward_workspace():
    # up to 16 tokens without dropout the backward keeps no W_hat^T: its
    # workspace holds the row-split fp32 partials of dX (sized for 512
    # workgroups over the in / 64 column strips), far below 2 out in bytes;
    # with dropout, or from 17 tokens on, the full size holds the expanded
    # W_hat^T (the faster dX route)
    lib = _api(_lib())
    i64, sz = ctypes.c_int64, ctypes.c_size_t
    lib.qlora_workspace_bytes_dropout.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.qlora_workspace_bytes_dropout.restype = sz
    for n_in, n_out, splits in ((4096, 14336, 8), (14336, 4096, 3), (4096, 4096, 8)):
        expanded = n_in * n_out * 2
        for T in (1, 7, 16):
            small = lib.qlora_workspace_bytes(T, n_in, n_out, 64, 1)
            assert splits * T * n_in * 4 <= small < expanded // 4, (n_in, n_out, T, small)
            assert lib.qlora_workspace_bytes_dropout(T, n_in, n_out, 64, 1) > expanded
        assert lib.qlora_workspace_bytes(17, n_in, n_out, 64, 1) > expanded
    # a weight with fewer 64-row chunks than splits: one split per chunk
    assert lib.qlora_workspace_bytes(16, 64, 128, 8, 1) >= 2 * 16 * 64 * 4


def test_backward_minimum_workspace():
    # qlora_workspace_bytes_bwd_min: the backward's layout without the expanded
    # W_hat^T (its dX GEMM then dequantizes the weight tiles while staging them):
    # no term in out * in from 17 tokens on or with dropout; the full size where
    # no such route exists (T <= 16 without dropout, the 4.5-bit format)
    lib = _api(_lib())
    i64, sz, F = ctypes.c_int64, ctypes.c_size_t, _FAKE
    lib.qlora_workspace_bytes_bwd_min.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.c_int, i64,
                                                  ctypes.c_int, ctypes.c_uint32]
    lib.qlora_workspace_bytes_bwd_min.restype = sz
    lib.qlora_workspace_bytes_flags.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.c_int, i64, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_uint32]
    lib.qlora_workspace_bytes_flags.restype = sz
    outs = lambda *o: (i64 * len(o))(*o)
    mn = lambda T, n_in, o, r=64, drop=0, flags=0: lib.qlora_workspace_bytes_bwd_min(
        T, n_in, outs(*o), len(o), r, drop, flags)
    full = lambda T, n_in, o, r=64, drop=0, flags=0: lib.qlora_workspace_bytes_flags(
        T, n_in, outs(*o), len(o), r, 1, drop, flags)
    for n_in, o in ((4096, [14336]), (14336, [4096]), (8192, [28672]), (4096, [4096, 1024, 1024])):
        weight = 2 * n_in * sum(o)
        for T in (17, 300, 4096):
            assert full(T, n_in, o) - mn(T, n_in, o) == weight, (n_in, o, T)
            assert mn(T, n_in, o) < (weight // 2 if len(o) == 1 else full(T, n_in, o))
            assert mn(T, n_in, o, flags=1) == full(T, n_in, o, flags=1)     # 4.5-bit: always expanded
        if len(o) == 1:
            assert full(64, n_in, o, drop=1) - mn(64, n_in, o, drop=1) == weight
        for T in (1, 16):
            assert mn(T, n_in, o) == full(T, n_in, o)                       # streamed, no W_hat^T
    # invalid arguments
    assert mn(17, 100, [128]) == 0 and mn(17, 256, [128], r=0) == 0
    assert mn(17, 256, [128], flags=2) == 0 and mn(17, 256, [128, 64], drop=1) == 0
    # the call accepts the minimum and refuses one byte less (before any HIP call)
    W = _W(F, F, F, 128, 256)
    least = mn(300, 256, [128], r=8)
    bwd = lambda wsb: lib.qlora_linear_bwd(ctypes.byref(W), F, F, 300, F, F, 8, 16.0, F, F, F, F, wsb, None)
    assert bwd(least - 1) == -4
    assert bwd(least) == -6       # valid: fails only at the device check
    assert bwd(full(300, 256, [128], r=8)) == -6


def test_forward_minimum_workspace():
    # qlora_workspace_bytes_fwd_min: the forward's layout without the expanded
    # W_hat (its GEMM then dequantizes the weight tiles while staging them);
    # from 512 tokens on exactly the expanded weight's bytes below the full
    # size, equal to it below 512 tokens and for the 4.5-bit format
    lib = _api(_lib())
    i64, sz, F = ctypes.c_int64, ctypes.c_size_t, _FAKE
    lib.qlora_workspace_bytes_fwd_min.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.c_int, i64,
                                                  ctypes.c_int, ctypes.c_uint32]
    lib.qlora_workspace_bytes_fwd_min.restype = sz
    lib.qlora_workspace_bytes_flags.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.c_int, i64, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_uint32]
    lib.qlora_workspace_bytes_flags.restype = sz
    outs = lambda *o: (i64 * len(o))(*o)
    mn = lambda T, n_in, o, r=16, drop=0, flags=0: lib.qlora_workspace_bytes_fwd_min(
        T, n_in, outs(*o), len(o), r, drop, flags)
    full = lambda T, n_in, o, r=16, drop=0, flags=0: lib.qlora_workspace_bytes_flags(
        T, n_in, outs(*o), len(o), r, 0, drop, flags)
    for n_in, o in ((4096, [14336]), (14336, [4096]), (4096, [4096, 1024, 1024])):
        weight = 2 * n_in * sum(o)
        for T in (512, 2048, 4096):
            assert full(T, n_in, o) - mn(T, n_in, o) == weight, (n_in, o, T)
            assert mn(T, n_in, o, flags=1) == full(T, n_in, o, flags=1)
        for T in (1, 16, 17, 300, 511):
            assert mn(T, n_in, o) == full(T, n_in, o)
        if len(o) == 1:
            assert full(1024, n_in, o, drop=1) - mn(1024, n_in, o, drop=1) == weight
    assert mn(17, 100, [128]) == 0 and mn(17, 256, [128], flags=2) == 0 and mn(17, 256, [128, 64], drop=1) == 0
    # the call accepts the minimum and refuses one byte less (before any HIP call)
    W = _W(F, F, F, 128, 256)
    least = mn(600, 256, [128], r=8)
    fwd = lambda wsb: lib.qlora_linear_fwd(ctypes.byref(W), F, 600, F, F, 8, 16.0, F, F, wsb, None)
    assert fwd(least - 1) == -4
    assert fwd(least) == -6 and fwd(full(600, 256, [128], r=8)) == -6   # valid: fail at the device check


def test_format_flags():
    # qlora_nf4_weight.flags: 0 = double-quantized, 1 = the 4.5-bit format
    # (fp32 block absmax in absmax_scale, absmax_q unused); other bits reserved
    lib = _api(_lib())
    i64, sz, F = ctypes.c_int64, ctypes.c_size_t, _FAKE
    lib.qlora_workspace_bytes_flags.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.c_int, i64, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_uint32]
    lib.qlora_workspace_bytes_flags.restype = sz
    lib.qlora_workspace_bytes_multi.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.c_int, i64, ctypes.c_int]
    lib.qlora_workspace_bytes_multi.restype = sz
    lib.qlora_workspace_bytes_dropout.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.qlora_workspace_bytes_dropout.restype = sz
    lib.qlora_merge.argtypes = [ctypes.POINTER(_W), ctypes.c_void_p, ctypes.c_void_p, i64, ctypes.c_float,
                                ctypes.c_void_p, ctypes.c_void_p, sz, ctypes.c_void_p]
    wsf = lambda T, outs, bwd=0, drop=0, flags=0, r=8: lib.qlora_workspace_bytes_flags(
        T, 256, (i64 * len(outs))(*outs), len(outs), r, bwd, drop, flags)
    # flags = 0 gives what the format-blind size functions give
    for T in (0, 1, 16, 32, 300, 2048, 4096):
        for b in (0, 1):
            assert wsf(T, [128], b) == lib.qlora_workspace_bytes(T, 256, 128, 8, b)
            assert wsf(T, [128], b, 1) == lib.qlora_workspace_bytes_dropout(T, 256, 128, 8, b)
            assert wsf(T, [128, 64], b) == lib.qlora_workspace_bytes_multi(T, 256, (i64 * 2)(128, 64), 2, 8, b)
    # the 4.5-bit forward expands W_hat into the workspace at every T
    for T in (1, 16, 300):
        assert wsf(T, [128], 0, 0, 1) >= wsf(T, [128]) + 128 * 256 * 2
        assert wsf(T, [128], 1, 0, 1) == wsf(T, [128], 1)        # the backward expands W_hat^T anyway
    assert wsf(16, [128, 64], 0, 0, 1) >= 192 * 256 * 2
    # reserved bits, and dropout with several projections
    assert wsf(16, [128], 0, 0, 2) == 0 and wsf(16, [128], 0, 0, 0x80000000) == 0
    assert wsf(16, [128, 64], 0, 1, 0) == 0
    ws1 = wsf(32, [128], 0, 0, 1)
    fwd = lambda W, wsb=ws1: lib.qlora_linear_fwd(ctypes.byref(W), F, 32, F, F, 8, 16.0, F, F, wsb, None)
    assert fwd(_W(F, F, F, 128, 256, 2)) == -7                  # reserved bit
    assert fwd(_W(None, None, None, 128, 256, 4)) == -7         # checked before the pointers
    assert fwd(_W(F, None, F, 128, 256, 0)) == -1               # double-quantized needs absmax_q
    assert fwd(_W(F, None, None, 128, 256, 1)) == -1            # 4.5-bit needs the absmax array
    # 4.5-bit: absmax_q NULL (or misaligned) is never read; the call gets as
    # far as the workspace check, which wants the expanded weight
    assert fwd(_W(F, None, F, 128, 256, 1), ws1 - 1) == -4
    assert fwd(_W(F, _MISALIGNED, F, 128, 256, 1), ws1 - 1) == -4
    # the merge reads the double-quantized format only
    assert lib.qlora_merge(ctypes.byref(_W(F, None, F, 128, 256, 1)), F, F, 8, 16.0, F, F, 1 << 20, None) == -7


def test_operand_size_limit():
    # every bf16 operand (X, Y / dY, dX, the dequantized weight) must stay
    # below 2^31 bytes: 2^31 - 2 bytes pass, 2^31 are refused, on every side
    lib = _api(_lib())
    i64, sz = ctypes.c_int64, ctypes.c_size_t
    lib.qlora_workspace_bytes_dropout.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.qlora_workspace_bytes_dropout.restype = sz
    lib.qlora_merge_workspace_bytes.argtypes = [i64, i64, i64]
    lib.qlora_merge_workspace_bytes.restype = sz
    limit = 1 << 30                                   # bf16 elements in 2^31 bytes
    assert lib.qlora_workspace_bytes(limit // 4096 - 1, 4096, 64, 16, 0) > 0
    assert lib.qlora_workspace_bytes(limit // 4096, 4096, 64, 16, 0) == 0     # X
    assert lib.qlora_workspace_bytes(limit // 8192, 64, 8192, 16, 1) == 0     # Y / dY
    assert lib.qlora_workspace_bytes(1, 1 << 15, 1 << 15, 16, 0) == 0         # weight
    assert lib.qlora_workspace_bytes(1, 1 << 15, (1 << 15) - 64, 16, 0) > 0
    assert lib.qlora_workspace_bytes_dropout(limit // 4096, 4096, 64, 16, 0) == 0
    assert lib.qlora_merge_workspace_bytes(1 << 15, 1 << 15, 16) == 0
    assert lib.qlora_merge_workspace_bytes(1 << 15, (1 << 15) - 64, 16) > 0
    F = _FAKE
    W = _W(F, F, F, 64, 4096)
    call = lambda T: lib.qlora_linear_fwd(ctypes.byref(W), F, T, F, F, 16, 32.0, F, F, 1 << 40, None)
    assert call(limit // 4096) == -2
    assert call(limit // 4096 - 1) == -6             # valid: fails only at the device check


def test_tensor_size_limit():
    # quantize / dequantize take at most 2^36 weights (one dequantize thread
    # per 32 weights stays below 2^32 threads)
    lib = _api(_lib())
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.nf4_quantize_nodq.argtypes = [vp, i64, vp, vp, vp]
    lib.nf4_dequantize_nodq.argtypes = [vp, vp, i64, vp, vp]
    F, big = _FAKE, (1 << 36) + 64
    assert lib.nf4_quantize(F, big, F, F, F, None) == -2
    assert lib.nf4_dequantize(F, F, F, big, F, None) == -2
    assert lib.nf4_quantize_nodq(F, big, F, F, None) == -2
    assert lib.nf4_dequantize_nodq(F, F, big, F, None) == -2
    assert lib.nf4_quantize(F, 1 << 36, F, F, F, None) == -6   # valid: only the device check fails


def test_multi_projection_validation():
    lib = _lib()
    i64, sz, vp = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    lib.qlora_workspace_bytes_multi.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.c_int, i64, ctypes.c_int]
    lib.qlora_workspace_bytes_multi.restype = sz
    lib.qlora_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.qlora_workspace_bytes.restype = sz
    lib.qlora_linear_fwd_multi.argtypes = [ctypes.POINTER(_W), ctypes.c_int, vp, i64, ctypes.POINTER(vp),
                                           ctypes.POINTER(vp), i64, ctypes.c_float, vp, vp, sz, vp]
    lib.qlora_linear_fwd_multi.restype = ctypes.c_int
    outs = (i64 * 3)(4096, 1024, 1024)
    one = (i64 * 1)(4096)
    # n = 1 is the single-projection size; more projections need more
    assert lib.qlora_workspace_bytes_multi(64, 4096, one, 1, 16, 1) == lib.qlora_workspace_bytes(64, 4096, 4096, 16, 1)
    assert lib.qlora_workspace_bytes_multi(64, 4096, outs, 3, 16, 1) > lib.qlora_workspace_bytes(64, 4096, 4096, 16, 1)
    assert lib.qlora_workspace_bytes_multi(64, 4096, outs, 0, 16, 0) == 0
    assert lib.qlora_workspace_bytes_multi(64, 4096, outs, 9, 16, 0) == 0
    assert lib.qlora_workspace_bytes_multi(64, 4096, None, 1, 16, 0) == 0
    F = _FAKE
    Ws = (_W * 2)(_W(F, F, F, 128, 256), _W(F, F, F, 64, 256))
    ptrs = (vp * 2)(F, F)
    nulls = (vp * 2)(F, None)
    ws = lib.qlora_workspace_bytes_multi(32, 256, (i64 * 2)(128, 64), 2, 8, 0)
    call = lambda **k: lib.qlora_linear_fwd_multi(k.get("W", Ws), k.get("n", 2), F, 32, k.get("A", ptrs),
                                                  ptrs, 8, 16.0, F, F, k.get("wsb", ws), None)
    assert call(n=0) == -2 and call(n=9) == -2
    assert call(W=(_W * 2)(_W(F, F, F, 128, 256), _W(F, F, F, 64, 320))) == -2  # in differs
    assert call(A=nulls) == -1
    assert call(wsb=ws - 1) == -4


def test_nodq_validation():
    lib = _lib()
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.nf4_quantize_nodq.argtypes = [vp, i64, vp, vp, vp]
    lib.nf4_dequantize_nodq.argtypes = [vp, vp, i64, vp, vp]
    F = _FAKE
    assert lib.nf4_quantize_nodq(F, 65, F, F, None) == -2
    assert lib.nf4_quantize_nodq(F, 64, F, None, None) == -1
    assert lib.nf4_quantize_nodq(F, 64, F, _MISALIGNED, None) == -3
    assert lib.nf4_quantize_nodq(F, 0, F, F, None) == 0
    assert lib.nf4_dequantize_nodq(F, F, -64, F, None) == -2
    assert lib.nf4_dequantize_nodq(F, None, 64, F, None) == -1
    assert lib.nf4_dequantize_nodq(F, F, 0, F, None) == 0


def test_merge_validation():
    lib = _lib()
    i64, sz, vp = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    lib.qlora_merge_workspace_bytes.argtypes = [i64, i64, i64]
    lib.qlora_merge_workspace_bytes.restype = sz
    lib.qlora_merge.argtypes = [ctypes.POINTER(_W), vp, vp, i64, ctypes.c_float, vp, vp, sz, vp]
    lib.qlora_merge.restype = ctypes.c_int
    F = _FAKE
    ws = lib.qlora_merge_workspace_bytes(256, 128, 8)
    # B padded [out][2 rp] + A^T padded [in][2 rp], bf16, rp = 64
    assert ws == 128 * 128 * 2 + 256 * 128 * 2
    assert lib.qlora_merge_workspace_bytes(100, 128, 8) == 0
    assert lib.qlora_merge_workspace_bytes(256, 128, 0) == 0
    W = _W(F, F, F, 128, 256)
    call = lambda **k: lib.qlora_merge(ctypes.byref(k.get("W", W)), k.get("A", F), F, k.get("r", 8),
                                       k.get("alpha", 16.0), k.get("out", F), k.get("ws", F),
                                       k.get("wsb", ws), None)
    assert call(W=_W(F, F, F, 128, 100)) == -2
    assert call(r=300) == -2
    assert call(A=None) == -1 and call(out=None) == -1
    assert call(out=_MISALIGNED) == -3
    assert call(alpha=float("nan")) == -7
    assert call(ws=None) == -4 and call(wsb=ws - 1) == -4


def test_dropout_validation():
    lib = _lib()
    i64, sz, vp, f32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    lib.qlora_workspace_bytes_dropout.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.qlora_workspace_bytes_dropout.restype = sz
    lib.qlora_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.qlora_workspace_bytes.restype = sz
    lib.qlora_linear_fwd_dropout.argtypes = [ctypes.POINTER(_W), vp, i64, vp, f32, vp, vp, i64, f32, vp,
                                             vp, sz, vp]
    lib.qlora_linear_fwd_dropout.restype = ctypes.c_int
    lib.qlora_linear_bwd_dropout.argtypes = [ctypes.POINTER(_W), vp, vp, i64, vp, f32, vp, vp, i64, f32,
                                             vp, vp, vp, vp, sz, vp]
    lib.qlora_linear_bwd_dropout.restype = ctypes.c_int
    # the dropout forward always takes the general path: at T <= 16 it needs
    # more workspace than the plain small-token forward, whose workspace only
    # holds U = X A^T (T * r fp32 values, 1 KiB here)
    assert lib.qlora_workspace_bytes(16, 4096, 4096, 16, 0) == 16 * 16 * 4
    assert lib.qlora_workspace_bytes_dropout(16, 4096, 4096, 16, 0) > 16 * 16 * 4
    assert lib.qlora_workspace_bytes_dropout(64, 4096, 4096, 16, 1) == lib.qlora_workspace_bytes(64, 4096, 4096, 16, 1)
    assert lib.qlora_workspace_bytes_dropout(16, 100, 4096, 16, 0) == 0
    F = _FAKE
    W = _W(F, F, F, 128, 256)
    ws = lib.qlora_workspace_bytes_dropout(32, 256, 128, 8, 0)
    fwd = lambda **k: lib.qlora_linear_fwd_dropout(ctypes.byref(W), F, k.get("T", 32), k.get("keep", F),
                                                   k.get("p", 0.05), F, F, 8, 16.0, F, F,
                                                   k.get("wsb", ws), None)
    assert fwd(keep=None) == -1
    assert fwd(p=1.0) == -7 and fwd(p=-0.1) == -7 and fwd(p=float("nan")) == -7
    assert fwd(wsb=ws - 1) == -4
    assert fwd(T=0, keep=None) == 0
    wsb = lib.qlora_workspace_bytes_dropout(32, 256, 128, 8, 1)
    bwd = lambda **k: lib.qlora_linear_bwd_dropout(ctypes.byref(W), F, F, 32, k.get("keep", F),
                                                   k.get("p", 0.05), F, F, 8, 16.0, F, F, F, F,
                                                   k.get("wsb", wsb), None)
    assert bwd(keep=None) == -1
    assert bwd(p=1.5) == -7
    # the backward also runs in the smaller workspace without W_hat^T
    i64, sz = ctypes.c_int64, ctypes.c_size_t
    lib.qlora_workspace_bytes_bwd_min.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.c_int, i64,
                                                  ctypes.c_int, ctypes.c_uint32]
    lib.qlora_workspace_bytes_bwd_min.restype = sz
    least = lib.qlora_workspace_bytes_bwd_min(32, 256, (i64 * 1)(128), 1, 8, 1, 0)
    assert least == wsb - 256 * 128 * 2
    assert bwd(wsb=least - 1) == -4
    assert bwd(wsb=least) == -6 and bwd(wsb=wsb - 1) == -6   # valid: fail only at the device check


def test_valid_call_without_gpu_reports_device_error():
    # with no HIP device the first HIP call fails and the call returns
    # ERR_DEVICE without launching anything (pointers are never touched)
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this checks the no-device path")
    lib = _api(_lib())
    F = _FAKE
    assert lib.nf4_quantize(F, 64, F, F, F, None) == -6
