"""Python binding of libqlora.so, the gfx950 NF4 / QLoRA-linear library.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch supplies device memory (``torch.empty``), raw pointers
(``data_ptr``) and the current stream; it computes nothing here.  If the
library has not been built, importing this package raises.

Names and semantics follow include/qlora.h:
    nf4_storage_bytes, nf4_quantize, nf4_dequantize, qlora_workspace_bytes,
    nf4_quantize_nodq, nf4_dequantize_nodq,
    qlora_linear_fwd, qlora_linear_bwd, qlora_workspace_bytes_multi, qlora_linear_fwd_multi,
    qlora_linear_bwd_multi, qlora_merge_workspace_bytes, qlora_merge,
    qlora_noalloc_scratch_bytes, qlora_linear_fwd_noalloc, qlora_workspace_bytes_flags,
    nf4_quantize_weight_nodq, nf4_code_buckets,
    nf4_codebook, nf4_code_thresholds, qlora_status_string
"""

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora.so")

QLORA_OK = 0
STATUS = {0: "OK", -1: "ERR_NULL", -2: "ERR_SHAPE", -3: "ERR_ALIGN", -4: "ERR_WORKSPACE",
          -5: "ERR_LAUNCH", -6: "ERR_DEVICE", -7: "ERR_VALUE"}


class QloraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_status_string(status)})")


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python bit_nf4_quantized_20_amd/build.py` "
                      "(hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)
_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class _NF4WeightC(ctypes.Structure):
    _fields_ = [("codes", _p), ("absmax_q", _p), ("absmax_scale", _p), ("rows", _i64),
                ("cols", _i64), ("flags", ctypes.c_uint32)]


QLORA_NF4_ABSMAX_FP32 = 0x1  # qlora_nf4_weight.flags: the 4.5-bit format (fp32 block absmax)


_lib.nf4_storage_bytes.argtypes = [_i64, ctypes.POINTER(_sz), ctypes.POINTER(_sz), ctypes.POINTER(_sz)]
_lib.nf4_storage_bytes.restype = ctypes.c_int
_lib.nf4_quantize.argtypes = [_p, _i64, _p, _p, _p, _p]
_lib.nf4_quantize.restype = ctypes.c_int
_lib.nf4_dequantize.argtypes = [_p, _p, _p, _i64, _p, _p]
_lib.nf4_dequantize.restype = ctypes.c_int
_lib.qlora_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int]
_lib.qlora_workspace_bytes.restype = _sz
_lib.qlora_linear_fwd.argtypes = [ctypes.POINTER(_NF4WeightC), _p, _i64, _p, _p, _i64, ctypes.c_float,
                                  _p, _p, _sz, _p]
_lib.qlora_linear_fwd.restype = ctypes.c_int
_lib.qlora_linear_bwd.argtypes = [ctypes.POINTER(_NF4WeightC), _p, _p, _i64, _p, _p, _i64,
                                  ctypes.c_float, _p, _p, _p, _p, _sz, _p]
_lib.qlora_linear_bwd.restype = ctypes.c_int
_lib.qlora_workspace_bytes_multi.argtypes = [_i64, _i64, ctypes.POINTER(_i64), ctypes.c_int, _i64,
                                             ctypes.c_int]
_lib.qlora_workspace_bytes_multi.restype = _sz
_lib.qlora_linear_fwd_multi.argtypes = [ctypes.POINTER(_NF4WeightC), ctypes.c_int, _p, _i64,
                                        ctypes.POINTER(_p), ctypes.POINTER(_p), _i64, ctypes.c_float,
                                        _p, _p, _sz, _p]
_lib.qlora_linear_fwd_multi.restype = ctypes.c_int
_lib.qlora_linear_bwd_multi.argtypes = [ctypes.POINTER(_NF4WeightC), ctypes.c_int, _p, _p, _i64,
                                        ctypes.POINTER(_p), ctypes.POINTER(_p), _i64, ctypes.c_float,
                                        _p, ctypes.POINTER(_p), ctypes.POINTER(_p), _p, _sz, _p]
_lib.qlora_linear_bwd_multi.restype = ctypes.c_int
_lib.nf4_quantize_nodq.argtypes = [_p, _i64, _p, _p, _p]
_lib.nf4_quantize_nodq.restype = ctypes.c_int
_lib.nf4_dequantize_nodq.argtypes = [_p, _p, _i64, _p, _p]
_lib.nf4_dequantize_nodq.restype = ctypes.c_int
_lib.qlora_merge_workspace_bytes.argtypes = [_i64, _i64, _i64]
_lib.qlora_merge_workspace_bytes.restype = _sz
_lib.qlora_merge.argtypes = [ctypes.POINTER(_NF4WeightC), _p, _p, _i64, ctypes.c_float, _p, _p, _sz, _p]
_lib.qlora_merge.restype = ctypes.c_int
_lib.qlora_workspace_bytes_dropout.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int]
_lib.qlora_workspace_bytes_dropout.restype = _sz
_lib.qlora_linear_fwd_dropout.argtypes = [ctypes.POINTER(_NF4WeightC), _p, _i64, _p, ctypes.c_float, _p,
                                          _p, _i64, ctypes.c_float, _p, _p, _sz, _p]
_lib.qlora_linear_fwd_dropout.restype = ctypes.c_int
_lib.qlora_linear_bwd_dropout.argtypes = [ctypes.POINTER(_NF4WeightC), _p, _p, _i64, _p, ctypes.c_float,
                                          _p, _p, _i64, ctypes.c_float, _p, _p, _p, _p, _sz, _p]
_lib.qlora_linear_bwd_dropout.restype = ctypes.c_int
_lib.qlora_workspace_bytes_flags.argtypes = [_i64, _i64, ctypes.POINTER(_i64), ctypes.c_int, _i64, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_uint32]
_lib.qlora_workspace_bytes_flags.restype = _sz
_lib.qlora_workspace_bytes_bwd_min.argtypes = [_i64, _i64, ctypes.POINTER(_i64), ctypes.c_int, _i64,
                                                ctypes.c_int, ctypes.c_uint32]
_lib.qlora_workspace_bytes_bwd_min.restype = _sz
_lib.qlora_workspace_bytes_fwd_min.argtypes = [_i64, _i64, ctypes.POINTER(_i64), ctypes.c_int, _i64,
                                                ctypes.c_int, ctypes.c_uint32]
_lib.qlora_workspace_bytes_fwd_min.restype = _sz
_lib.nf4_code_buckets.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_uint32)]
_lib.nf4_code_buckets.restype = None
_lib.qlora_noalloc_scratch_bytes.argtypes = []
_lib.qlora_noalloc_scratch_bytes.restype = _sz
_lib.qlora_linear_fwd_noalloc.argtypes = [ctypes.POINTER(_NF4WeightC), _p, _i64, _p, _p, _i64, ctypes.c_float,
                                          _p, _p]
_lib.qlora_linear_fwd_noalloc.restype = ctypes.c_int
_lib.nf4_codebook.argtypes = [ctypes.POINTER(ctypes.c_float)]
_lib.nf4_codebook.restype = None
_lib.nf4_code_thresholds.argtypes = [ctypes.POINTER(ctypes.c_float)]
_lib.nf4_code_thresholds.restype = None
_lib.qlora_status_string.argtypes = [ctypes.c_int]
_lib.qlora_status_string.restype = ctypes.c_char_p


def _status_string(status: int) -> str:
    return _lib.qlora_status_string(int(status)).decode()


qlora_status_string = _status_string


def _check(status: int, where: str):
    if status != QLORA_OK:
        raise QloraError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, dtype, name: str, numel: int = None):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")


@dataclass
class NF4Weight:
    """Frozen NF4 weight [rows = out_features, cols = in_features].  flags 0:
    double-quantized (absmax_q uint8 per block, absmax_scale fp32 per 256
    blocks); QLORA_NF4_ABSMAX_FP32: the 4.5-bit format (absmax_q None,
    absmax_scale the fp32 absmax of each block)."""
    codes: torch.Tensor          # uint8 [rows*cols/2]
    absmax_q: torch.Tensor       # uint8 [rows*cols/64], or None (4.5-bit format)
    absmax_scale: torch.Tensor   # float32 [ceil(rows*cols/16384)], or [rows*cols/64]
    rows: int
    cols: int
    flags: int = 0

    def _c(self):
        q = None if self.absmax_q is None else self.absmax_q.data_ptr()
        return _NF4WeightC(self.codes.data_ptr(), q, self.absmax_scale.data_ptr(), self.rows, self.cols,
                           self.flags)


def nf4_storage_bytes(numel: int):
    c, q, s = _sz(), _sz(), _sz()
    _check(_lib.nf4_storage_bytes(numel, ctypes.byref(c), ctypes.byref(q), ctypes.byref(s)),
           "nf4_storage_bytes")
    return c.value, q.value, s.value


def nf4_quantize(w: torch.Tensor, codes=None, absmax_q=None, absmax_scale=None):
    """fp32 device tensor (any shape, numel % 64 == 0) -> (codes, absmax_q, absmax_scale)."""
    _need(w, torch.float32, "w")
    n = w.numel()
    cb, qb, sb = nf4_storage_bytes(n)
    dev = w.device
    if codes is None:
        codes = torch.empty(cb, dtype=torch.uint8, device=dev)
    if absmax_q is None:
        absmax_q = torch.empty(qb, dtype=torch.uint8, device=dev)
    if absmax_scale is None:
        absmax_scale = torch.empty(sb // 4, dtype=torch.float32, device=dev)
    _need(codes, torch.uint8, "codes", cb)
    _need(absmax_q, torch.uint8, "absmax_q", qb)
    _need(absmax_scale, torch.float32, "absmax_scale", sb // 4)
    _check(_lib.nf4_quantize(_ptr(w), n, _ptr(codes), _ptr(absmax_q), _ptr(absmax_scale),
                             _stream(dev)), "nf4_quantize")
    return codes, absmax_q, absmax_scale


def nf4_quantize_weight(w: torch.Tensor) -> NF4Weight:
    """Quantizes a [out, in] fp32 weight into an NF4Weight."""
    if w.dim() != 2:
        raise ValueError("weight must be 2-D [out, in]")
    c, q, s = nf4_quantize(w)
    return NF4Weight(c, q, s, w.shape[0], w.shape[1])


def nf4_quantize_weight_nodq(w: torch.Tensor) -> NF4Weight:
    """Quantizes a [out, in] fp32 weight into an NF4Weight of the 4.5-bit
    format (exact fp32 block absmax, no double quantization)."""
    if w.dim() != 2:
        raise ValueError("weight must be 2-D [out, in]")
    c, a = nf4_quantize_nodq(w)
    return NF4Weight(c, None, a, w.shape[0], w.shape[1], QLORA_NF4_ABSMAX_FP32)


def nf4_dequantize(codes, absmax_q, absmax_scale, numel: int, out=None):
    """-> bf16 device tensor [numel]."""
    if out is None:
        out = torch.empty(numel, dtype=torch.bfloat16, device=codes.device)
    _need(out, torch.bfloat16, "out", numel)
    _check(_lib.nf4_dequantize(_ptr(codes), _ptr(absmax_q), _ptr(absmax_scale), numel, _ptr(out),
                               _stream(codes.device)), "nf4_dequantize")
    return out


def nf4_quantize_nodq(w: torch.Tensor, codes=None, absmax=None):
    """fp32 device tensor (numel % 64 == 0) -> (codes uint8 [numel/2], absmax fp32 [numel/64]),
    no double quantization (4.5 bits per weight)."""
    _need(w, torch.float32, "w")
    n = w.numel()
    if codes is None:
        codes = torch.empty(n // 2, dtype=torch.uint8, device=w.device)
    if absmax is None:
        absmax = torch.empty(n // 64, dtype=torch.float32, device=w.device)
    _need(codes, torch.uint8, "codes", n // 2)
    _need(absmax, torch.float32, "absmax", n // 64)
    _check(_lib.nf4_quantize_nodq(_ptr(w), n, _ptr(codes), _ptr(absmax), _stream(w.device)),
           "nf4_quantize_nodq")
    return codes, absmax


def nf4_dequantize_nodq(codes, absmax, numel: int, out=None):
    """-> bf16 device tensor [numel] (fp32 block absmax, no double quantization)."""
    if out is None:
        out = torch.empty(numel, dtype=torch.bfloat16, device=codes.device)
    _need(out, torch.bfloat16, "out", numel)
    _check(_lib.nf4_dequantize_nodq(_ptr(codes), _ptr(absmax), numel, _ptr(out), _stream(codes.device)),
           "nf4_dequantize_nodq")
    return out


def qlora_workspace_bytes(T: int, in_features: int, out_features: int, r: int, backward: bool) -> int:
    return int(_lib.qlora_workspace_bytes(T, in_features, out_features, r, 1 if backward else 0))


_WS_CACHE = {}


def make_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace of at least nbytes (the library needs it uninitialised)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def qlora_workspace_bytes_flags(T: int, in_features: int, out_features, r: int, backward: bool,
                                dropout: bool = False, flags: int = 0) -> int:
    outs = (_i64 * len(out_features))(*[int(o) for o in out_features])
    return int(_lib.qlora_workspace_bytes_flags(T, in_features, outs, len(out_features), r,
                                                1 if backward else 0, 1 if dropout else 0, flags))


def qlora_workspace_bytes_fwd_min(T: int, in_features: int, out_features, r: int, dropout: bool = False,
                                  flags: int = 0) -> int:
    """The smallest forward workspace: no expanded W_hat (the GEMM then
    dequantizes the weight tiles while staging them)."""
    outs = (_i64 * len(out_features))(*[int(o) for o in out_features])
    return int(_lib.qlora_workspace_bytes_fwd_min(T, in_features, outs, len(out_features), r,
                                                  1 if dropout else 0, flags))


def qlora_workspace_bytes_bwd_min(T: int, in_features: int, out_features, r: int, dropout: bool = False,
                                  flags: int = 0) -> int:
    """The smallest backward workspace: no expanded W_hat^T (the dX GEMM then
    dequantizes the weight tiles while staging them)."""
    outs = (_i64 * len(out_features))(*[int(o) for o in out_features])
    return int(_lib.qlora_workspace_bytes_bwd_min(T, in_features, outs, len(out_features), r,
                                                  1 if dropout else 0, flags))


def _workspace(ws, T, n_in, n_out, r, backward, device, flags=0):
    """Caller's workspace, or a cached one per (device, stream) that grows as
    needed (concurrent streams get separate buffers)."""
    need = qlora_workspace_bytes_flags(T, n_in, [n_out], r, backward, False, flags)
    if ws is None:
        key = (torch.device(device).index, torch.cuda.current_stream(device).cuda_stream)
        ws = _WS_CACHE.get(key)
        if ws is None or ws.numel() < need:
            ws = make_workspace(need, device)
            _WS_CACHE[key] = ws
    return ws, ws.numel() * ws.element_size()


def qlora_linear_fwd(W: NF4Weight, X, A, B, r: int, alpha: float, Y=None, ws=None):
    """Y [T, out] bf16 = X W_hat^T + (alpha/r) (X A^T) B^T."""
    T = X.shape[0]
    _need(X, torch.bfloat16, "X", T * W.cols)
    _need(A, torch.bfloat16, "A", r * W.cols)
    _need(B, torch.bfloat16, "B", W.rows * r)
    if Y is None:
        Y = torch.empty(T, W.rows, dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, "Y", T * W.rows)
    ws, ws_bytes = _workspace(ws, T, W.cols, W.rows, r, False, X.device, W.flags)
    wc = W._c()
    _check(_lib.qlora_linear_fwd(ctypes.byref(wc), _ptr(X), T, _ptr(A), _ptr(B), r, float(alpha),
                                 _ptr(Y), _ptr(ws), ws_bytes, _stream(X.device)), "qlora_linear_fwd")
    return Y


def qlora_noalloc_scratch_bytes() -> int:
    return int(_lib.qlora_noalloc_scratch_bytes())


def qlora_linear_fwd_noalloc(W: NF4Weight, X, A, B, r: int, alpha: float, Y):
    """qlora_linear_fwd on the library's static scratch: Y must be given (the
    call allocates nothing); calls that overlap on one GPU race."""
    T = X.shape[0]
    _need(X, torch.bfloat16, "X", T * W.cols)
    _need(A, torch.bfloat16, "A", r * W.cols)
    _need(B, torch.bfloat16, "B", W.rows * r)
    _need(Y, torch.bfloat16, "Y", T * W.rows)
    wc = W._c()
    _check(_lib.qlora_linear_fwd_noalloc(ctypes.byref(wc), _ptr(X), T, _ptr(A), _ptr(B), r, float(alpha),
                                         _ptr(Y), _stream(X.device)), "qlora_linear_fwd_noalloc")
    return Y


def qlora_linear_bwd(W: NF4Weight, X, dY, A, B, r: int, alpha: float, dX=None, dA=None, dB=None,
                     ws=None):
    """-> (dX [T, in] bf16, dA [r, in] fp32, dB [out, r] fp32)."""
    T = X.shape[0]
    _need(X, torch.bfloat16, "X", T * W.cols)
    _need(dY, torch.bfloat16, "dY", T * W.rows)
    _need(A, torch.bfloat16, "A", r * W.cols)
    _need(B, torch.bfloat16, "B", W.rows * r)
    dev = X.device
    if dX is None:
        dX = torch.empty(T, W.cols, dtype=torch.bfloat16, device=dev)
    if dA is None:
        dA = torch.empty(r, W.cols, dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty(W.rows, r, dtype=torch.float32, device=dev)
    _need(dX, torch.bfloat16, "dX", T * W.cols)
    _need(dA, torch.float32, "dA", r * W.cols)
    _need(dB, torch.float32, "dB", W.rows * r)
    ws, ws_bytes = _workspace(ws, T, W.cols, W.rows, r, True, dev, W.flags)
    wc = W._c()
    _check(_lib.qlora_linear_bwd(ctypes.byref(wc), _ptr(X), _ptr(dY), T, _ptr(A), _ptr(B), r,
                                 float(alpha), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), ws_bytes,
                                 _stream(dev)), "qlora_linear_bwd")
    return dX, dA, dB


def qlora_workspace_bytes_dropout(T: int, in_features: int, out_features: int, r: int,
                                  backward: bool) -> int:
    return int(_lib.qlora_workspace_bytes_dropout(T, in_features, out_features, r, 1 if backward else 0))


def _dropout_ws(ws, T, n_in, n_out, r, backward, device, flags=0):
    need = qlora_workspace_bytes_flags(T, n_in, [n_out], r, backward, True, flags)
    if ws is None:
        key = (torch.device(device).index, torch.cuda.current_stream(device).cuda_stream)
        ws = _WS_CACHE.get(key)
        if ws is None or ws.numel() < need:
            ws = make_workspace(need, device)
            _WS_CACHE[key] = ws
    return ws, ws.numel() * ws.element_size()


def qlora_linear_fwd_dropout(W: NF4Weight, X, keep, p: float, A, B, r: int, alpha: float, Y=None,
                             ws=None):
    """Y = X W_hat^T + (alpha/r) ((keep o X / (1 - p)) A^T) B^T; keep is the
    packed mask [T, in/8] uint8 (bit k % 8 of byte k / 8 = element k kept)."""
    T = X.shape[0]
    _need(X, torch.bfloat16, "X", T * W.cols)
    _need(keep, torch.uint8, "keep", T * (W.cols // 8))
    _need(A, torch.bfloat16, "A", r * W.cols)
    _need(B, torch.bfloat16, "B", W.rows * r)
    if Y is None:
        Y = torch.empty(T, W.rows, dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, "Y", T * W.rows)
    ws, ws_bytes = _dropout_ws(ws, T, W.cols, W.rows, r, False, X.device, W.flags)
    wc = W._c()
    _check(_lib.qlora_linear_fwd_dropout(ctypes.byref(wc), _ptr(X), T, _ptr(keep), float(p), _ptr(A),
                                         _ptr(B), r, float(alpha), _ptr(Y), _ptr(ws), ws_bytes,
                                         _stream(X.device)), "qlora_linear_fwd_dropout")
    return Y


def qlora_linear_bwd_dropout(W: NF4Weight, X, dY, keep, p: float, A, B, r: int, alpha: float, dX=None,
                             dA=None, dB=None, ws=None):
    """Backward of qlora_linear_fwd_dropout with the same mask ->
    (dX [T, in] bf16, dA [r, in] fp32, dB [out, r] fp32)."""
    T = X.shape[0]
    _need(X, torch.bfloat16, "X", T * W.cols)
    _need(dY, torch.bfloat16, "dY", T * W.rows)
    _need(keep, torch.uint8, "keep", T * (W.cols // 8))
    _need(A, torch.bfloat16, "A", r * W.cols)
    _need(B, torch.bfloat16, "B", W.rows * r)
    dev = X.device
    if dX is None:
        dX = torch.empty(T, W.cols, dtype=torch.bfloat16, device=dev)
    if dA is None:
        dA = torch.empty(r, W.cols, dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty(W.rows, r, dtype=torch.float32, device=dev)
    _need(dX, torch.bfloat16, "dX", T * W.cols)
    _need(dA, torch.float32, "dA", r * W.cols)
    _need(dB, torch.float32, "dB", W.rows * r)
    ws, ws_bytes = _dropout_ws(ws, T, W.cols, W.rows, r, True, dev, W.flags)
    wc = W._c()
    _check(_lib.qlora_linear_bwd_dropout(ctypes.byref(wc), _ptr(X), _ptr(dY), T, _ptr(keep), float(p),
                                         _ptr(A), _ptr(B), r, float(alpha), _ptr(dX), _ptr(dA), _ptr(dB),
                                         _ptr(ws), ws_bytes, _stream(dev)), "qlora_linear_bwd_dropout")
    return dX, dA, dB


def qlora_merge_workspace_bytes(in_features: int, out_features: int, r: int) -> int:
    return int(_lib.qlora_merge_workspace_bytes(in_features, out_features, r))


def qlora_merge(W: NF4Weight, A, B, r: int, alpha: float, out=None, ws=None):
    """W_merged [out, in] bf16 = bf16(W_hat + (alpha/r) B A)."""
    _need(A, torch.bfloat16, "A", r * W.cols)
    _need(B, torch.bfloat16, "B", W.rows * r)
    dev = A.device
    if out is None:
        out = torch.empty(W.rows, W.cols, dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out", W.rows * W.cols)
    need = qlora_merge_workspace_bytes(W.cols, W.rows, r)
    if ws is None:
        ws = make_workspace(need, dev)
    wc = W._c()
    _check(_lib.qlora_merge(ctypes.byref(wc), _ptr(A), _ptr(B), r, float(alpha), _ptr(out), _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(dev)), "qlora_merge")
    return out


def qlora_workspace_bytes_multi(T: int, in_features: int, out_features, r: int, backward: bool) -> int:
    outs = (_i64 * len(out_features))(*[int(o) for o in out_features])
    return int(_lib.qlora_workspace_bytes_multi(T, in_features, outs, len(out_features), r,
                                                1 if backward else 0))


def _multi_ws(ws, T, n_in, outs, r, backward, device, flags=0):
    need = qlora_workspace_bytes_flags(T, n_in, outs, r, backward, False, flags)
    if ws is None:
        ws = make_workspace(need, device)
    return ws, ws.numel() * ws.element_size()


def _ptr_array(ts):
    return (_p * len(ts))(*[t.data_ptr() for t in ts])


def qlora_linear_fwd_multi(Ws, X, As, Bs, r: int, alpha: float, Y=None, ws=None):
    """Projections sharing X (e.g. q|k|v, gate|up): Y [T, sum out_i] bf16 with
    projection i's columns side by side."""
    n = len(Ws)
    T = X.shape[0]
    n_in = Ws[0].cols
    outs = [W.rows for W in Ws]
    _need(X, torch.bfloat16, "X", T * n_in)
    for W, A, B in zip(Ws, As, Bs):
        _need(A, torch.bfloat16, "A", r * W.cols)
        _need(B, torch.bfloat16, "B", W.rows * r)
    if Y is None:
        Y = torch.empty(T, sum(outs), dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, "Y", T * sum(outs))
    ws, ws_bytes = _multi_ws(ws, T, n_in, outs, r, False, X.device, Ws[0].flags)
    wc = (_NF4WeightC * n)(*[W._c() for W in Ws])
    _check(_lib.qlora_linear_fwd_multi(wc, n, _ptr(X), T, _ptr_array(As), _ptr_array(Bs), r,
                                       float(alpha), _ptr(Y), _ptr(ws), ws_bytes, _stream(X.device)),
           "qlora_linear_fwd_multi")
    return Y


def qlora_linear_bwd_multi(Ws, X, dY, As, Bs, r: int, alpha: float, dX=None, dAs=None, dBs=None,
                           ws=None):
    """-> (dX [T, in] bf16 summed over the projections, [dA_i fp32], [dB_i fp32])."""
    n = len(Ws)
    T = X.shape[0]
    n_in = Ws[0].cols
    outs = [W.rows for W in Ws]
    dev = X.device
    _need(X, torch.bfloat16, "X", T * n_in)
    _need(dY, torch.bfloat16, "dY", T * sum(outs))
    if dX is None:
        dX = torch.empty(T, n_in, dtype=torch.bfloat16, device=dev)
    if dAs is None:
        dAs = [torch.empty(r, n_in, dtype=torch.float32, device=dev) for _ in range(n)]
    if dBs is None:
        dBs = [torch.empty(o, r, dtype=torch.float32, device=dev) for o in outs]
    ws, ws_bytes = _multi_ws(ws, T, n_in, outs, r, True, dev, Ws[0].flags)
    wc = (_NF4WeightC * n)(*[W._c() for W in Ws])
    _check(_lib.qlora_linear_bwd_multi(wc, n, _ptr(X), _ptr(dY), T, _ptr_array(As), _ptr_array(Bs),
                                       r, float(alpha), _ptr(dX), _ptr_array(dAs), _ptr_array(dBs),
                                       _ptr(ws), ws_bytes, _stream(dev)), "qlora_linear_bwd_multi")
    return dX, dAs, dBs


def nf4_codebook():
    out = (ctypes.c_float * 16)()
    _lib.nf4_codebook(out)
    return [float(v) for v in out]


def nf4_code_buckets():
    """-> (thr [33], base [33]): the quantize kernel's code lookup on X = 16 x."""
    thr, base = (ctypes.c_float * 33)(), (ctypes.c_uint32 * 33)()
    _lib.nf4_code_buckets(thr, base)
    return [float(v) for v in thr], [int(v) for v in base]


def nf4_code_thresholds():
    out = (ctypes.c_float * 15)()
    _lib.nf4_code_thresholds(out)
    return [float(v) for v in out]
