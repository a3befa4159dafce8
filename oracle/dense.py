"""fp64 forward and backward of the QLoRA linear (oracle; test infrastructure
only).

The method reaches, up to rounding order, the plain dense result, so the
oracle is that definition written out: the bf16 inputs are widened exactly to
fp64 and every product is a fp64 matmul (a library primitive).  No result is
rounded.

Shapes (row-major):  X [T, in], W_hat [out, in], A [r, in], B [out, r],
dY [T, out].  Scale s = alpha / r.

Forward (paperclase "QLoRA", Parte 4, "El gradiente atraviesa la base de 4
bits", h = W_hat x + (alpha/r) B A x; same page, the layer's forward adds
escala * x A^T B^T to the linear):
    U = X A^T                      [T, r]
    Y = X W_hat^T + s U B^T        [T, out]
Backward (same section: dL/dx = (W_hat + (alpha/r) B A)^T dL/dh; no gradient
for W_hat, the codes are not parameters; A and B are the only trained
tensors, their gradients by the chain rule):
    V  = dY B                      [T, r]
    dX = dY W_hat + s V A          [T, in]
    dA = s V^T X                   [r, in]
    dB = s dY^T U                  [out, r]
"""

import numpy as np

from .nf4 import bf16_bits_to_f32


def widen(bits_or_f32: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or fp32 values -> exact fp64."""
    a = np.asarray(bits_or_f32)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def linear_fwd(W_hat, X, A, B, alpha: float, r: int) -> np.ndarray:
    """Y = X W_hat^T + (alpha/r) (X A^T) B^T, fp64."""
    s = float(alpha) / float(r)
    Xd, Wd, Ad, Bd = widen(X), widen(W_hat), widen(A), widen(B)
    U = Xd @ Ad.T
    return Xd @ Wd.T + s * (U @ Bd.T)


def linear_bwd(W_hat, X, dY, A, B, alpha: float, r: int):
    """(dX, dA, dB) in fp64 for the forward above."""
    s = float(alpha) / float(r)
    Xd, Wd, Ad, Bd, Gd = widen(X), widen(W_hat), widen(A), widen(B), widen(dY)
    U = Xd @ Ad.T
    V = Gd @ Bd
    dX = Gd @ Wd + s * (V @ Ad)
    dA = s * (V.T @ Xd)
    dB = s * (Gd.T @ U)
    return dX, dA, dB


def merge(W_hat, A, B, alpha: float, r: int) -> np.ndarray:
    """W_hat + (alpha/r) B A in fp64, unrounded: the adapter folded into the
    dequantized base for serving (coddykit "LoRA y QLoRA": merge_and_unload;
    ultralytics glossary "QLoRA", "Compromissos": the 4-bit base is
    dequantized to 16 bits before the merge).  Serving the merged weight is
    the same linear map as the forward above: X merge^T = X W_hat^T + s U B^T."""
    s = float(alpha) / float(r)
    return widen(W_hat) + s * (widen(B) @ widen(A))


def unpack_keep(keep_bytes, T: int, n_in: int) -> np.ndarray:
    """The dropout keep mask as a bool [T, in] array from its packed form:
    bytes [T, in/8], bit k % 8 of byte k / 8 of row t set = element (t, k)
    kept (the layout the library's dropout calls take)."""
    b = np.asarray(keep_bytes, dtype=np.uint8).reshape(T, n_in // 8)
    bits = (b[:, :, None] >> np.arange(8, dtype=np.uint8)[None, None, :]) & 1
    return bits.reshape(T, n_in).astype(bool)


def dropped_input(X, keep, p: float) -> np.ndarray:
    """X~ = keep o X / (1 - p): the adapter's input under LoRA dropout
    (coddykit "LoRA y QLoRA" configures lora_dropout = 0.05; reading: inverted
    dropout on the adapter input only, the base sees X)."""
    return np.where(keep, widen(X), 0.0) / (1.0 - float(p))


def linear_fwd_dropout(W_hat, X, A, B, alpha: float, r: int, keep, p: float) -> np.ndarray:
    """Y = X W_hat^T + (alpha/r) (X~ A^T) B^T, fp64, X~ as in dropped_input."""
    s = float(alpha) / float(r)
    Xd, Wd, Ad, Bd = widen(X), widen(W_hat), widen(A), widen(B)
    Xt = dropped_input(X, keep, p)
    return Xd @ Wd.T + s * ((Xt @ Ad.T) @ Bd.T)


def linear_bwd_dropout(W_hat, X, dY, A, B, alpha: float, r: int, keep, p: float):
    """(dX, dA, dB) in fp64 for linear_fwd_dropout with the mask held fixed
    (the chain rule through X~ = keep o X / (1 - p)):
        V  = dY B
        dX = dY W_hat + (keep / (1 - p)) o (s V A)
        dA = s V^T X~,   dB = s dY^T (X~ A^T)"""
    s = float(alpha) / float(r)
    Xd, Wd, Ad, Bd, Gd = widen(X), widen(W_hat), widen(A), widen(B), widen(dY)
    Xt = dropped_input(X, keep, p)
    V = Gd @ Bd
    dX = Gd @ Wd + np.where(keep, s * (V @ Ad), 0.0) / (1.0 - float(p))
    dA = s * (V.T @ Xt)
    dB = s * (Gd.T @ (Xt @ Ad.T))
    return dX, dA, dB


def rel_frobenius(got, ref) -> float:
    """||got - ref||_F / ||ref||_F in fp64 (the acceptance measure)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(r)
    num = np.linalg.norm(g - r)
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)
