"""NF4 blockwise quantization with double quantization (oracle; test
infrastructure only).

Every step is the plain definition, evaluated in IEEE fp32 with NumPy, in the
order the pages give it.  Readings of points the pages leave open are marked
"Reading:".

Storage produced by :func:`quantize` (numel must be a multiple of 64):
    codes     uint8[numel/2]      two 4-bit codes per byte
    absmax_q  uint8[numel/64]     8-bit double-quantized block absmax
    scale     float32[ceil(numel/16384)]  one fp32 scale per 256 blocks
"""

import numpy as np

from .codebook import nf4_levels

BLOCK = 64          # weights per absmax block (ultralytics "QLoRA", NF4 bullet)
GROUP = 256         # blocks per double-quant scale (same page, double-quant bullet)
DQ_LEVELS = 255     # largest 8-bit code


# --------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------

def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """IEEE round-to-nearest-even of finite fp32 values to bfloat16; returns
    the raw 16-bit patterns (uint16).  The pages keep the dequantized weight
    in bfloat16 ("bnb_4bit_compute_dtype=torch.bfloat16"; ultralytics
    "QLoRA": NF4 weights are dequantized to bfloat16 right before the matmul).
    Rounding of the 32-bit pattern: add 0x7FFF plus the lowest kept bit, then
    drop the low 16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    return ((u + 0x7FFF + keep_lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Steps Q1..Q4
# --------------------------------------------------------------------------

def block_absmax(w: np.ndarray) -> np.ndarray:
    """Q1.  One scale per 64 consecutive weights of the row-major flattening:
    the largest |w| in the block (paperclase "QLoRA", Parte 4 layer:
    weight.reshape(-1, 64) then abs().max; ultralytics "QLoRA": one absmax
    scale per block of 64 weights).  Exact in fp32."""
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    if w.size % BLOCK:
        raise ValueError("numel must be a multiple of 64")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight (precondition violation)")
    return np.abs(w.reshape(-1, BLOCK)).max(axis=1)


def normalized(w: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """x = fl32(w / absmax) per block (correctly rounded fp32 division, as the
    page's `weights / absmax`).  Reading: a block whose absmax is 0 holds only
    zeros; its x is defined as 0 (0/0 is not taken)."""
    wb = np.ascontiguousarray(w, dtype=np.float32).reshape(-1, BLOCK)
    a = absmax.astype(np.float32)[:, None]
    safe = np.where(a == 0, np.float32(1), a)
    with np.errstate(invalid="ignore", divide="ignore"):
        x = (wb / safe).astype(np.float32)
    x[np.broadcast_to(a == 0, x.shape)] = np.float32(0)
    return x


def nearest_level(x: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Q3 (definition).  Code = index of the level nearest to x: the first
    index j minimising the fp32 distance |fl32(x - L_j)| (torch argmin returns
    the first minimum; paperclase "QLoRA", Parte 4: "argmin de la distancia";
    ultralytics "QLoRA" listing: `(x - levels).abs().argmin`).  Brute force
    over all levels.  Works on any shape; returns uint8 codes."""
    x = np.asarray(x, dtype=np.float32)
    lv = np.asarray(levels, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint8)
    step = 1 << 20
    for s in range(0, flat.size, step):
        chunk = flat[s:s + step]
        d = np.abs(chunk[:, None] - lv[None, :])      # fp32 subtraction, exact |.|
        out[s:s + step] = d.argmin(axis=1)             # first minimum wins ties
    return out.reshape(x.shape)


def double_quantize(absmax: np.ndarray):
    """Q2.  Double quantization of the block absmax values: per group of 256
    consecutive blocks one fp32 scale s_g and one 8-bit code per block
    (ultralytics "QLoRA", double-quant bullet: scales quantized to 8 bits in
    blocks of 256; paperclase "QLoRA", Parte 3: 8 bits per absmax plus a
    32-bit scale every 256 blocks).

    Reading (the pages give only the bit budget): the absmax recipe of
    paperclase Parte 1 (divide by the group's largest value, scale, round)
    carried to 8 bits over non-negative data:
        s_g = max_b a_b                  (fp32, exact)
        q_b = rne(fl32(fl32(a_b / s_g) * 255))   in 0..255
    A group whose s_g is 0 stores s_g = 0 and q_b = 0.  The last group may be
    partial (its own max over the blocks present)."""
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    nb = a.size
    ng = (nb + GROUP - 1) // GROUP
    # zero padding of a partial last group leaves its max unchanged (a >= 0)
    padded = np.zeros(ng * GROUP, dtype=np.float32)
    padded[:nb] = a
    groups = padded.reshape(ng, GROUP)
    scale = groups.max(axis=1)                                  # s_g
    s_b = np.repeat(scale, GROUP)[:nb]                          # each block's s_g
    nonzero = s_b > 0
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = (a / np.where(nonzero, s_b, np.float32(1))).astype(np.float32)
    scaled = (ratio * np.float32(DQ_LEVELS)).astype(np.float32)
    q = np.where(nonzero, np.rint(scaled), 0).astype(np.uint8)  # rint: half to even
    return q, scale.astype(np.float32)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Q4.  Two 4-bit codes per byte (paperclase "QLoRA", Parte 4: one byte per
    code in the lesson, "a real format packs two").  Reading of the order:
    element 2i in the low nibble, element 2i+1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        raise ValueError("odd number of codes")
    return (c[0::2] & 0xF) | ((c[1::2] & 0xF) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & 0xF
    out[1::2] = p >> 4
    return out


def nf4_codes(w: np.ndarray, absmax: np.ndarray, levels=None, nearest=None) -> np.ndarray:
    """Q3 on a whole tensor: per block x = fl32(w / a_b), then nearest NF4
    level.  The codes use the exact fp32 absmax; double quantization
    compresses the scales afterwards (paperclase Parte 3: each block stores
    its absmax and QLoRA compresses that too).  `nearest` lets the tests
    swap in the plain-C brute force (same definition) for big tensors."""
    lv = nf4_levels() if levels is None else levels
    x = normalized(w, absmax)
    find = nearest_level if nearest is None else nearest
    return find(x, lv).reshape(-1)


def quantize(w: np.ndarray, nearest=None):
    """Q1..Q4: fp32 weight (any shape, row-major, numel % 64 == 0) ->
    (codes uint8[numel/2], absmax_q uint8[numel/64], scale f32[ceil(numel/16384)])."""
    a = block_absmax(w)
    codes = nf4_codes(w, a, nearest=nearest)
    q, s = double_quantize(a)
    return pack_nibbles(codes), q, s


# --------------------------------------------------------------------------
# Step D1
# --------------------------------------------------------------------------

def dequant_absmax(absmax_q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Reading: the inverse of Q2 in the order of paperclase Parte 1's
    `codigo / 7 * absmax`: a_hat_b = fl32(fl32(q_b / 255) * s_g)."""
    q = np.asarray(absmax_q, dtype=np.uint8).astype(np.float32)
    g = np.arange(q.size) // GROUP
    ratio = (q / np.float32(DQ_LEVELS)).astype(np.float32)
    return (ratio * np.asarray(scale, dtype=np.float32)[g]).astype(np.float32)


def dequantize_f32(codes_packed, absmax_q, scale, levels=None) -> np.ndarray:
    """fl32(L[c] * a_hat) per element (paperclase "QLoRA", Parte 2:
    w_hat = NF4[c] * absmax; Parte 4 forward: NF4[codigo] * absmax)."""
    lv = nf4_levels() if levels is None else levels
    c = unpack_nibbles(codes_packed)
    ahat = dequant_absmax(absmax_q, scale)
    per_elem = np.repeat(ahat, BLOCK)
    return (lv[c] * per_elem).astype(np.float32)


def dequantize(codes_packed, absmax_q, scale) -> np.ndarray:
    """D1: the dequantized weight as bf16 bit patterns (uint16[numel]):
    w_hat = bf16_rne(fl32(L[c] * a_hat))."""
    return bf16_rne_bits(dequantize_f32(codes_packed, absmax_q, scale))


# --------------------------------------------------------------------------
# The format without double quantization (4 + 32/64 = 4.5 bits per weight)
# --------------------------------------------------------------------------

def quantize_nodq(w: np.ndarray, nearest=None):
    """Q1, Q3, Q4 with the exact fp32 block absmax stored as is (paperclase
    "QLoRA", Parte 3: 4 bits plus the absmax per block; ultralytics "QLoRA":
    the MSE comparison quantizes with exact block absmax values) ->
    (codes uint8[numel/2], absmax f32[numel/64])."""
    a = block_absmax(w)
    return pack_nibbles(nf4_codes(w, a, nearest=nearest)), a


def dequantize_nodq_f32(codes_packed, absmax, levels=None) -> np.ndarray:
    """fl32(L[c] * a_b) per element."""
    lv = nf4_levels() if levels is None else levels
    c = unpack_nibbles(codes_packed)
    return (lv[c] * np.repeat(np.asarray(absmax, dtype=np.float32), BLOCK)).astype(np.float32)


def dequantize_nodq(codes_packed, absmax) -> np.ndarray:
    """bf16_rne(fl32(L[c] * a_b)) as bf16 bit patterns."""
    return bf16_rne_bits(dequantize_nodq_f32(codes_packed, absmax))


# --------------------------------------------------------------------------
# Quantizers used only for the pages' worked examples
# --------------------------------------------------------------------------

def absmax_int4(w: np.ndarray):
    """paperclase "QLoRA", Parte 1, "absmax, en formulas": one block,
    c_i = round(7 * w_i / max|w|) (half to even, fp32 in the lesson's order
    w / absmax * 7), w_hat_i = c_i / 7 * absmax.  Returns (absmax, c, w_hat)."""
    w = np.asarray(w, dtype=np.float32)
    a = np.abs(w).max()
    c = np.rint(((w / a).astype(np.float32) * np.float32(7)).astype(np.float32))
    w_hat = ((c / np.float32(7)).astype(np.float32) * a).astype(np.float32)
    return a, c.astype(np.int32), w_hat


def blockwise_restore(w: np.ndarray, levels: np.ndarray, nearest=None) -> np.ndarray:
    """Exact-absmax reconstruction with a given level set, no double quant and
    no bf16: levels[nearest(w / a)] * a (ultralytics "QLoRA" MSE experiment)."""
    a = block_absmax(w)
    find = nearest_level if nearest is None else nearest
    c = find(normalized(w, a), levels).reshape(-1, BLOCK)
    return (levels[c] * a[:, None]).astype(np.float32).reshape(np.shape(w))
