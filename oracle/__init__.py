"""CPU oracle for the NF4 / double-quant / QLoRA-linear path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The product path (the HIP library and its Python binding) never imports it,
and this package imports nothing from the product path: the two share no
kernels, headers, tables, constant generators or pre/post-processing.

Everything here is the plain, slow, obviously-correct definition of what the
path computes, written from these pages:

* ultralytics glossary page "QLoRA" (pt), section "Como funciona a QLoRA":
  the NF4 bullet (16 quantile levels, one absmax per 64-weight block), the
  double-quantization bullet (absmax values to 8 bits in blocks of 256,
  overhead 0.5 -> ~0.127 bits/param), the NF4 construction listing and the
  MSE comparison printed after it, and the dequantize-to-bf16-before-matmul
  paragraph.
* paperclase lesson "QLoRA" (es): Parte 1 (absmax worked example and its three
  formulas), Parte 2 (quantile construction, toy codebook), Parte 3 (bits per
  parameter, Gemma 2 2B storage table), Parte 4 (the hand-written 4-bit layer
  and the gradient equations under "El gradiente atraviesa la base de 4 bits").

Modules:
    codebook  -- NF4 levels (page construction), toy levels, uniform levels
    nf4       -- blockwise absmax, nearest-level codes, double quantization,
                 nibble packing, dequantization to bf16, int4 absmax quantizer
    dense     -- fp64 forward/backward of the QLoRA linear
    storage   -- bits/param and storage closed forms
    native    -- ctypes loader for the plain-C brute-force nearest-level search

Pins (what each part is checked against) live in tests/test_oracle_*.py.
Parity unpinned: none of the functions here; the page figures that need
trained weights or datasets (Gemma q_proj errors, mirrored-digits accuracy,
the 0.19 toy-layer deviation) are not reproduced and not claimed.
"""

from . import codebook, nf4, dense, storage  # noqa: F401

__all__ = ["codebook", "nf4", "dense", "storage"]
