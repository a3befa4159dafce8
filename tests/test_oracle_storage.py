"""Pins of the storage arithmetic against the tables the pages print."""

import numpy as np

from oracle import nf4 as onf4
from oracle import storage


def test_bits_and_gemma_table(golden):
    # paperclase "QLoRA", Parte 3, "Gemma 2 2B en cada formato"
    g = golden("paperclase_storage.txt")
    params = float(g["params"])
    for name in ("float32", "bfloat16", "4 + absmax", "4 + double"):
        bits_s, gb_s = g[name].split()
        bits = storage.BITS[name]
        assert f"{bits:.3f}" == bits_s
        assert f"{storage.gigabytes(params, bits):.2f}" == gb_s


def test_overhead_and_65b(golden):
    # ultralytics "QLoRA": 0.5 -> ~0.127 bits/param, ~3 GB saved on 65B,
    # ~130 GB in 16 bits, ~34 GB in 4 bits + double-quantized scales
    g = golden("paperclase_storage.txt")
    before = storage.BITS["4 + absmax"] - 4
    after = storage.BITS["4 + double"] - 4
    assert before == float(g["overhead_before"])
    assert f"{after:.3f}" == g["overhead_after_3dp"]
    p65 = float(g["params_65b"])
    saving = storage.gigabytes(p65, before - after)
    assert round(saving) == int(g["saving_65b_gb_approx"])
    assert round(storage.gigabytes(p65, 16)) == int(g["bf16_65b_gb_approx"])
    assert round(storage.gigabytes(p65, storage.BITS["4 + double"])) == int(g["nf4dq_65b_gb_approx"])


def test_buffers_realise_the_bit_budget(golden):
    # the oracle's actual buffers cost exactly 4 + 8/64 + 32/16384 bits per weight
    n = 64 * 256 * 3
    w = np.random.default_rng(0).standard_normal(n).astype(np.float32)
    packed, q, s = onf4.quantize(w)
    total_bits = 8 * (packed.nbytes + q.nbytes + s.nbytes)
    assert total_bits / n == storage.BITS["4 + double"] == 4.126953125
    assert (packed.nbytes, q.nbytes, s.nbytes) == storage.buffer_bytes(n)
    # paperclase Parte 4: a 256 x 256 layer holds 1024 blocks
    g = golden("paperclase_storage.txt")
    assert storage.buffer_bytes(256 * 256)[1] == int(g["layer_256x256_blocks"])
