"""Storage arithmetic of the NF4 format (oracle; test infrastructure only).

paperclase "QLoRA", Parte 3, "Bits por parametro": 4 bits per code; a 32-bit
absmax per 64 weights adds 32/64 = 0.5 bit (4.5 total); double quantization
stores the absmax in 8 bits (8/64) plus a 32-bit scale per 64*256 weights,
4 + 8/64 + 32/(64*256) ~ 4.127 bits.  ultralytics "QLoRA", double-quant
bullet: overhead 0.5 -> ~0.127 bits per parameter.
"""

BLOCK = 64
GROUP = 256

BITS = {
    "float32": 32.0,
    "bfloat16": 16.0,
    "4 + absmax": 4.0 + 32.0 / BLOCK,
    "4 + double": 4.0 + 8.0 / BLOCK + 32.0 / (BLOCK * GROUP),
}


def buffer_bytes(numel: int):
    """Bytes of the three NF4 buffers for a tensor of numel weights
    (numel % 64 == 0): packed codes, 8-bit absmax codes, fp32 group scales."""
    if numel % BLOCK:
        raise ValueError("numel must be a multiple of 64")
    blocks = numel // BLOCK
    groups = (blocks + GROUP - 1) // GROUP
    return numel // 2, blocks, 4 * groups


def gigabytes(n_params: float, bits_per_param: float) -> float:
    """Decimal GB (8e9 bits per GB, as the lesson's table)."""
    return n_params * bits_per_param / 8e9
