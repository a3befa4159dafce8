"""Seeded synthetic inputs for tests and benchmarks.

This module only draws random numbers and converts them to the storage types
the library takes (fp32, and bf16 by round-to-nearest-even through torch's
CPU conversion).  It holds none of the quantization or linear-layer
arithmetic, and imports neither the oracle nor the library.

Recipe (stands in for trained Llama/Gemma projections, which are not
available): numpy Generator(PCG64(seed)) with
    seed = 1000 * workload + 10 * projection + tensor
    tensor ids: W = 0, X = 1, A = 2, B = 3, dY = 4
draws standard_normal in fp32, scaled by the standard deviation:
    W ~ N(0, 0.02)       (the pages' law for pretrained weights)
    X, dY ~ N(0, 1)
    A ~ N(0, 1/in)       B ~ N(0, 0.01)
LoRA dropout keep masks (tensor id 5): element (t, k) kept when a uniform
draw in [0, 1) is >= p, packed 8 elements per byte, element k in bit k % 8
of byte k / 8 of its row.
"""

from dataclasses import dataclass

import numpy as np
import torch

W_STD = 0.02
B_STD = 0.01
TENSOR_ID = {"W": 0, "X": 1, "A": 2, "B": 3, "dY": 4, "keep": 5}


def seed_for(workload: int, projection: int, tensor: str) -> int:
    return 1000 * workload + 10 * projection + TENSOR_ID[tensor]


def normal_f32(seed: int, shape, std: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even, torch CPU) as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


@dataclass(frozen=True)
class Projection:
    name: str
    out_features: int
    in_features: int


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    projections: tuple
    tokens: tuple          # token counts exercised
    r: int
    alpha: float
    backward: bool


WORKLOADS = {
    1: Workload(1, "single 256x256 linear, T=16, r=8", (Projection("linear", 256, 256),),
                (16,), 8, 16.0, True),
    2: Workload(2, "8B q_proj 4096x4096 decode, T=1 and T=16, r=16",
                (Projection("q_proj", 4096, 4096),), (1, 16), 16, 32.0, False),
    3: Workload(3, "8B MLP gate/up 4096->14336, down 14336->4096, T=4096, r=64",
                (Projection("gate", 14336, 4096), Projection("up", 14336, 4096),
                 Projection("down", 4096, 14336)), (4096,), 64, 128.0, True),
    4: Workload(4, "8B attention q,o 4096x4096, k,v 4096->1024, T=8192, r=16",
                (Projection("q", 4096, 4096), Projection("k", 1024, 4096),
                 Projection("v", 1024, 4096), Projection("o", 4096, 4096)),
                (8192,), 16, 32.0, True),
    5: Workload(5, "70B MLP gate/up 8192->28672, down 28672->8192, T=4096, r=64",
                (Projection("gate", 28672, 8192), Projection("up", 28672, 8192),
                 Projection("down", 8192, 28672)), (4096,), 64, 16.0, True),
}

#: flat fp32 tensor quantized on its own (70B-scale quantize workload)
FLAT_QUANTIZE_NUMEL = 1 << 30
FLAT_QUANTIZE_SEED = 5000


def weight(workload: int, projection: int, out_f: int, in_f: int) -> np.ndarray:
    return normal_f32(seed_for(workload, projection, "W"), (out_f, in_f), W_STD)


def activations(workload: int, projection: int, T: int, in_f: int, tensor: str = "X") -> np.ndarray:
    """X [T, in] (or dY [T, out] with tensor='dY'), bf16 bits."""
    return bf16_bits(normal_f32(seed_for(workload, projection, tensor), (T, in_f), 1.0))


def lora_A(workload: int, projection: int, r: int, in_f: int) -> np.ndarray:
    return bf16_bits(normal_f32(seed_for(workload, projection, "A"), (r, in_f), 1.0 / in_f))


def lora_B(workload: int, projection: int, out_f: int, r: int) -> np.ndarray:
    return bf16_bits(normal_f32(seed_for(workload, projection, "B"), (out_f, r), B_STD))


def keep_mask(seed: int, T: int, in_f: int, p: float) -> np.ndarray:
    """Dropout keep mask [T, in/8] uint8 (bit k % 8 of byte k / 8 = element k
    kept), each element kept with probability 1 - p."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kept = rng.random((T, in_f)) >= p
    return np.packbits(kept, axis=1, bitorder="little")
