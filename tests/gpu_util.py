"""Shared helpers for the GPU parity tests (moves seeded host inputs to the
device and back; no arithmetic of the method)."""

import sys

import numpy as np
import pytest
import torch

TOL = 2e-3  # relative Frobenius bound on Y, dX, dA, dB


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    if not name.startswith("gfx950"):
        pytest.skip(f"device is {name}, not gfx950")
    import bit_nf4_quantized_20_amd as q  # raises if the library is not built
    return q


def banner(msg: str):
    """Names the case on stdout before GPU work, flushed."""
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.cuda().view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()
