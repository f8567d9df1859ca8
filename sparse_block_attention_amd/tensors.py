"""Moving bf16-valued numpy arrays to and from device memory (torch as plumbing)."""
from __future__ import annotations

import numpy as np
import torch

from .synth import bf16_bits


def to_device_bf16(x: np.ndarray, device="cuda") -> torch.Tensor:
    """float32 array of bf16-representable values -> contiguous bf16 device tensor."""
    bits = np.ascontiguousarray(bf16_bits(x)).view(np.int16)
    return torch.from_numpy(bits).view(torch.bfloat16).to(device)


def to_device_f32(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def from_device_bf16(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> float32 numpy array holding the same values."""
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
