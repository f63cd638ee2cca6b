"""Helpers shared by the GPU tests: torch <-> numpy bf16 bit patterns."""
import numpy as np
import torch


def to_dev_bf16(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rel_frobenius(a_bits: np.ndarray, b_bits: np.ndarray) -> float:
    import oracle
    return oracle.nrmse(oracle.bf16_bits_to_f32(a_bits), oracle.bf16_bits_to_f32(b_bits))


def same_bf16(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Elementwise equality of bf16 values with +0 and -0 taken as equal."""
    a = a_bits.copy()
    b = b_bits.copy()
    a[a == 0x8000] = 0
    b[b == 0x8000] = 0
    return a == b
