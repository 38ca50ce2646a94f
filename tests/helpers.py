"""Test helpers: move tensors between torch (GPU side) and numpy (oracle side).

bf16 tensors cross as their raw 16-bit patterns; the oracle widens them
itself.  Nothing here does any arithmetic of the method.
"""
import numpy as np
import torch

import oracle


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit pattern of a tensor as an unsigned numpy array (bit-exact compare)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype == torch.int64:
        return t.numpy()
    raise TypeError(t.dtype)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a bf16/fp32 tensor, widened by the oracle."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(bits(t))
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    raise TypeError(t.dtype)


def relf(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


# tolerances on relative Frobenius error against the fp64 oracle
TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}
