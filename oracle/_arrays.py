"""Exact upcast of inputs to float64 numpy arrays (bf16 and f32 values are
representable in fp64, so the conversion changes no value)."""
import numpy as np


def f64(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # a CPU torch tensor (bf16 has no numpy dtype)
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)
