"""Shared helpers of the GPU parity tests."""
import numpy as np


def torch():
    import torch as t
    return t


def dev(a, dtype=None):
    """numpy -> torch CUDA tensor (float32 by default for floats)."""
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        x = x.to(dtype)
    elif x.dtype == t.float64:
        x = x.to(t.float32)
    return x.cuda()


def bf16_exact(a):
    """Round to the nearest bf16 value (RNE) and return it as float32, so the
    oracle sees exactly the operand values the bf16 kernels read."""
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(t.bfloat16).to(t.float32).numpy()


def act(a, precision):
    """Activation tensor on the device: bf16 (precision 1) or fp32 (0)."""
    t = torch()
    return dev(np.asarray(a, np.float32), t.bfloat16 if precision else t.float32)


def host(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def cos(a, b):
    a, b = np.asarray(a, np.float64).ravel(), np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))
