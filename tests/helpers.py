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


def act_dtype(precision):
    """Storage type of activations: fp32 (precision 0), bf16 (1), fp16 (2)."""
    t = torch()
    return {0: t.float32, 1: t.bfloat16, 2: t.float16}[precision]


def exact(a, precision):
    """a rounded (RNE) to the activation type of `precision`, as float32, so
    the oracle sees exactly the operand values the kernels read."""
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return x.to(act_dtype(precision)).to(t.float32).numpy()


def act(a, precision):
    """Activation tensor on the device in the type of `precision`."""
    return dev(np.asarray(a, np.float32), act_dtype(precision))


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
