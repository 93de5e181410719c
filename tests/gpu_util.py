"""Helpers shared by the GPU parity tests: device upload and error metrics."""
import sys

import numpy as np


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits):
    """uint16 bf16 bit patterns -> a torch.bfloat16 device tensor."""
    import torch
    return dev(bits.astype(np.uint16)).view(torch.bfloat16)


def to_f64(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def rel_l2(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def max_rel(got, ref):
    """max |got - ref| / max |ref| (normwise, stable near zeros)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))


# tolerances fixed by the accuracy targets of this layer: fp32 outputs within
# a relative L2 error of 1e-3, bf16 outputs within a normwise max relative
# error of 2e-2
TOL_F32_REL_L2 = 1e-3
TOL_BF16_MAX_REL = 2e-2
