"""Helpers shared by the GPU test modules (no tests here)."""
import sys

import numpy as np
import torch

TOL_BF16 = 1e-2
TOL_F32 = 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def normwise(got, ref):
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / den) if den > 0 else float(np.abs(got).max())
