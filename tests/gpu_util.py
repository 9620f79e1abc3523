"""Helpers for the GPU parity tests (no arithmetic of the method here)."""
import numpy as np
import torch

import memory_bound_weight_amd as L

BOUND = 1e-3   # |y_gpu - y| <= BOUND * sum_k |W[n][k] x[m][k]| per output


def worst_ratio(y_gpu, Y, B):
    """max over outputs of |y_gpu - Y| / (BOUND * B); outputs with B == 0 must be exact."""
    y = y_gpu.detach().cpu().numpy().astype(np.float64) if isinstance(y_gpu, torch.Tensor) else y_gpu
    d = np.abs(y - Y)
    zero = B == 0
    if np.any(d[zero] != 0):
        return np.inf
    if np.all(zero):
        return 0.0
    return float(np.max(d[~zero] / (BOUND * B[~zero])))


def assert_within_bound(y_gpu, Y, B, what=""):
    r = worst_ratio(y_gpu, Y, B)
    assert np.isfinite(r) and r <= 1.0, "%s: worst |err|/bound = %.4g" % (what, r)
    return r


class pinned:
    """Pin one candidate configuration for a shape; restore the table after."""

    def __init__(self, kind, M, N, K, cfg):
        self.args = (kind, M, N, K)
        self.cfg = cfg

    def __enter__(self):
        L.lin_set_config(*self.args, self.cfg)
        return self

    def __exit__(self, *exc):
        L.lin_set_config(*self.args, None)
        return False


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
