"""fp64 CPU oracle of rotary position embedding (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; it shares nothing with the HIP library. It computes the
reading used for the pages' rope step (the RoFormer rotation of interleaved
pairs, position = row index):
    theta(n, k) = n * base^(-2k / d)
    y[2k]     = x[2k] cos theta - x[2k+1] sin theta
    y[2k + 1] = x[2k] sin theta + x[2k+1] cos theta
in fp64 on the given values.

    rope_fp64(x, base, pos0=0) -> y   (x: [..., N, d], float array or tensor)
"""
from __future__ import annotations

import numpy as np


def rope_fp64(x, base: float, pos0: int = 0) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    X = np.asarray(x, dtype=np.float64)
    N, d = X.shape[-2], X.shape[-1]
    if d % 2:
        raise ValueError("d must be even")
    k = np.arange(d // 2, dtype=np.float64)
    inv_freq = np.power(np.float64(base), -2.0 * k / d)
    theta = (pos0 + np.arange(N, dtype=np.float64))[:, None] * inv_freq[None, :]
    c, s = np.cos(theta), np.sin(theta)
    xe, xo = X[..., 0::2], X[..., 1::2]
    Y = np.empty_like(X)
    Y[..., 0::2] = xe * c - xo * s
    Y[..., 1::2] = xe * s + xo * c
    return Y
