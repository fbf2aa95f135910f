"""RMSNorm and the residual add on either side of the GEMVs -- TEST INFRASTRUCTURE ONLY.

realizar 0.8.4 ``src/gpu/adapters/using.rs``, ``rms_norm_inplace``: the mean of
the squares is taken over the n values, the root of (mean + eps) is the RMS,
and every value is multiplied by the reciprocal of the RMS and then by its
weight.  realizar 0.8.5 ``src/cuda/executor/cached.rs``,
``transformer_layer_gpu_true_dp4a``: the pre-attention RMSNorm (step 1) and the
pre-FFN RMSNorm (step 8) feed the Q8_1 quantize; the O projection and the FFN
output are each added to the layer's running hidden state (steps 7 and 10).

The oracle evaluates the definition in float64.  An fp32 implementation
differs from it by rounding only; ``rmsnorm_tolerance`` bounds that difference
from the longest chain of dependent fp32 additions in the sum of squares.
"""
from __future__ import annotations

import numpy as np

_U32 = 2.0 ** -24   # unit roundoff of fp32


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    """x * (1 / sqrt(mean(x^2) + eps)) * gamma per row (the last axis), float64."""
    x = np.asarray(x, np.float64)
    g = np.asarray(gamma, np.float64)
    assert np.all(np.isfinite(x)) and np.all(np.isfinite(g)) and eps >= 0
    ms = np.mean(x * x, axis=-1, keepdims=True)
    scale = 1.0 / np.sqrt(ms + eps)
    return x * scale * g


def rmsnorm_tolerance(normed_ref, chain: int) -> np.ndarray:
    """Bound on |fp32 result - normed_ref| per value.

    ``chain`` is the longest sequence of dependent fp32 additions in the sum of
    squares (for a per-thread loop over k values followed by a tree over T
    threads: k + log2(T)).  Relative error budget, in units of 2**-24: squares
    1, sum ``chain``, division by n 1, adding eps 1 -- of which the square root
    keeps half -- then the reciprocal 1 and the two products 2; doubled."""
    rel = 2.0 * ((chain + 3) / 2.0 + 3.0) * _U32
    return rel * np.abs(np.asarray(normed_ref, np.float64)) + 1e-30


def residual_add(r, y) -> np.ndarray:
    """The running hidden state plus a projection's output, float64."""
    return np.asarray(r, np.float64) + np.asarray(y, np.float64)
