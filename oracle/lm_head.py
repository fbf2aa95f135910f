"""LM head: Q4_0 GEMV, bias, and the greedy token (oracle; test infrastructure only).

Sources:

* realizar 0.8.4 ``src/gpu/adapters/using.rs``, ``GpuModelQ4::forward`` step 5:
  the logits are ``q4_0_gemv_into(lm_head, normed, logits, vocab, hidden)``;
* realizar 0.8.5 ``src/cuda/executor/cached.rs``, ``preload_lm_head_bias``: some
  models carry an output bias of ``vocab`` values that is added to the logits
  after the LM-head GEMV, and ``dispatch_lm_head_and_download`` then brings the
  logits to the host; realizar 0.8.4 ``src/gguf/cuda/clone_layer_weights.rs``
  adds the same bias after the projection (``ops::add_bias``).

The pages stop at the downloaded logits.  The greedy choice made from them is
read here as the index of the largest logit, the smallest such index when
several are equal, so that the choice is unique.  The top-k selection (the k
candidates a sampler draws from) is read the same way: the k largest logits
in descending order, equal values ordered by index, so that it is unique too.
"""
from __future__ import annotations

import numpy as np

from .q4_0 import gemv_q4_0_f32, gemv_q4_0_q8_int


def lm_head_q4_0(blob, x, bias=None, x_format: int = 0):
    """logits = W x (+ bias), float64, and the terms of the pass bound (the
    GEMV's terms plus |bias|).  x_format 0: fp32 x; 1: Q8Blocks."""
    if x_format == 0:
        y, terms = gemv_q4_0_f32(blob, x)
    else:
        y, terms = gemv_q4_0_q8_int(blob, x)
    if bias is not None:
        b = np.asarray(bias, np.float32).astype(np.float64)
        assert b.shape == y.shape and np.all(np.isfinite(b))
        y = y + b
        terms = terms + np.abs(b)
    return y, terms


def argmax_first(values) -> int:
    """Index of the largest value; among equal largest values the smallest
    index.  -0.0 and +0.0 are equal.  Written as a scan so that the tie rule is
    explicit."""
    v = np.asarray(values)
    assert v.ndim == 1 and v.size > 0 and np.all(np.isfinite(v))
    best = 0
    for i in range(1, v.size):
        if v[i] > v[best]:
            best = i
    return best


def topk_first(values, k: int):
    """The k largest values and their indices, largest first; among equal
    values the smaller index first.  -0.0 and +0.0 are equal.  Returns
    (indices int64 [k], values [k]).  Written as a sort on the key
    (-value, index), which is that order exactly."""
    v = np.asarray(values)
    assert v.ndim == 1 and 1 <= k <= v.size and np.all(np.isfinite(v))
    order = sorted(range(v.size), key=lambda i: (-float(v[i]), i))[:k]
    idx = np.asarray(order, np.int64)
    return idx, v[idx]
