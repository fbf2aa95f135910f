"""Q4_0 GEMV, fp32 or Q8_1 activation (oracle; test infrastructure only).

Source: realizar 0.8.4 ``src/gpu/adapters/using.rs``, ``GpuModelQ4::forward``
step 5 "LM head projection (GPU, Q4_0)": ``q4_0_gemv_into(lm_head, normed, logits,
vocab_size, hidden_dim)`` -- a Q4_0 weight matrix times the fp32 output of the
final RMSNorm; ``forward_layer`` and ``ffn_swiglu_gpu`` use the same call for
every Q4_0 projection.

Block reading (GGML Q4_0), 18 bytes: fp16 ``d`` then ``qs[16]``; value ``l < 16``
is the low nibble of ``qs[l]``, value ``16 + l`` the high nibble; the weight is
``(q - 8) * d``.

* fp32 activation: ``y[r] = sum_k w[r, k] * x[k]`` in float64; ``terms`` is
  ``sum_k |w x|``.
* Q8_1 activation (the integer variant): ``isum_b = sum_l (q - 8) * q8`` exactly,
  ``y[r] = sum_b d_b * d_x,b * isum_b``; ``terms`` is ``sum_b |d d_x isum|``.
"""
from __future__ import annotations

import numpy as np

from .q8_1 import Q8Blocks, QK8_1

Q4_0_BLOCK_BYTES = 18
ROW_CHUNK = 8192


def q4_0_fields(blob: np.ndarray):
    """(rows, nb, 18) blob -> d float64 (rows, nb), q int64 (rows, nb, 32) in 0..15."""
    blob = np.asarray(blob, np.uint8)
    assert blob.ndim == 3 and blob.shape[2] == Q4_0_BLOCK_BYTES
    d = np.ascontiguousarray(blob[..., 0:2]).view('<f2')[..., 0].astype(np.float64)
    qs = blob[..., 2:18].astype(np.int64)
    q = np.empty(blob.shape[:2] + (32,), np.int64)
    q[..., 0:16] = qs & 15
    q[..., 16:32] = qs >> 4
    return d, q


def dequantize_q4_0(blob: np.ndarray) -> np.ndarray:
    d, q = q4_0_fields(blob)
    return ((q - 8) * d[..., None]).reshape(blob.shape[0], -1)


def gemv_q4_0_f32(blob: np.ndarray, x: np.ndarray):
    """fp32 activation.  Returns (y, terms) float64."""
    x = np.asarray(x, np.float32).astype(np.float64)
    if x.shape[0] != blob.shape[1] * QK8_1:
        raise ValueError("activation length must equal the padded in_dim")
    rows = blob.shape[0]
    y = np.empty(rows, np.float64)
    terms = np.empty(rows, np.float64)
    ax = np.abs(x)
    for r0 in range(0, rows, ROW_CHUNK):
        w = dequantize_q4_0(blob[r0:r0 + ROW_CHUNK])
        y[r0:r0 + ROW_CHUNK] = w @ x
        terms[r0:r0 + ROW_CHUNK] = np.abs(w) @ ax
    return y, terms


def gemv_q4_0_q8_int(blob: np.ndarray, x: Q8Blocks):
    """Q8_1 activation, integer form.  Returns (y, terms) float64."""
    nb = blob.shape[1]
    if x.n_blocks != nb:
        raise ValueError("activation block count must equal the weight block count")
    xd = x.d.astype(np.float64)
    xq = x.q.astype(np.int64)
    rows = blob.shape[0]
    y = np.empty(rows, np.float64)
    terms = np.empty(rows, np.float64)
    for r0 in range(0, rows, ROW_CHUNK):
        d, q = q4_0_fields(blob[r0:r0 + ROW_CHUNK])
        isum = np.einsum('rbl,bl->rb', q - 8, xq)     # exact integers
        t = d * xd[None, :] * isum
        y[r0:r0 + ROW_CHUNK] = t.sum(axis=1)
        terms[r0:r0 + ROW_CHUNK] = np.abs(t).sum(axis=1)
    return y, terms
