"""Q4_K weights x Q8_1 activation GEMV (oracle; test infrastructure only).

Source: realizar 0.8.5 ``src/cuda/executor/cached.rs``,
``transformer_layer_gpu_true_dp4a`` steps 3 and 6 (Q/K/V/O projections as
"Q4K x Q8 integer dot product"; the doc comment says every GEMV on this path uses
integer arithmetic, four int8 multiply-adds per dot instruction), and
``src/cuda/executor/layers/forward_utils.rs``, ``pad_and_upload_input`` (256-value
super-blocks; the activation is zero-padded to a multiple of 256).  Argument
order is (out_dim, in_dim) as in the ``q4k_q8_gemv_async`` calls.

Super-block reading (GGML Q4_K, type id 12 as tested in
``src/gguf/cuda/clone_layer_weights.rs``, ``cuda_layer_ffn``), 144 bytes:

* bytes 0-1 ``d`` fp16, bytes 2-3 ``dmin`` fp16, bytes 4-15 ``scales[12]``,
  bytes 16-143 ``qs[128]``;
* eight sub-blocks of 32 values; 6-bit scale ``sc_j`` and min ``m_j``:
  j < 4:  sc_j = scales[j] & 63,  m_j = scales[j+4] & 63;
  j >= 4: sc_j = (scales[j+4] & 15) | ((scales[j-4] >> 6) << 4),
          m_j  = (scales[j+4] >> 4) | ((scales[j] >> 6) << 4);
* value ``32 j + l`` of the super-block: chunk ``c = j // 2`` holds bytes
  ``qs[32 c : 32 c + 32]``; even j takes the low nibble of ``qs[32 c + l]``, odd
  j the high nibble;
* dequantized weight ``w = d * sc_j * q - dmin * m_j``.

Two statements of the product, both in float64:

* definition: ``y[r] = sum_k w[r, k] * x_hat[k]`` with ``x_hat = d_x * q_x``;
* integer form: ``isum_j = sum_l q4 * q8`` exactly (int64), then
  ``y[r] = sum_{b, j} d * sc_j * d_x * isum_j - dmin * m_j * s_j``.

They differ only by the fp32 rounding of ``s_j``.  ``gemv_q4k_f32`` states the
product with an fp32 activation (no Q8_1), the definition again.  ``terms`` is
``sum |d sc d_x isum| + |dmin m s|``, the summands an fp32 kernel rounds; the
pass bound of an fp32 result is ``1e-5 * terms + 1e-6``.
"""
from __future__ import annotations

import numpy as np

from .q8_1 import Q8Blocks, QK8_1

QK_K = 256
Q4K_BLOCK_BYTES = 144
ROW_CHUNK = 2048


def _f16(raw2: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(raw2).view('<f2')[..., 0].astype(np.float64)


def q4k_unpack_scales(scales: np.ndarray):
    """``scales`` uint8 (..., 12) -> (sc, m), each int64 (..., 8)."""
    s = scales.astype(np.int64)
    sc = np.empty(s.shape[:-1] + (8,), np.int64)
    m = np.empty(s.shape[:-1] + (8,), np.int64)
    for j in range(4):
        sc[..., j] = s[..., j] & 63
        m[..., j] = s[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j - 4] >> 6) << 4)
        m[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return sc, m


def q4k_fields(blob: np.ndarray):
    """Decode a (rows, nsb, 144) blob into d, dmin (rows, nsb) float64,
    sc, m (rows, nsb, 8) int64 and the quants q (rows, nsb, 8, 32) int64."""
    blob = np.asarray(blob, np.uint8)
    assert blob.ndim == 3 and blob.shape[2] == Q4K_BLOCK_BYTES
    d = _f16(blob[..., 0:2])
    dmin = _f16(blob[..., 2:4])
    sc, m = q4k_unpack_scales(blob[..., 4:16])
    qs = blob[..., 16:144].astype(np.int64)
    q = np.empty(blob.shape[:2] + (8, 32), np.int64)
    for j in range(8):
        chunk = qs[..., 32 * (j // 2): 32 * (j // 2) + 32]
        q[..., j, :] = (chunk & 15) if j % 2 == 0 else (chunk >> 4)
    return d, dmin, sc, m, q


def dequantize_q4k(blob: np.ndarray) -> np.ndarray:
    """Dequantized weights, float64 (rows, nsb * 256)."""
    d, dmin, sc, m, q = q4k_fields(blob)
    w = (d[..., None, None] * sc[..., None] * q) - (dmin[..., None, None] * m[..., None])
    return w.reshape(blob.shape[0], -1)


def _x_parts(x: Q8Blocks, nsb: int):
    if x.n_blocks != nsb * 8:
        raise ValueError("activation has %d Q8_1 blocks, weights need %d" % (x.n_blocks, nsb * 8))
    xd = x.d.astype(np.float64).reshape(nsb, 8)
    xs = x.s.astype(np.float64).reshape(nsb, 8)
    xq = x.q.astype(np.int64).reshape(nsb, 8, QK8_1)
    return xd, xs, xq


def gemv_q4k_q8_def(blob: np.ndarray, x: Q8Blocks) -> np.ndarray:
    """Definition: dequantized weights times dequantized activation, float64."""
    from .q8_1 import dequantize_q8_1
    xh = dequantize_q8_1(x)
    y = np.empty(blob.shape[0], np.float64)
    for r0 in range(0, blob.shape[0], ROW_CHUNK):
        y[r0:r0 + ROW_CHUNK] = dequantize_q4k(blob[r0:r0 + ROW_CHUNK]) @ xh
    return y


def gemv_q4k_f32(blob: np.ndarray, x: np.ndarray):
    """fp32 activation (realizar 0.8.5 ``src/cuda/executor/cached.rs``,
    ``transformer_layer_gpu_cached`` steps 2 and 4: ``q4k_gemv_cached_async`` /
    ``tiled_q4k_gemv_cached_async`` over the fp32 normed activation, no Q8_1).

    Returns (y, terms) float64 (rows,).  ``y`` is the definition
    ``sum_k w[r, k] * x[k]``.  ``terms`` counts the summands of the factored
    form a kernel evaluates per sub-block, ``d * sc_j * sum_l q_l x_l -
    dmin * m_j * sum_l x_l``: ``sum_{b,j} d sc_j sum_l |q_l x_l| + dmin m_j
    sum_l |x_l|``.  It is never below ``sum_k |w[r, k] x[k]|``, so a direct
    evaluation of the definition meets the same bound."""
    x = np.asarray(x, np.float32).astype(np.float64)
    nsb = blob.shape[1]
    if x.shape[0] != nsb * QK_K:
        raise ValueError("activation length must equal the padded in_dim")
    assert np.all(np.isfinite(x))
    rows = blob.shape[0]
    y = np.empty(rows, np.float64)
    terms = np.empty(rows, np.float64)
    ax = np.abs(x).reshape(nsb, 8, QK8_1)
    ax_sum = ax.sum(axis=2)                                     # (nsb, 8)
    for r0 in range(0, rows, ROW_CHUNK):
        part = blob[r0:r0 + ROW_CHUNK]
        y[r0:r0 + ROW_CHUNK] = dequantize_q4k(part) @ x
        d, dmin, sc, m, q = q4k_fields(part)
        qx = np.einsum('rbjl,bjl->rbj', q, ax)                  # sum_l |q_l x_l| (q >= 0)
        t = d[..., None] * sc * qx + dmin[..., None] * m * ax_sum[None]
        terms[r0:r0 + ROW_CHUNK] = t.sum(axis=(1, 2))
    return y, terms


def gemv_q4k_q8_int(blob: np.ndarray, x: Q8Blocks, return_isum: bool = False):
    """Integer form.  Returns (y, terms) float64 (rows,), plus the exact
    sub-block sums isum int64 (rows, nsb, 8) when ``return_isum``."""
    nsb = blob.shape[1]
    xd, xs, xq = _x_parts(x, nsb)
    rows = blob.shape[0]
    y = np.empty(rows, np.float64)
    terms = np.empty(rows, np.float64)
    isums = np.empty((rows, nsb, 8), np.int64) if return_isum else None
    for r0 in range(0, rows, ROW_CHUNK):
        d, dmin, sc, m, q = q4k_fields(blob[r0:r0 + ROW_CHUNK])
        isum = np.einsum('rbjl,bjl->rbj', q, xq)              # exact integers
        scale_part = d[..., None] * sc * xd[None] * isum       # d sc d_x isum
        min_part = dmin[..., None] * m * xs[None]              # dmin m s
        y[r0:r0 + ROW_CHUNK] = (scale_part - min_part).sum(axis=(1, 2))
        terms[r0:r0 + ROW_CHUNK] = (np.abs(scale_part) + np.abs(min_part)).sum(axis=(1, 2))
        if return_isum:
            isums[r0:r0 + ROW_CHUNK] = isum
    if return_isum:
        return y, terms, isums
    return y, terms
