"""Q8_1 activation quantization (oracle; test infrastructure only).

Source: realizar 0.8.5 ``src/cuda/executor/cached.rs``,
``transformer_layer_gpu_true_dp4a`` step 2 (the normed fp32 activation is
quantized to Q8_1 once and shared by Q/K/V) and step 5 (the attention output is
quantized the same way before the O projection).  The pages name the format but
do not print it; the reading used here:

* a block holds 32 consecutive values;
* ``amax = max |x|`` over the block, ``d = fp32(amax) / fp32(127)`` (one IEEE
  fp32 division, correctly rounded);
* ``q = round_half_even(fp32(x / d))`` -- again a true fp32 division -- clamped to
  [-127, 127] (it binds only where d is a
  denormal rounded down, e.g. amax = 190 * 2^-149 with d = 2^-149);
* an all-zero block has ``d = 0``, ``q = 0``, ``s = 0``; so has a block whose
  ``d`` rounds to 0 (a denormal ``amax`` of at most 63 * 2^-149), where the
  quotients ``x / d`` have no value and the pages say nothing;
* ``s = fp32(d * fp32(sum q))`` with the sum taken exactly in integers;
* stored as 40 bytes: fp32 ``d``, fp32 ``s`` (little endian), then 32 int8 codes.
  Blocks are contiguous; the tokens of a batch follow each other.

Values past the logical length ``n`` (up to the padded length) are +0.0, which is
the zero padding of ``pad_and_upload_input`` in realizar 0.8.5
``src/cuda/executor/layers/forward_utils.rs``.

Every decision that produces a code is taken in fp32, the precision the values
are stored in; nothing here is vectorised across blocks.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

QK8_1 = 32
Q8_1_BLOCK_BYTES = 40
_F127 = np.float32(127.0)


@dataclass
class Q8Blocks:
    """Decoded Q8_1 blocks: ``d`` and ``s`` float32 (..., nb), ``q`` int8 (..., nb, 32)."""
    d: np.ndarray
    s: np.ndarray
    q: np.ndarray

    @property
    def n_blocks(self) -> int:
        return self.d.shape[-1]

    def token(self, t: int) -> "Q8Blocks":
        """Blocks of token ``t`` of a batched (n_tokens, nb) set."""
        return Q8Blocks(self.d[t], self.s[t], self.q[t])


def _quantize_block(xb: np.ndarray):
    """One 32-value block; ``xb`` is float32."""
    amax = np.float32(0.0)
    for v in xb:                       # exact: max of absolute values
        a = np.float32(abs(v))
        if a > amax:
            amax = a
    d = np.float32(amax / _F127)       # fp32 / fp32 -> correctly rounded fp32
    if d == np.float32(0.0):
        # amax == 0, or a denormal amax of at most 63 * 2^-149 for which
        # amax / 127 rounds to 0: x / d has no value, so the block is zeros
        return np.float32(0.0), np.float32(0.0), np.zeros(QK8_1, np.int8)
    q = np.empty(QK8_1, np.int8)
    total = 0
    for i, v in enumerate(xb):
        r = np.float32(v / d)          # fp32 division, not a reciprocal multiply
        c = int(np.rint(r))            # numpy rint rounds half to even
        c = max(-127, min(127, c))
        q[i] = c
        total += c
    s = np.float32(d * np.float32(total))
    return d, s, q


def quantize_q8_1(x, n_padded: int | None = None) -> Q8Blocks:
    """Quantize fp32 ``x`` of shape (n,) or (n_tokens, n) to Q8_1 blocks.

    ``n_padded`` (a multiple of 32, >= n) is the padded length; the tail is zero.
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("Q8_1 input must be float32")
    single = x.ndim == 1
    x2 = x[None, :] if single else x
    n_tok, n = x2.shape
    if n_padded is None:
        n_padded = -(-n // QK8_1) * QK8_1
    if n_padded % QK8_1 or n > n_padded:
        raise ValueError("n_padded must be a multiple of 32 and >= n")
    if not np.all(np.isfinite(x2)):
        raise ValueError("non-finite activations are outside the Q8_1 contract")
    nb = n_padded // QK8_1
    d = np.zeros((n_tok, nb), np.float32)
    s = np.zeros((n_tok, nb), np.float32)
    q = np.zeros((n_tok, nb, QK8_1), np.int8)
    for t in range(n_tok):
        xp = np.zeros(n_padded, np.float32)
        xp[:n] = x2[t]
        for b in range(nb):
            d[t, b], s[t, b], q[t, b] = _quantize_block(xp[b * QK8_1:(b + 1) * QK8_1])
    if single:
        return Q8Blocks(d[0], s[0], q[0])
    return Q8Blocks(d, s, q)


def q8_1_to_bytes(blocks: Q8Blocks) -> np.ndarray:
    """Serialise to the 40-byte block layout; returns uint8 (..., nb, 40)."""
    shape = blocks.d.shape
    out = np.empty(shape + (Q8_1_BLOCK_BYTES,), np.uint8)
    out[..., 0:4] = blocks.d.astype('<f4').reshape(shape + (1,)).view(np.uint8)
    out[..., 4:8] = blocks.s.astype('<f4').reshape(shape + (1,)).view(np.uint8)
    out[..., 8:40] = blocks.q.view(np.uint8)
    return out


def q8_1_from_bytes(raw: np.ndarray) -> Q8Blocks:
    """Parse uint8 (..., nb, 40) blocks (used for hand-built inputs)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    d = raw[..., 0:4].copy().view('<f4')[..., 0].astype(np.float32)
    s = raw[..., 4:8].copy().view('<f4')[..., 0].astype(np.float32)
    q = raw[..., 8:40].copy().view(np.int8)
    return Q8Blocks(d, s, q)


def dequantize_q8_1(blocks: Q8Blocks) -> np.ndarray:
    """x_hat = d * q in float64, shape (..., nb * 32)."""
    xh = blocks.d.astype(np.float64)[..., None] * blocks.q.astype(np.float64)
    return xh.reshape(xh.shape[:-2] + (-1,))
