"""Seeded synthetic inputs for the Q4_K / Q4_0 x Q8_1 GEMV path.

This module is shared by the tests, the benchmark and the CPU reference checks.
It holds none of the quantize or dot-product arithmetic: a weight blob is made of
uniform random bytes with fp16 block scales written at their byte offsets, and an
activation is a float32 draw.  Every stream is seeded by ``(config_id, tensor_id)``
so that any two callers asking for the same tensor get the same bytes.

Workload recipe (all synthetic; the pages print no data):

* Q4_K super-block (256 weights, 144 bytes): fp16 ``d`` and ``dmin`` uniform in
  [1e-3, 1e-2]; 12 bytes of packed 6-bit scales/mins; 128 bytes of packed 4-bit
  quants.  The 12 scale bytes carry sixteen 6-bit fields (8 scales, 8 mins) in
  exactly 96 bits, so uniform random bytes give sixteen independent uniform values
  in 0..63.  Uniform qs bytes give uniform nibbles in 0..15.
* Q4_0 block (32 weights, 18 bytes): fp16 ``d`` uniform in [1e-3, 1e-2] and 16
  bytes of uniform nibbles.
* Activations: fp32 cast of float64 N(0, 1) draws.  The attention-projection
  workload normalises such a draw with RMSNorm weights (``norm_weights``: fp32
  cast of N(1, 0.1) draws, eps 1e-5) before quantizing it; the norm itself is
  computed by the caller (the oracle on the CPU side, the library on the GPU).
"""
from __future__ import annotations

import numpy as np

# Byte geometry of the block formats (the generator's own copy).
Q4K_VALUES = 256
Q4K_BYTES = 144
Q4_0_VALUES = 32
Q4_0_BYTES = 18

# tensor ids inside one config
T_ACT = 0
T_W0 = 1      # first weight tensor; further weights are T_W0 + i
T_GAMMA = 9


def rng(config_id: int, tensor_id: int) -> np.random.Generator:
    """Independent, reproducible stream for one tensor of one workload."""
    return np.random.default_rng([int(config_id), int(tensor_id)])


def _f16_bytes(values: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(values.astype(np.float16))
    return v.view(np.uint8).reshape(values.shape + (2,))


def q4k_weights(g: np.random.Generator, out_dim: int, in_dim: int,
                d_range=(1e-3, 1e-2), d_fixed: float | None = None,
                dmin_fixed: float | None = None) -> np.ndarray:
    """Row-major Q4_K blob, shape (out_dim, in_dim // 256, 144), dtype uint8.

    ``d_fixed`` / ``dmin_fixed`` replace the random fp16 scales by a constant
    (used by the integer-exact cases, where d = dmin = 1).
    """
    assert in_dim % Q4K_VALUES == 0 and out_dim >= 0
    nsb = in_dim // Q4K_VALUES
    blob = np.empty((out_dim, nsb, Q4K_BYTES), np.uint8)
    lo, hi = d_range
    d = rng_uniform(g, lo, hi, (out_dim, nsb)) if d_fixed is None else np.full((out_dim, nsb), d_fixed)
    dmin = rng_uniform(g, lo, hi, (out_dim, nsb)) if dmin_fixed is None else np.full((out_dim, nsb), dmin_fixed)
    blob[..., 0:2] = _f16_bytes(d)
    blob[..., 2:4] = _f16_bytes(dmin)
    blob[..., 4:16] = g.integers(0, 256, size=(out_dim, nsb, 12), dtype=np.uint8)
    blob[..., 16:144] = g.integers(0, 256, size=(out_dim, nsb, 128), dtype=np.uint8)
    return blob


def q4_0_weights(g: np.random.Generator, out_dim: int, in_dim: int,
                 d_range=(1e-3, 1e-2), d_fixed: float | None = None) -> np.ndarray:
    """Row-major Q4_0 blob, shape (out_dim, in_dim // 32, 18), dtype uint8."""
    assert in_dim % Q4_0_VALUES == 0 and out_dim >= 0
    nb = in_dim // Q4_0_VALUES
    blob = np.empty((out_dim, nb, Q4_0_BYTES), np.uint8)
    lo, hi = d_range
    d = rng_uniform(g, lo, hi, (out_dim, nb)) if d_fixed is None else np.full((out_dim, nb), d_fixed)
    blob[..., 0:2] = _f16_bytes(d)
    blob[..., 2:18] = g.integers(0, 256, size=(out_dim, nb, 16), dtype=np.uint8)
    return blob


def rng_uniform(g: np.random.Generator, lo: float, hi: float, shape) -> np.ndarray:
    return g.uniform(lo, hi, size=shape)


def activation(g: np.random.Generator, n: int, n_tokens: int | None = None) -> np.ndarray:
    """fp32 N(0,1) activation, shape (n,) or (n_tokens, n)."""
    shape = (n,) if n_tokens is None else (n_tokens, n)
    return g.standard_normal(shape).astype(np.float32)


def norm_weights(g: np.random.Generator, n: int) -> np.ndarray:
    """RMSNorm weights: fp32 cast of N(1, 0.1) draws."""
    return (1.0 + 0.1 * g.standard_normal(n)).astype(np.float32)


def weight_copies(make, count: int):
    """``count`` independent weight blobs from a factory ``make(copy_index)``."""
    return [make(i) for i in range(count)]


# --------------------------------------------------------------------------
# Named workloads.  Sizes are those of the five measured configurations.
# --------------------------------------------------------------------------
WORKLOADS = {
    # Q4_K GEMV 896 -> 896 rows, activation zero-padded to 1024 (4 super-blocks)
    "q4k_896x896": dict(config_id=0, out_dim=896, n=896, in_dim=1024),
    # attention projections of a 7B GQA layer sharing one activation
    "attn_4096": dict(config_id=1, n=4096, in_dim=4096,
                      shapes=(("q", 4096), ("k", 1024), ("v", 1024), ("o", 4096))),
    # SwiGLU FFN 4096 -> 14336 -> 4096
    "ffn_4096_14336": dict(config_id=2, hidden=4096, inter=14336),
    # Q4_0 LM head 151936 x (896 padded to 1024)
    "lm_head_q4_0": dict(config_id=3, out_dim=151936, n=896, in_dim=1024),
    # 8-token Q4_K GEMM 4096 -> 14336
    "q4k_batch8": dict(config_id=4, out_dim=14336, in_dim=4096, n_tokens=8),
    # GELU FFN of a phi-2-sized layer on Q4_0 weights: 2560 -> 10240 -> 2560,
    # with up and down biases
    "gelu_ffn_2560_10240": dict(config_id=5, hidden=2560, inter=10240),
}
