"""SwiGLU FFN on the integer GEMV path (oracle; test infrastructure only).

Sources:

* realizar 0.8.5 ``src/cuda/executor/cached.rs``, ``transformer_layer_gpu_true_dp4a``
  step 9: the FFN runs as ``fused_ffn_swiglu_gpu_true_dp4a(normed, gate, up, down,
  hidden_dim, intermediate_dim)`` -- gate and up are (intermediate x hidden), down is
  (hidden x intermediate);
* realizar 0.8.4 ``src/gguf/cuda/clone_layer_weights.rs``, ``cuda_swiglu_ffn``: SiLU
  on the gate projection, then an elementwise product with the up projection,
  then the down projection;
* realizar 0.8.4 ``src/gpu/adapters/using.rs``, ``ffn_swiglu_gpu``: the same order
  (gate GEMV, up GEMV, fused SwiGLU, down GEMV).

On the integer path the down projection takes a Q8_1 activation, so ``h`` is
requantized exactly like the attention output before the O projection (step 5
of ``transformer_layer_gpu_true_dp4a``).  Reading: ``silu(g) = g / (1 + exp(-g))``.

The chain here is float64 for the projections and SiLU; ``h`` is rounded to fp32
once (its storage type) before it is requantized.
"""
from __future__ import annotations

import numpy as np

from .q4k import gemv_q4k_f32, gemv_q4k_q8_int
from .q8_1 import quantize_q8_1
from .tolerance import gemv_tolerance


def silu(g):
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def silu_grad(g):
    """d silu / d g = sigma(g) * (1 + g * (1 - sigma(g)))."""
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    return sig * (1.0 + g * (1.0 - sig))


# sup |silu'| and sup |silu''| over the reals (silu'' peaks at g = 0 with 1/2),
# and the Lipschitz constant of A(g) = 2 - g tanh(g/2), the second factor of
# silu'' = sigma'(g) A(g) (sup |A'| = 1.19968, near g = -2.4); the pins check
# them on a dense grid.
SILU_GRAD_MAX = 1.0999
SILU_CURV_MAX = 0.5
SILU_A_LIP = 1.2


def _sigma_prime(g):
    """sigma'(g) = e^-|g| / (1 + e^-|g|)^2, without cancellation for large |g|."""
    e = np.exp(-np.abs(np.asarray(g, np.float64)))
    return e / (1.0 + e) ** 2


def silu_curv(g):
    """d^2 silu / d g^2 = sigma'(g) * (2 - g tanh(g/2))  (1 - 2 sigma(g) = -tanh(g/2))."""
    g = np.asarray(g, np.float64)
    return _sigma_prime(g) * (2.0 - g * np.tanh(0.5 * g))


def silu_curv_bound(g, r):
    """An upper bound on |silu''| over [g - r, g + r]: log sigma' has slope at
    most 1 in magnitude and A(g) = 2 - g tanh(g/2) is SILU_A_LIP-Lipschitz, so
    |silu''(xi)| <= sigma'(g) e^r (|A(g)| + SILU_A_LIP r)."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    return _sigma_prime(g) * np.exp(r) * (np.abs(2.0 - g * np.tanh(0.5 * g)) + SILU_A_LIP * r)


def swiglu(g, u):
    """h = silu(g) * u, float64."""
    return silu(g) * np.asarray(u, np.float64)


def h_tolerance(g, u, tol_g, tol_u, h_ref):
    """Bound on |h_kernel - h_ref| when the kernel's g and u are within
    ``tol_g`` / ``tol_u`` of the oracle's and h is formed in fp32.

    h = silu(g) * u is linear in u, so its change under (dg, du) is exactly
      silu'(g) u dg + silu(g) du + silu'(g) dg du + silu''(xi) dg^2 (u + du) / 2
    for some xi within dg of g.  Each term is bounded here, the curvature by
    ``silu_curv_bound`` over [g - tol_g, g + tol_g], and a fp32 budget of 8 ulp
    for exp, the division and the two products is added (device exp is not
    bit-reproducible on the host).
    """
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    tol_g = np.asarray(tol_g, np.float64)
    tol_u = np.asarray(tol_u, np.float64)
    d1 = np.abs(silu_grad(g))
    first = d1 * np.abs(u) * tol_g + np.abs(silu(g)) * tol_u
    second = d1 * tol_g * tol_u + 0.5 * silu_curv_bound(g, tol_g) * tol_g ** 2 * (np.abs(u) + tol_u)
    rounding = 8.0 * 2.0 ** -24 * np.abs(h_ref) + 1e-6
    return first + second + rounding


def ffn_swiglu_q4k(w_gate, w_up, w_down, x_q8):
    """The whole chain from a Q8_1 activation.  Returns a dict of every stage:
    g, u (+ terms), h (float64), h32 (fp32), h_q8 (Q8Blocks), y (+ terms)."""
    g, tg = gemv_q4k_q8_int(w_gate, x_q8)
    u, tu = gemv_q4k_q8_int(w_up, x_q8)
    h = swiglu(g, u)
    h32 = h.astype(np.float32)
    h_q8 = quantize_q8_1(h32)
    y, ty = gemv_q4k_q8_int(w_down, h_q8)
    return dict(g=g, g_terms=tg, u=u, u_terms=tu, h=h, h32=h32, h_q8=h_q8,
                y=y, y_terms=ty,
                tol_g=gemv_tolerance(tg), tol_u=gemv_tolerance(tu))


def ffn_swiglu_q4k_f32(w_gate, w_up, w_down, x):
    """The chain on the fp32-activation path (realizar 0.8.5
    ``src/cuda/executor/cached.rs``, ``transformer_layer_gpu_cached`` step 7,
    ``fused_ffn_swiglu_gpu``; realizar 0.8.4 ``src/gpu/adapters/using.rs``,
    ``ffn_swiglu_gpu``: gate and up GEMVs of the fp32 input, the fused SwiGLU,
    then the down GEMV of its fp32 output).  No Q8_1 anywhere: h is rounded to
    fp32 (its storage type) and is the down projection's activation.
    Returns g, u (+ terms), h (float64), h32 (fp32), y (+ terms)."""
    g, tg = gemv_q4k_f32(w_gate, x)
    u, tu = gemv_q4k_f32(w_up, x)
    h = swiglu(g, u)
    h32 = h.astype(np.float32)
    y, ty = gemv_q4k_f32(w_down, h32)
    return dict(g=g, g_terms=tg, u=u, u_terms=tu, h=h, h32=h32, y=y, y_terms=ty,
                tol_g=gemv_tolerance(tg), tol_u=gemv_tolerance(tu))
