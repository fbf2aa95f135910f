"""GELU FFN on Q4_0 weights and fp32 activations (oracle; test infrastructure only).

Sources:

* realizar 0.8.4 ``src/gpu/adapters/using.rs``, ``ffn_standard_gpu``: the up
  projection ``q4_0_gemv_into(up, input, up_gpu, intermediate, hidden)`` over the
  fp32 input, GELU applied in place, then the down projection of the GELU output
  (``q4_0_gemv_into(down, up_gpu, down_gpu, hidden, intermediate)``);
* realizar 0.8.4 ``src/gguf/cuda/clone_layer_weights.rs``, ``cuda_gelu_ffn`` (the
  path for phi-2-style models): the same chain, with an optional bias added to
  the up projection before GELU and to the down projection after it.

Reading: ``ops::gelu`` is named but not printed.  The models the pages route
here (phi-2 style) use the tanh form of GELU,
``gelu(u) = 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))``, which is taken
here.  It equals ``u * sigmoid(2 sqrt(2/pi) (u + 0.044715 u^3))``.  The chain is
float64; h is rounded to fp32 (its storage type) before the down projection.
"""
from __future__ import annotations

import numpy as np

from .q4_0 import gemv_q4_0_f32
from .tolerance import gemv_tolerance

GELU_K = np.sqrt(2.0 / np.pi)
GELU_C = 0.044715
# sup |gelu'| and sup |gelu''| of the tanh form over the reals (reached near
# u = 1.42 and at u = 0; the pins check them on a dense grid).
GELU_GRAD_MAX = 1.13
GELU_CURV_MAX = 0.80


def gelu(u):
    u = np.asarray(u, np.float64)
    return 0.5 * u * (1.0 + np.tanh(GELU_K * (u + GELU_C * u ** 3)))


def gelu_grad(u):
    """d gelu / d u of the tanh form."""
    u = np.asarray(u, np.float64)
    t = np.tanh(GELU_K * (u + GELU_C * u ** 3))
    return 0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * GELU_K * (1.0 + 3.0 * GELU_C * u * u)


def gelu_h_tolerance(u, tol_u, h_ref):
    """Bound on |h_kernel - h_ref| when the kernel's pre-activation is within
    tol_u of the oracle's and gelu is evaluated in fp32: first- and second-order
    propagation plus 8 ulp for exp, the division and the products (the device
    exp is not bit-reproducible on the host)."""
    u = np.asarray(u, np.float64)
    first = np.abs(gelu_grad(u)) * tol_u
    second = 0.5 * GELU_CURV_MAX * tol_u ** 2
    rounding = 8.0 * 2.0 ** -24 * np.abs(h_ref) + 1e-6
    return first + second + rounding


def ffn_gelu_q4_0(w_up, w_down, x, up_bias=None, down_bias=None):
    """The whole chain from an fp32 activation.  Returns every stage: u (+ terms),
    h (float64), h32 (fp32), y (+ terms), tol_u."""
    u, tu = gemv_q4_0_f32(w_up, x)
    if up_bias is not None:
        b = np.asarray(up_bias, np.float32).astype(np.float64)
        u, tu = u + b, tu + np.abs(b)
    h = gelu(u)
    h32 = h.astype(np.float32)
    y, ty = gemv_q4_0_f32(w_down, h32)
    if down_bias is not None:
        b = np.asarray(down_bias, np.float32).astype(np.float64)
        y, ty = y + b, ty + np.abs(b)
    return dict(u=u, u_terms=tu, h=h, h32=h32, y=y, y_terms=ty, tol_u=gemv_tolerance(tu))
