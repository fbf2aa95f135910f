"""Pass bound for fp32 GEMV outputs (oracle; test infrastructure only).

An fp32 result passes when ``|y_kernel - y_oracle| <= 1e-5 * terms + 1e-6``,
where ``terms`` is the sum of the absolute values of the summands the kernel
rounds (``gemv_q4k_q8_int``, ``gemv_q4_0_*`` return it).  With fp32 unit
roundoff 2**-24 this leaves room for about 160 roundings along any chain, far
more than a blocked reduction of a 14336-long row performs.
"""
from __future__ import annotations

import numpy as np

GEMV_REL = 1e-5
GEMV_ABS = 1e-6


def gemv_tolerance(terms):
    return GEMV_REL * np.asarray(terms, np.float64) + GEMV_ABS
