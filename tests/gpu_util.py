"""Helpers for the GPU parity tests: device buffers from numpy, results back,
and a printed banner naming each case before it touches the GPU."""
import sys

import numpy as np


def banner(*parts):
    print("[gpu case]", *parts, flush=True)
    sys.stdout.flush()


def torch():
    import torch as _t
    return _t


def dev_bytes(arr: np.ndarray):
    t = torch()
    a = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
    return t.from_numpy(a.copy()).to("cuda")


def dev_f32(arr: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(arr, dtype=np.float32).copy()).to("cuda")


def empty_bytes(n: int, fill: int = 0xA5):
    t = torch()
    return t.full((n,), fill, dtype=t.uint8, device="cuda")


def empty_f32(n: int, fill: float = float("nan")):
    t = torch()
    return t.full((n,), fill, dtype=t.float32, device="cuda")


def host(t_):
    torch().cuda.synchronize()
    return t_.cpu().numpy()


def q8_host_bytes(t_, nblocks: int):
    return host(t_)[: nblocks * 40].reshape(nblocks, 40)


def first_mismatch(a, b, tol=None):
    """Index and values of the first element where a and b differ (beyond tol)."""
    a = np.asarray(a)
    b = np.asarray(b)
    bad = (a != b) if tol is None else (np.abs(a - b) > tol)
    idx = np.argwhere(bad)
    if idx.size == 0:
        return None
    i = tuple(idx[0])
    return i, a[i], b[i], int(bad.sum())
