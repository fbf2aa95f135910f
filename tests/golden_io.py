"""Reader for the hand-worked fixtures under tests/golden/ (``key = values`` lines)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (p.strip() for p in line.split("=", 1))
            out[key] = val
    return out


def floats(s):
    return [float(v) for v in s.split()]


def ints(s):
    return [int(v) for v in s.split()]


def hexbytes(s):
    return bytes(int(v, 16) for v in s.split())


def pairs(s, conv_key=int, conv_val=float):
    res = []
    for item in s.split():
        k, v = item.split(":")
        res.append((conv_key(k), conv_val(v)))
    return res
