"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (the oracle decides; see oracle/):
  * Q8_1 blocks: byte-exact (codes, d, s);
  * GEMV outputs: |y_gpu - y_oracle| <= 1e-5 * terms + 1e-6 per output, where
    terms = sum of |summands| of the integer form;
  * integer-exact inputs (d = dmin = 1, activation scale 1, small codes): every
    sub-block sum and every partial sum is an integer below 2**24, so y must
    match bit for bit -- this pins the int32 sub-block sums;
  * SwiGLU chain: per stage (see test_swiglu_*).
Inputs are seeded synthetic tensors (synth/); weights are fed to both sides,
and the GEMV tests give the GPU the oracle's own Q8_1 bytes so that a GEMV
failure is never a quantize failure in disguise.
"""
import os

import numpy as np
import pytest

import oracle
import synth
import q4_q8_integer_quantize_amd as rz
from golden_io import floats, hexbytes, ints, load, pairs
from gpu_util import (banner, dev_bytes, dev_f32, empty_bytes, empty_f32, first_mismatch, host,
                      q8_host_bytes)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ helpers
def gpu_quantize(x: np.ndarray, n_padded: int):
    x2 = x if x.ndim == 2 else x[None, :]
    nt, n = x2.shape
    xd = dev_f32(x2)
    out = empty_bytes(rz.q8_1_nbytes(n_padded, nt))
    rz.rz_q8_1_quantize(xd, n, n_padded, nt, out)
    return q8_host_bytes(out, nt * n_padded // 32).reshape(nt, n_padded // 32, 40)


def gpu_q4k(blob: np.ndarray, xq_bytes: np.ndarray, n_tokens: int = 1):
    out_dim, nsb, _ = blob.shape
    y = empty_f32(out_dim * n_tokens)
    rz.rz_q4k_q8_gemv(dev_bytes(blob), dev_bytes(xq_bytes), y, out_dim, nsb * 256, n_tokens)
    return host(y).reshape(n_tokens, out_dim)


def gpu_q4_0(blob: np.ndarray, x, x_format: int):
    out_dim, nb, _ = blob.shape
    y = empty_f32(out_dim)
    xd = dev_f32(x) if x_format == 0 else dev_bytes(x)
    rz.rz_q4_0_gemv(dev_bytes(blob), xd, x_format, y, out_dim, nb * 32)
    return host(y)


def assert_within(y_gpu, y_ref, terms, what):
    tol = oracle.gemv_tolerance(terms)
    err = np.abs(np.asarray(y_gpu, np.float64) - y_ref)
    bad = err > tol
    if bad.any():
        r = int(np.argmax(bad))
        raise AssertionError("%s: %d of %d outputs outside 1e-5*terms+1e-6; first row %d: "
                             "gpu=%r oracle=%r tol=%r terms=%r"
                             % (what, int(bad.sum()), bad.size, r, float(y_gpu[r]),
                                float(y_ref[r]), float(tol[r]), float(terms[r])))


def normed_activation(cid, n):
    """The attention workload's input: an fp32 N(0,1) hidden state through the
    oracle's RMSNorm (gamma ~ N(1, 0.1), eps 1e-5), rounded once to fp32."""
    x = synth.activation(synth.rng(cid, synth.T_ACT), n)
    gamma = synth.norm_weights(synth.rng(cid, synth.T_GAMMA), n)
    return oracle.rmsnorm(x, gamma, 1e-5).astype(np.float32)


def oracle_q4k(blob, xq, n_tokens=1):
    """Oracle y and terms for every token: (n_tokens, out_dim) each."""
    if n_tokens == 1 and xq.d.ndim == 1:
        y, t = oracle.gemv_q4k_q8_int(blob, xq)
        return y[None], t[None]
    ys, ts = zip(*(oracle.gemv_q4k_q8_int(blob, xq.token(t)) for t in range(n_tokens)))
    return np.stack(ys), np.stack(ts)


# ------------------------------------------------------------------ seeded random shapes
def _random_shapes(count, seed, max_k, step, budget, max_tokens=1):
    """(out_dim, in_dim, n, n_tokens, seed) with log-uniform out_dim, in_dim a
    multiple of `step` up to max_k steps, n <= in_dim (a ragged tail of zeros)
    and out_dim * in_dim * n_tokens within `budget` (oracle time)."""
    g = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        nt = int(g.integers(1, max_tokens + 1))
        in_dim = step * int(g.integers(1, max_k + 1))
        hi = max(1, min(4000, budget // (in_dim * nt)))
        out_dim = int(np.exp(g.uniform(0, np.log(hi + 1))))
        out_dim = max(1, min(out_dim, hi))
        n = int(g.integers(max(1, in_dim - step + 1), in_dim + 1))
        cases.append((out_dim, in_dim, n, nt, int(g.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("out_dim,in_dim,n,n_tokens,seed",
                         _random_shapes(24, 71, 80, 256, 24_000_000, max_tokens=8))
def test_q4k_q8_gemv_random_shapes(out_dim, in_dim, n, n_tokens, seed):
    """rz_q4k_q8_gemv on seeded random shapes: 1..8 tokens (3 and more on the
    matrix cores), rows up to 20480 values (column chunks past the register
    window), ragged row counts and activation tails; every output of every
    token within the bound of the oracle."""
    banner("q4k random", out_dim, in_dim, n, n_tokens)
    blob = synth.q4k_weights(synth.rng(72, seed), out_dim, in_dim)
    X = synth.activation(np.random.default_rng(seed), in_dim, n_tokens=n_tokens)
    X = X.reshape(n_tokens, in_dim)
    X[:, n:] = 0.0
    xq = oracle.quantize_q8_1(X if n_tokens > 1 else X[0])
    Y = gpu_q4k(blob, oracle.q8_1_to_bytes(xq), n_tokens)
    y_ref, terms = oracle_q4k(blob, xq, n_tokens)
    for t in range(n_tokens):
        assert_within(Y[t], y_ref[t], terms[t], "token %d" % t)


@pytest.mark.parametrize("out_dim,in_dim,n,n_tokens,seed",
                         _random_shapes(16, 73, 64, 256, 16_000_000))
def test_q4k_q8_gemv_f32_random_shapes(out_dim, in_dim, n, n_tokens, seed):
    """The fused quantize + GEMV on seeded random shapes, n <= in_dim values
    (zero tail, dword activation loads when n is not a multiple of 4): the
    Q8_1 side output byte-equal to the oracle's, y within its bound."""
    banner("q4k f32 random", out_dim, in_dim, n)
    blob = synth.q4k_weights(synth.rng(74, seed), out_dim, in_dim)
    x = synth.activation(np.random.default_rng(seed), n)
    xq_ref = oracle.quantize_q8_1(x, in_dim)
    xq = empty_bytes(rz.q8_1_nbytes(in_dim))
    y = empty_f32(out_dim)
    rz.rz_q4k_q8_gemv_f32(dev_bytes(blob), dev_f32(x), n, xq, y, out_dim, in_dim)
    assert np.array_equal(host(xq), oracle.q8_1_to_bytes(xq_ref).reshape(-1))
    y_ref, terms = oracle.gemv_q4k_q8_int(blob, xq_ref)
    assert_within(host(y), y_ref, terms, "fused")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("out_dim,in_dim,n,n_tokens,seed",
                         _random_shapes(12, 75, 600, 64, 24_000_000))
def test_q4_0_gemv_random_shapes(fmt, out_dim, in_dim, n, n_tokens, seed):
    """rz_q4_0_gemv on seeded random shapes, rows up to 38400 values (several
    column chunks in both formats), both activation formats, within the bound
    of the oracle."""
    banner("q4_0 random", fmt, out_dim, in_dim, n)
    blob = synth.q4_0_weights(synth.rng(76, seed), out_dim, in_dim)
    x = _padded(synth.activation(np.random.default_rng(seed), n), in_dim)
    if fmt == 0:
        y_ref, terms = oracle.gemv_q4_0_f32(blob, x)
        y = gpu_q4_0(blob, x, 0)
    else:
        xq = oracle.quantize_q8_1(x)
        y_ref, terms = oracle.gemv_q4_0_q8_int(blob, xq)
        y = gpu_q4_0(blob, oracle.q8_1_to_bytes(xq), 1)
    assert_within(y, y_ref, terms, "q4_0 fmt %d" % fmt)


@pytest.mark.parametrize("out_dim,in_dim,n,n_tokens,seed",
                         _random_shapes(12, 77, 80, 256, 16_000_000))
def test_q4k_xf32_random_shapes(out_dim, in_dim, n, n_tokens, seed):
    """rz_q4k_gemv (fp32 activation, no Q8_1) on seeded random shapes with a
    ragged activation length n, within the bound of the oracle's fp32 form."""
    banner("q4k xf32 random", out_dim, in_dim, n)
    blob = synth.q4k_weights(synth.rng(78, seed), out_dim, in_dim)
    x = synth.activation(np.random.default_rng(seed), n)
    y = gpu_q4k_xf32(blob, x)
    y_ref, terms = oracle.gemv_q4k_f32(blob, _padded(x, in_dim))
    assert_within(y, y_ref, terms, "xf32")


# ------------------------------------------------------------------ Q8_1
def test_q8_1_hand_worked_blocks_gpu():
    banner("q8_1 hand-worked blocks")
    fx = load("q8_1_blocks.txt")
    x = np.zeros(128, np.float32)
    for b, key in enumerate("ABCD"):
        vals = floats(fx[key + ".x"])
        x[32 * b: 32 * b + len(vals)] = vals
    got = gpu_quantize(x, 128)[0]
    for b, key in enumerate("ABCD"):
        blk = got[b]
        assert blk[0:4].view("<f4")[0] == np.float32(float(fx[key + ".d"]))
        assert blk[4:8].view("<f4")[0] == np.float32(float(fx[key + ".s"]))
        q = np.zeros(32, np.int64)
        qv = ints(fx[key + ".q"])
        q[:len(qv)] = qv
        assert np.array_equal(blk[8:40].view(np.int8).astype(np.int64), q), key
    assert np.array_equal(got, oracle.q8_1_to_bytes(oracle.quantize_q8_1(x, 128)))


def _q8_case(kind, n, nt, seed):
    g = np.random.default_rng(seed)
    if kind == "normal":
        return synth.activation(g, n, nt if nt > 1 else None)
    if kind == "rmsnorm":
        return normed_activation(1, n)
    if kind == "wide":
        x = g.standard_normal((nt, n)) * np.exp(g.uniform(-20, 20, (nt, n)))
        return x.astype(np.float32)[0] if nt == 1 else x.astype(np.float32)
    if kind == "tiny":
        return (g.standard_normal((nt, n)) * 1e-30).astype(np.float32).squeeze(0) if nt == 1 else \
            (g.standard_normal((nt, n)) * 1e-30).astype(np.float32)
    if kind == "huge":
        return (g.standard_normal((nt, n)) * 1e30).astype(np.float32).squeeze(0) if nt == 1 else \
            (g.standard_normal((nt, n)) * 1e30).astype(np.float32)
    if kind == "denormal":
        # per block a scale of 2^-149 .. 2^-118 (denormal and smallest normal
        # d, and blocks whose d rounds to 0) times integers up to 127
        e = g.integers(-149, -117, (nt, n // 32 + 1)).repeat(32, axis=1)[:, :n]
        kmax = g.integers(1, 128, (nt, n // 32 + 1)).repeat(32, axis=1)[:, :n]
        k = np.rint(g.uniform(-1, 1, (nt, n)) * kmax)
        x = np.ldexp(k, e).astype(np.float32)
        return x[0] if nt == 1 else x
    if kind == "scale_edge":
        # block maxima on both sides of 2^-60, where the kernel's exact 2^64 scaling starts
        e = g.uniform(-64, -56, (nt, n // 32 + 1)).repeat(32, axis=1)[:, :n]
        x = (g.uniform(-1, 1, (nt, n)) * np.exp2(e)).astype(np.float32)
        return x[0] if nt == 1 else x
    if kind == "boundary":
        # values within a few ulps of (k + 1/2) d: every code is a close rounding decision
        nb = n // 32
        amax = np.exp2(g.uniform(-30, 30, (nt, nb))).astype(np.float32)
        d = (amax / np.float32(127)).astype(np.float32)
        k = g.integers(-127, 127, (nt, nb, 32)) + 0.5
        x = (k * d[..., None].astype(np.float64)).astype(np.float32)
        x = (x.view(np.int32) + g.integers(-3, 4, x.shape).astype(np.int32)).view(np.float32)
        x = np.clip(x, -amax[..., None], amax[..., None])
        x[..., 0] = amax
        x = x.reshape(nt, nb * 32)
        return x[0] if nt == 1 else x
    if kind == "recip_edge":
        # blocks whose d = RN(amax/127) has an all-ones significand (2 - 2^-23
        # times a power of two, the one divisor whose reciprocal a Newton step
        # cannot always correct), with values within ulps of (k + 1/2) d
        nb = n // 32
        e = g.integers(-40, 40, (nt, nb))
        d = np.ldexp(2.0 - 2.0 ** -23, e).astype(np.float32)
        amax = (d.astype(np.float64) * 127).astype(np.float32)
        for _ in range(4):   # step amax until amax / 127 rounds to d
            lo = (amax / np.float32(127)).astype(np.float32) < d
            hi = (amax / np.float32(127)).astype(np.float32) > d
            amax = (amax.view(np.int32) + lo.astype(np.int32) - hi.astype(np.int32)).view(np.float32)
        assert np.array_equal((amax / np.float32(127)).astype(np.float32), d)
        k = g.integers(-127, 127, (nt, nb, 32)) + 0.5
        x = (k * d[..., None].astype(np.float64)).astype(np.float32)
        x = (x.view(np.int32) + g.integers(-2, 3, x.shape).astype(np.int32)).view(np.float32)
        x = np.clip(x, -amax[..., None], amax[..., None])
        x[..., 0] = amax
        x = x.reshape(nt, nb * 32)
        return x[0] if nt == 1 else x
    if kind == "ties":
        # halves at d = 1: every code is a round-half-to-even decision
        x = (g.integers(-254, 255, (nt, n)) / 2.0).astype(np.float32)
        x[:, ::32] = 127.0
        return x[0] if nt == 1 else x
    raise ValueError(kind)


@pytest.mark.parametrize("kind,n,n_padded,nt", [
    ("normal", 896, 1024, 1),      # padded activation of the 896-wide workloads
    ("rmsnorm", 4096, 4096, 1),    # attention-projection input
    ("normal", 4096, 4096, 8),     # 8-token batch
    ("normal", 14336, 14336, 1),   # requantized FFN width
    ("normal", 1000, 1024, 1),     # ragged tail inside a block
    ("normal", 33, 64, 3),
    ("normal", 1, 32, 1),
    ("normal", 100, 128, 5),
    ("wide", 2048, 2048, 2),
    ("tiny", 512, 512, 1),
    ("huge", 512, 512, 2),
    ("ties", 1024, 1024, 4),
    ("denormal", 4096, 4096, 2),
    ("scale_edge", 4096, 4096, 1),
    ("boundary", 8192, 8192, 4),
    ("recip_edge", 4096, 4096, 2),
])
def test_q8_1_matches_oracle(kind, n, n_padded, nt):
    banner("q8_1", kind, n, n_padded, nt)
    x = _q8_case(kind, n, nt, seed=n + nt)
    got = gpu_quantize(x, n_padded)
    want = oracle.q8_1_to_bytes(oracle.quantize_q8_1(x, n_padded)).reshape(got.shape)
    mm = first_mismatch(got, want)
    assert mm is None, "first differing byte %s gpu=%d oracle=%d (%d bytes differ)" % mm


def test_q8_1_zero_input_gives_zero_blocks():
    banner("q8_1 zeros")
    got = gpu_quantize(np.zeros(256, np.float32), 256)
    assert not got.any()


# ------------------------------------------------------------------ Q4_K pins
def test_q4k_hand_worked_superblock_gpu():
    banner("q4k hand-worked super-block")
    fx = load("q4k_superblock.txt")
    sb = hexbytes(fx["header_hex"]) + hexbytes(fx["qs_fill_hex"]) * 128
    blob = np.frombuffer(sb * 3, np.uint8).reshape(3, 1, 144).copy()   # three identical rows
    ones = np.zeros((8, 40), np.uint8)
    ones[:, 0:4] = np.frombuffer(np.float32(1).tobytes(), np.uint8)
    ones[:, 4:8] = np.frombuffer(np.float32(32).tobytes(), np.uint8)
    ones[:, 8:40] = 1
    y = gpu_q4k(blob, ones)[0]
    assert np.all(y == float(fx["y_ones"])), y


def test_q4k_nibble_order_gpu():
    banner("q4k nibble order")
    fx = load("q4k_nibble_order.txt")
    raw = bytearray(hexbytes(fx["header_hex"]) + bytes(128))
    for k, v in pairs(fx["qs_set"], int, lambda s: int(s, 16)):
        raw[16 + k] = v
    blob = np.frombuffer(bytes(raw), np.uint8).reshape(1, 1, 144).copy()
    x = np.zeros((8, 40), np.uint8)
    x[1, 0:4] = np.frombuffer(np.float32(1).tobytes(), np.uint8)
    x[1, 4:8] = np.frombuffer(np.float32(1).tobytes(), np.uint8)
    x[1, 8] = 1
    assert gpu_q4k(blob, x)[0][0] == float(fx["y_onehot32"])


def _integer_q8(nblocks, seed, qmax=8):
    g = np.random.default_rng(seed)
    q = g.integers(-qmax, qmax + 1, size=(nblocks, 32)).astype(np.int8)
    xq = oracle.Q8Blocks(np.ones(nblocks, np.float32), q.sum(axis=1).astype(np.float32), q)
    return xq


@pytest.mark.parametrize("out_dim,in_dim", [(5, 256), (64, 512), (300, 1024), (37, 2048),
                                            (19, 1280)])
def test_q4k_integer_exact_inputs_bit_exact(out_dim, in_dim):
    """d = dmin = 1, activation d = 1, codes in [-8, 8]: y is an integer below
    2**24 computed exactly by any summation order, so the GPU must match the
    oracle bit for bit; any wrong int32 sub-block sum shows up as a difference."""
    banner("q4k integer-exact", out_dim, in_dim)
    blob = synth.q4k_weights(synth.rng(60, out_dim), out_dim, in_dim, d_fixed=1.0, dmin_fixed=1.0)
    xq = _integer_q8(in_dim // 32, seed=in_dim)
    y_ref, _ = oracle.gemv_q4k_q8_int(blob, xq)
    y = gpu_q4k(blob, oracle.q8_1_to_bytes(xq))[0]
    assert np.all(np.abs(y_ref) < 2 ** 24)
    mm = first_mismatch(y.astype(np.float64), y_ref)
    assert mm is None, "row %s gpu=%r oracle=%r (%d rows differ)" % mm


# ------------------------------------------------------------------ Q4_K parity
@pytest.mark.parametrize("out_dim,in_dim", [
    (1, 256), (3, 256), (64, 256), (65, 256), (257, 256),
    (1, 512), (3, 512), (64, 512), (65, 512), (257, 512),
    (896, 1024),          # the 896-wide workload, in_dim padded to 1024
    (100, 768), (129, 1280), (70, 3072), (33, 14336),
    (40, 20480),          # longer than one register window: two column chunks
])
def test_q4k_matches_oracle(out_dim, in_dim):
    banner("q4k", out_dim, in_dim)
    blob = synth.q4k_weights(synth.rng(10, out_dim * 7 + in_dim), out_dim, in_dim)
    xq = oracle.quantize_q8_1(synth.activation(synth.rng(10, in_dim), in_dim))
    y_ref, terms = oracle.gemv_q4k_q8_int(blob, xq)
    y = gpu_q4k(blob, oracle.q8_1_to_bytes(xq))[0]
    assert_within(y, y_ref, terms, "q4k %dx%d" % (out_dim, in_dim))


def test_q4k_padding_invariance_gpu():
    """in_dim 896 zero-padded to 1024: re-randomising the padded half of the last
    super-block (nibbles and 6-bit fields of sub-blocks 4..7) leaves y bit-identical,
    and y agrees with the oracle restricted to the first 896 values."""
    banner("q4k padding invariance 896->1024")
    n, in_dim, rows = 896, 1024, 896
    blob = synth.q4k_weights(synth.rng(0, synth.T_W0), rows, in_dim)
    x = synth.activation(synth.rng(0, synth.T_ACT), n)
    xq = oracle.quantize_q8_1(x, in_dim)
    xb = oracle.q8_1_to_bytes(xq)
    y1 = gpu_q4k(blob, xb)[0]
    g = np.random.default_rng(1234)
    b2 = blob.copy()
    b2[:, -1, 16 + 64:144] = g.integers(0, 256, (rows, 64), dtype=np.uint8)
    r = g.integers(0, 256, (rows, 12), dtype=np.uint8)
    b2[:, -1, 4:12] = (blob[:, -1, 4:12] & 63) | (r[:, 0:8] & 0xC0)
    b2[:, -1, 12:16] = r[:, 8:12]
    y2 = gpu_q4k(b2, xb)[0]
    assert np.array_equal(y1, y2)
    w = oracle.dequantize_q4k(blob)[:, :n]
    xh = oracle.dequantize_q8_1(xq)[:n]
    assert_within(y1, w @ xh, np.abs(w) @ np.abs(xh) + oracle.gemv_q4k_q8_int(blob, xq)[1],
                  "q4k padded")


def test_q4k_scaling_and_row_permutation_gpu():
    """Doubling every activation d and s doubles y exactly; permuting weight rows
    permutes y exactly."""
    banner("q4k scaling/permutation")
    out_dim, in_dim = 333, 4096
    blob = synth.q4k_weights(synth.rng(11, 1), out_dim, in_dim)
    xq = oracle.quantize_q8_1(synth.activation(synth.rng(11, 0), in_dim))
    y = gpu_q4k(blob, oracle.q8_1_to_bytes(xq))[0]
    x2 = oracle.Q8Blocks(xq.d * np.float32(2), xq.s * np.float32(2), xq.q)
    y2 = gpu_q4k(blob, oracle.q8_1_to_bytes(x2))[0]
    assert np.array_equal(y2, 2 * y)
    perm = np.random.default_rng(3).permutation(out_dim)
    yp = gpu_q4k(blob[perm].copy(), oracle.q8_1_to_bytes(xq))[0]
    assert np.array_equal(yp, y[perm])


@pytest.mark.parametrize("n_tokens", [1, 2, 3, 4, 5, 6, 7, 8])
def test_q4k_token_batch(n_tokens):
    """Each token against the oracle; the tokens of a batch do not interact:
    reversing their order reverses the outputs bit for bit."""
    banner("q4k batch", n_tokens)
    out_dim, in_dim = 515, 4096
    blob = synth.q4k_weights(synth.rng(4, 1), out_dim, in_dim)
    X = synth.activation(synth.rng(4, 0), in_dim, n_tokens=n_tokens)
    xq = oracle.quantize_q8_1(X)
    xb = oracle.q8_1_to_bytes(xq)
    Y = gpu_q4k(blob, xb, n_tokens)
    y_ref, terms = oracle_q4k(blob, xq, n_tokens)
    for t in range(n_tokens):
        assert_within(Y[t], y_ref[t], terms[t], "token %d" % t)
    Yr = gpu_q4k(blob, np.ascontiguousarray(xb.reshape(n_tokens, -1)[::-1]), n_tokens)
    assert np.array_equal(Yr, Y[::-1]), "token order changes the results"


@pytest.mark.parametrize("n_tokens,out_dim,in_dim", [
    (8, 515, 4096), (3, 64, 1024), (5, 100, 2048), (8, 33, 14336), (7, 17, 3072), (4, 16, 256),
])
def test_q4k_batch_integer_exact_bit_exact(n_tokens, out_dim, in_dim):
    """d = dmin = 1, activation d = 1, codes in [-8, 8] for every token: each
    output is an integer below 2**24 that any summation order reaches exactly,
    so the batched GPU result must equal the oracle bit for bit; a wrong int32
    sub-block sum, or a token or sub-block mixed into another, shows up here."""
    banner("q4k batch integer-exact", n_tokens, out_dim, in_dim)
    blob = synth.q4k_weights(synth.rng(61, out_dim), out_dim, in_dim, d_fixed=1.0, dmin_fixed=1.0)
    nb = in_dim // 32
    toks = [_integer_q8(nb, seed=1000 * t + in_dim) for t in range(n_tokens)]
    xb = np.concatenate([oracle.q8_1_to_bytes(q) for q in toks])
    Y = gpu_q4k(blob, xb, n_tokens)
    for t, q in enumerate(toks):
        y_ref, _ = oracle.gemv_q4k_q8_int(blob, q)
        assert np.all(np.abs(y_ref) < 2 ** 24)
        mm = first_mismatch(Y[t].astype(np.float64), y_ref)
        assert mm is None, "token %d: row %s gpu=%r oracle=%r (%d rows differ)" % ((t,) + mm)


# ------------------------------------------------------------------ fused quantize + GEMV
@pytest.mark.parametrize("out_dim,n,in_dim", [
    (3, 200, 256), (65, 512, 512), (896, 896, 1024), (129, 1280, 1280), (1000, 3000, 3072),
    (1024, 4096, 4096), (2047, 4000, 4096), (2048, 4096, 4096),   # one / two rows a group
    (14336, 4096, 4096), (4096, 14336, 14336), (77, 16384, 16384),
])
def test_q4k_gemv_f32_matches_two_step_and_oracle(out_dim, n, in_dim):
    """One launch (quantize in LDS + GEMV) equals rz_q8_1_quantize followed by
    rz_q4k_q8_gemv bit for bit; its Q8_1 side output equals the oracle's bytes;
    y is within the GEMV bound of the oracle."""
    banner("q4k gemv f32", out_dim, n, in_dim)
    blob = synth.q4k_weights(synth.rng(12, out_dim + in_dim), out_dim, in_dim)
    x = synth.activation(synth.rng(12, n), n)
    wd = dev_bytes(blob)
    xd = dev_f32(x)
    xq = empty_bytes(rz.q8_1_nbytes(in_dim))
    y = empty_f32(out_dim)
    rz.rz_q4k_q8_gemv_f32(wd, xd, n, xq, y, out_dim, in_dim)
    y_f = host(y)
    xq_f = q8_host_bytes(xq, in_dim // 32)
    xq_ref = oracle.quantize_q8_1(x, in_dim)
    assert np.array_equal(xq_f, oracle.q8_1_to_bytes(xq_ref))
    xq2 = empty_bytes(rz.q8_1_nbytes(in_dim))
    rz.rz_q8_1_quantize(xd, n, in_dim, 1, xq2)
    y2 = empty_f32(out_dim)
    rz.rz_q4k_q8_gemv(wd, xq2, y2, out_dim, in_dim, 1)
    assert np.array_equal(y_f, host(y2))
    y_ref, terms = oracle.gemv_q4k_q8_int(blob, xq_ref)
    assert_within(y_f, y_ref, terms, "q4k gemv f32 %dx%d" % (out_dim, in_dim))


def test_q4k_gemv_f32_without_side_output():
    banner("q4k gemv f32 no x_q8")
    out_dim, in_dim = 300, 2048
    blob = synth.q4k_weights(synth.rng(13, 1), out_dim, in_dim)
    x = synth.activation(synth.rng(13, 0), in_dim)
    y1, y2 = empty_f32(out_dim), empty_f32(out_dim)
    rz.rz_q4k_q8_gemv_f32(dev_bytes(blob), dev_f32(x), in_dim, None, y1, out_dim, in_dim)
    xq = empty_bytes(rz.q8_1_nbytes(in_dim))
    rz.rz_q4k_q8_gemv_f32(dev_bytes(blob), dev_f32(x), in_dim, xq, y2, out_dim, in_dim)
    assert np.array_equal(host(y1), host(y2))


# ------------------------------------------------------------------ full-size workloads
def test_q4k_attention_projections_full():
    """Q 4096x4096, K/V 1024x4096, O 4096x4096 sharing one RMSNorm'd activation."""
    w = synth.WORKLOADS["attn_4096"]
    x = normed_activation(1, w["n"])
    xq = oracle.quantize_q8_1(x, w["in_dim"])
    got_q8 = gpu_quantize(x, w["in_dim"])[0]
    assert np.array_equal(got_q8, oracle.q8_1_to_bytes(xq))
    for k, (name, rows) in enumerate(w["shapes"]):
        banner("attention", name, rows)
        blob = synth.q4k_weights(synth.rng(1, synth.T_W0 + k), rows, w["in_dim"])
        y_ref, terms = oracle.gemv_q4k_q8_int(blob, xq)
        y = gpu_q4k(blob, got_q8)[0]
        assert_within(y, y_ref, terms, "attention " + name)


def test_q4k_multi_attention_one_launch():
    """The four attention projections in one rz_q4k_q8_gemv_multi launch: each
    output equals its own rz_q4k_q8_gemv call bit for bit and the oracle within
    the GEMV bound."""
    w = synth.WORKLOADS["attn_4096"]
    x = normed_activation(1, w["n"])
    xq = oracle.quantize_q8_1(x, w["in_dim"])
    xb = dev_bytes(oracle.q8_1_to_bytes(xq))
    blobs = [synth.q4k_weights(synth.rng(1, synth.T_W0 + k), rows, w["in_dim"])
             for k, (_, rows) in enumerate(w["shapes"])]
    dws = [dev_bytes(b) for b in blobs]
    ys = [empty_f32(rows) for _, rows in w["shapes"]]
    banner("multi attention", len(ys))
    rz.rz_q4k_q8_gemv_multi(dws, xb, ys, [rows for _, rows in w["shapes"]], w["in_dim"])
    for k, (name, rows) in enumerate(w["shapes"]):
        single = empty_f32(rows)
        rz.rz_q4k_q8_gemv(dws[k], xb, single, rows, w["in_dim"], 1)
        assert np.array_equal(host(ys[k]), host(single)), name
        y_ref, terms = oracle.gemv_q4k_q8_int(blobs[k], xq)
        assert_within(host(ys[k]), y_ref, terms, "multi " + name)


@pytest.mark.parametrize("n_tokens,out_dims,in_dim", [
    (1, [1, 65, 257], 512), (2, [3, 64], 1024), (1, [896, 100, 7, 33, 1, 2, 3, 129], 1280),
    (5, [33, 64], 4096), (2, [17, 40], 20480),
])
def test_q4k_multi_matches_single_calls(n_tokens, out_dims, in_dim):
    """Ragged matrices, up to 8 of them, one and two tokens in one launch, and
    the per-matrix fallbacks (more tokens, longer rows): every output equals
    its own single-matrix call bit for bit; the first matrix is also checked
    against the oracle."""
    banner("multi", n_tokens, out_dims, in_dim)
    blobs = [synth.q4k_weights(synth.rng(70, 10 * k + o), o, in_dim) for k, o in enumerate(out_dims)]
    X = synth.activation(synth.rng(70, in_dim), in_dim, n_tokens=n_tokens)
    xq = oracle.quantize_q8_1(X)
    xb = dev_bytes(oracle.q8_1_to_bytes(xq))
    dws = [dev_bytes(b) for b in blobs]
    ys = [empty_f32(o * n_tokens) for o in out_dims]
    rz.rz_q4k_q8_gemv_multi(dws, xb, ys, out_dims, in_dim, n_tokens)
    for k, o in enumerate(out_dims):
        single = empty_f32(o * n_tokens)
        rz.rz_q4k_q8_gemv(dws[k], xb, single, o, in_dim, n_tokens)
        assert np.array_equal(host(ys[k]), host(single)), "matrix %d" % k
    y_ref, terms = oracle_q4k(blobs[0], xq, n_tokens)
    Y = host(ys[0]).reshape(n_tokens, out_dims[0])
    for t in range(n_tokens):
        assert_within(Y[t], y_ref[t], terms[t], "multi token %d" % t)


def test_q4k_gate_4096_to_14336_full():
    """The measured GEMV (4096 -> 14336, one token) in the launch configuration
    the benchmark times: GPU quantize then GPU GEMV, every output checked."""
    banner("q4k 4096->14336 full")
    blob = synth.q4k_weights(synth.rng(2, synth.T_W0), 14336, 4096)
    x = synth.activation(synth.rng(2, synth.T_ACT), 4096)
    xq = oracle.quantize_q8_1(x)
    got_q8 = gpu_quantize(x, 4096)[0]
    assert np.array_equal(got_q8, oracle.q8_1_to_bytes(xq))
    y_ref, terms = oracle.gemv_q4k_q8_int(blob, xq)
    assert_within(gpu_q4k(blob, got_q8)[0], y_ref, terms, "gate 4096->14336")


def test_q4k_batch8_full():
    """8 tokens x 4096 -> 14336 (the small-batch decode workload): every output
    of every token against the oracle, each token with its own Q8_1 vector."""
    banner("q4k batch8 4096->14336")
    w = synth.WORKLOADS["q4k_batch8"]
    blob = synth.q4k_weights(synth.rng(4, synth.T_W0), w["out_dim"], w["in_dim"])
    X = synth.activation(synth.rng(4, synth.T_ACT), w["in_dim"], n_tokens=8)
    xq = oracle.quantize_q8_1(X)
    got_q8 = gpu_quantize(X, w["in_dim"])
    assert np.array_equal(got_q8, oracle.q8_1_to_bytes(xq))
    Y = gpu_q4k(blob, got_q8, 8)
    for t in range(8):
        y_ref, terms = oracle.gemv_q4k_q8_int(blob, xq.token(t))
        assert_within(Y[t], y_ref, terms, "batch8 token %d" % t)


def test_q4k_largest_matrix_sampled():
    """The largest matrix the ABI accepts (just under 2 GiB, whose last bytes
    sit 8 KB below 2**31, where a signed 32-bit offset would overflow): rows
    at both ends and sampled rows in between, for one token, 8 tokens (the
    matrix-core path in four column passes), the fused quantize + GEMV entry
    and the fp32-activation GEMV, each against the oracle."""
    in_dim = 16384
    row_bytes = in_dim // 256 * 144
    out_dim = (2 ** 31 - 1) // row_bytes              # 233016 rows, 2,147,475,456 bytes
    banner("q4k largest matrix %d x %d" % (out_dim, in_dim))
    blob = synth.q4k_weights(synth.rng(11, 1), out_dim, in_dim)
    assert blob.nbytes < 2 ** 31 and blob.nbytes > 2 ** 31 - 2 * row_bytes
    g = np.random.default_rng(11)
    rows = np.unique(np.concatenate([np.arange(64), out_dim - 64 + np.arange(64),
                                     g.choice(out_dim, 128, replace=False)]))
    X = synth.activation(synth.rng(11, synth.T_ACT), in_dim, n_tokens=8)
    xq = oracle.quantize_q8_1(X)
    xq_bytes = oracle.q8_1_to_bytes(xq)
    wd = dev_bytes(blob)
    sub = blob[rows]
    # 1 and 8 tokens on the GEMV entry
    for nt in (1, 8):
        y = empty_f32(out_dim * nt)
        rz.rz_q4k_q8_gemv(wd, dev_bytes(xq_bytes[:nt]), y, out_dim, in_dim, nt)
        Y = host(y).reshape(nt, out_dim)
        for t in range(nt):
            y_ref, terms = oracle.gemv_q4k_q8_int(sub, xq.token(t))
            assert_within(Y[t, rows], y_ref, terms, "largest matrix, %d tokens, token %d" % (nt, t))
    # the fused entry: quantize token 0 in the kernel, then the GEMV
    y = empty_f32(out_dim)
    rz.rz_q4k_q8_gemv_f32(wd, dev_f32(X[0]), in_dim, None, y, out_dim, in_dim)
    y_ref, terms = oracle.gemv_q4k_q8_int(sub, xq.token(0))
    assert_within(host(y)[rows], y_ref, terms, "largest matrix, fused quantize + GEMV")
    # the fp32-activation GEMV
    y = empty_f32(out_dim)
    rz.rz_q4k_gemv(wd, dev_f32(X[0]), in_dim, y, out_dim, in_dim)
    y_ref, terms = oracle.gemv_q4k_f32(sub, X[0])
    assert_within(host(y)[rows], y_ref, terms, "largest matrix, fp32 activation")


def test_q4_0_largest_matrix_sampled():
    """The largest Q4_0 matrix the ABI accepts at the LM head's row length
    (3,728,270 x 1024, less than one row below 2 GiB): rows at both ends and
    sampled rows, fp32 and Q8_1 activations, against the oracle; with a bias
    and the greedy token, the logits are the plain GEMV plus the bias bit for
    bit and the chosen row is the first maximum of them."""
    in_dim = 1024
    row_bytes = in_dim // 32 * 18
    out_dim = (2 ** 31 - 1) // row_bytes
    banner("q4_0 largest matrix %d x %d" % (out_dim, in_dim))
    blob = synth.q4_0_weights(synth.rng(12, 1), out_dim, in_dim)
    assert 2 ** 31 - 2 * row_bytes < blob.nbytes < 2 ** 31
    g = np.random.default_rng(12)
    rows = np.unique(np.concatenate([np.arange(64), out_dim - 64 + np.arange(64),
                                     g.choice(out_dim, 128, replace=False)]))
    sub = blob[rows]
    x = synth.activation(synth.rng(12, synth.T_ACT), in_dim)
    xq = oracle.quantize_q8_1(x)
    wd = dev_bytes(blob)
    for fmt in (0, 1):
        y = empty_f32(out_dim)
        xd = dev_f32(x) if fmt == 0 else dev_bytes(oracle.q8_1_to_bytes(xq))
        rz.rz_q4_0_gemv(wd, xd, fmt, y, out_dim, in_dim)
        if fmt == 0:
            y_ref, terms = oracle.gemv_q4_0_f32(sub, x)
        else:
            y_ref, terms = oracle.gemv_q4_0_q8_int(sub, xq)
        assert_within(host(y)[rows], y_ref, terms, "largest Q4_0 matrix, x_format %d" % fmt)
        bias = synth.activation(synth.rng(12, 2), out_dim)
        logits = empty_f32(out_dim)
        idx = __import__("torch").full((1,), -7, dtype=__import__("torch").int32, device="cuda")
        ws = empty_bytes(rz.rz_lm_head_q4_0_workspace_bytes(out_dim, in_dim, fmt))
        rz.rz_lm_head_q4_0(wd, xd, fmt, dev_f32(bias), logits, out_dim, in_dim, idx, None, ws)
        lg = host(logits)
        # one column pass at 1024 values: logits are fl32(W x + bias) bit for bit
        mm = first_mismatch(lg, (host(y) + bias).astype(np.float32))
        assert mm is None, "logit %s fused=%r plain+bias=%r (%d differ)" % mm
        assert int(host(idx)[0]) == oracle.argmax_first(lg)


# ------------------------------------------------------------------ Q4_0
def test_q4_0_hand_worked_block_gpu():
    banner("q4_0 hand-worked block")
    fx = load("q4_0_block.txt")
    blk = hexbytes(fx["block_hex"])
    zero_blk = np.float16(0).tobytes() + bytes(16)
    blob = np.frombuffer(blk + zero_blk, np.uint8).reshape(1, 2, 18).copy()
    for k, key in ((0, "y_onehot0"), (16, "y_onehot16")):
        x = np.zeros(64, np.float32)
        x[k] = 1.0
        assert gpu_q4_0(blob, x, 0)[0] == float(fx[key])
        xq = np.zeros((2, 40), np.uint8)
        xq[0, 0:4] = np.frombuffer(np.float32(1).tobytes(), np.uint8)
        xq[0, 4:8] = np.frombuffer(np.float32(1).tobytes(), np.uint8)
        xq[0, 8 + k] = 1
        assert gpu_q4_0(blob, xq, 1)[0] == float(fx[key])


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("out_dim,in_dim", [
    (1, 64), (3, 128), (65, 192), (257, 1024), (130, 4096),
    (70, 1536),      # fp32: 8 lanes x 3 pairs a row
    (129, 2560),     # fp32: 16 lanes x 3 pairs, 8 of 48 slots idle
    (66, 6144),      # fp32: 32 lanes x 3 pairs
    (33, 8192),      # fp32: 32 lanes x 4 pairs
    (9, 10240),      # fp32: 64 lanes x 3 pairs, 32 of 192 slots idle
    (5, 12288),      # fp32: 64 lanes x 3 pairs, all busy
    (3072, 10240),   # fp32: 3072 one-row waves in 12-wave workgroups (256)
    (2560, 10240),   # fp32: 2560 one-row waves in 10-wave workgroups (256)
    (17, 16384),     # fp32: two column chunks
    (40, 20480),     # both formats chunked
])
def test_q4_0_matches_oracle(fmt, out_dim, in_dim):
    banner("q4_0", "fp32" if fmt == 0 else "q8_1", out_dim, in_dim)
    blob = synth.q4_0_weights(synth.rng(30, out_dim + in_dim), out_dim, in_dim)
    x = synth.activation(synth.rng(30, in_dim), in_dim)
    if fmt == 0:
        y_ref, terms = oracle.gemv_q4_0_f32(blob, x)
        y = gpu_q4_0(blob, x, 0)
    else:
        xq = oracle.quantize_q8_1(x)
        y_ref, terms = oracle.gemv_q4_0_q8_int(blob, xq)
        y = gpu_q4_0(blob, oracle.q8_1_to_bytes(xq), 1)
    assert_within(y, y_ref, terms, "q4_0 %dx%d fmt %d" % (out_dim, in_dim, fmt))


@pytest.mark.parametrize("fmt", [0, 1])
def test_q4_0_lm_head_full(fmt):
    """LM head 151936 x (896 padded to 1024), every logit checked."""
    banner("q4_0 lm head full", fmt)
    w = synth.WORKLOADS["lm_head_q4_0"]
    blob = synth.q4_0_weights(synth.rng(3, synth.T_W0), w["out_dim"], w["in_dim"])
    x = np.zeros(w["in_dim"], np.float32)
    x[:w["n"]] = synth.activation(synth.rng(3, synth.T_ACT), w["n"])
    if fmt == 0:
        y_ref, terms = oracle.gemv_q4_0_f32(blob, x)
        y = gpu_q4_0(blob, x, 0)
    else:
        xq = oracle.quantize_q8_1(x[:w["n"]], w["in_dim"])
        y_ref, terms = oracle.gemv_q4_0_q8_int(blob, xq)
        y = gpu_q4_0(blob, oracle.q8_1_to_bytes(xq), 1)
    assert_within(y, y_ref, terms, "lm head fmt %d" % fmt)


def test_q4_0_padding_invariance_gpu():
    banner("q4_0 padding invariance")
    rows, n, in_dim = 500, 896, 1024
    blob = synth.q4_0_weights(synth.rng(3, 1), rows, in_dim)
    x = np.zeros(in_dim, np.float32)
    x[:n] = synth.activation(synth.rng(3, 0), n)
    y1 = gpu_q4_0(blob, x, 0)
    b2 = blob.copy()
    b2[:, 28:, 2:18] = np.random.default_rng(5).integers(0, 256, (rows, 4, 16), dtype=np.uint8)
    assert np.array_equal(y1, gpu_q4_0(b2, x, 0))


# ------------------------------------------------------------------ SwiGLU chain
def run_ffn(wg, wu, wd, xq_bytes, hidden, inter, with_gu=True):
    h = empty_f32(inter)
    hq = empty_bytes(rz.q8_1_nbytes(inter))
    y = empty_f32(hidden)
    gu = empty_f32(2 * inter) if with_gu else None
    rz.rz_swiglu_ffn_q4k(dev_bytes(wg), dev_bytes(wu), dev_bytes(wd), dev_bytes(xq_bytes), h, hq,
                         y, gu, hidden, inter)
    out = dict(h=host(h), hq=q8_host_bytes(hq, inter // 32), y=host(y))
    if with_gu:
        g_u = host(gu)
        out["g"], out["u"] = g_u[:inter], g_u[inter:]
    return out


@pytest.mark.parametrize("hidden,inter", [(256, 512), (512, 768), (1024, 2816), (4096, 14336)])
def test_swiglu_ffn_chain(hidden, inter):
    """Stage by stage:
      (i)   g, u within the GEMV bound of the oracle's g, u;
      (ii)  h within the bound propagated through silu(g) * u;
      (iii) h_q8 byte-equal to the oracle's Q8_1 of the GPU's own h; and against
            the oracle's h_q8 (of the oracle's h): d within the propagated bound,
            codes within one step, equal wherever the oracle's h/d is clear of a
            rounding tie;
      (iv)  y equals the standalone GPU GEMV over the GPU's h_q8 (bit-exact), the
            standalone down GEMV over the oracle's h_q8 is within the GEMV bound of
            the oracle, and the chain's y is within the GEMV bound plus the
            activation difference |W| . |x_hat_gpu - x_hat_oracle|."""
    banner("swiglu", hidden, inter)
    cid = 2 if (hidden, inter) == (4096, 14336) else 20 + hidden // 256
    wg = synth.q4k_weights(synth.rng(cid, synth.T_W0), inter, hidden)
    wu = synth.q4k_weights(synth.rng(cid, synth.T_W0 + 1), inter, hidden)
    wd = synth.q4k_weights(synth.rng(cid, synth.T_W0 + 2), hidden, inter)
    x = synth.activation(synth.rng(cid, synth.T_ACT), hidden)
    xq = oracle.quantize_q8_1(x)
    st = oracle.ffn_swiglu_q4k(wg, wu, wd, xq)
    got = run_ffn(wg, wu, wd, oracle.q8_1_to_bytes(xq), hidden, inter)

    # (i)
    assert_within(got["g"], st["g"], st["g_terms"], "gate")
    assert_within(got["u"], st["u"], st["u_terms"], "up")
    # (ii)
    tol_h = oracle.h_tolerance(st["g"], st["u"], st["tol_g"], st["tol_u"], st["h"])
    err_h = np.abs(got["h"].astype(np.float64) - st["h"])
    assert np.all(err_h <= tol_h), "h: %d outside, worst ratio %.3g" % (
        int((err_h > tol_h).sum()), float(np.max(err_h / tol_h)))
    # (iii) byte-exact: the oracle's Q8_1 of the GPU's own h (exactly one block
    # string is correct for given fp32 values)
    want_hq = oracle.q8_1_to_bytes(oracle.quantize_q8_1(got["h"], inter))
    bad = first_mismatch(got["hq"], want_hq)
    assert bad is None, "h_q8 differs from the oracle's quantize of the GPU's h: %r" % (bad,)
    # (iii) against the oracle's blocks
    d_gpu = got["hq"][:, 0:4].copy().view("<f4")[:, 0].astype(np.float64)
    q_gpu = got["hq"][:, 8:40].copy().view(np.int8).astype(np.int64)
    d_ref = st["h_q8"].d.astype(np.float64)
    q_ref = st["h_q8"].q.astype(np.int64)
    amax_tol = np.max(tol_h.reshape(-1, 32), axis=1)
    assert np.all(np.abs(d_gpu - d_ref) <= amax_tol / 127 + 4 * 2.0 ** -24 * d_ref)
    assert np.all(np.abs(q_gpu - q_ref) <= 1)
    ratio = st["h"].reshape(-1, 32) / np.where(d_ref > 0, d_ref, 1.0)[:, None]
    frac = np.abs(ratio - np.floor(ratio) - 0.5)
    margin = (tol_h.reshape(-1, 32) / np.where(d_ref > 0, d_ref, 1.0)[:, None]
              + np.abs(ratio) * (np.abs(d_gpu - d_ref) / np.where(d_ref > 0, d_ref, 1.0))[:, None]
              + 1e-4)
    clear = frac > margin
    assert np.array_equal(q_gpu[clear], q_ref[clear])
    # (iv)
    y_chain = gpu_q4k(wd, got["hq"])[0]
    assert np.array_equal(y_chain, got["y"])
    y_std = gpu_q4k(wd, oracle.q8_1_to_bytes(st["h_q8"]))[0]
    assert_within(y_std, st["y"], st["y_terms"], "down over oracle h_q8")
    xhat_gpu = (d_gpu[:, None] * q_gpu).reshape(-1)
    xhat_ref = oracle.dequantize_q8_1(st["h_q8"])
    w_abs = np.abs(oracle.dequantize_q4k(wd))
    extra = w_abs @ np.abs(xhat_gpu - xhat_ref)
    assert_within(got["y"], st["y"], st["y_terms"] + extra / oracle.GEMV_REL, "chain y")


def test_swiglu_zero_up_gives_zero_gpu():
    banner("swiglu zero up")
    hidden, inter = 512, 1024
    wg = synth.q4k_weights(synth.rng(5, 1), inter, hidden)
    wu = synth.q4k_weights(synth.rng(5, 2), inter, hidden, d_fixed=0.0, dmin_fixed=0.0)
    wd = synth.q4k_weights(synth.rng(5, 3), hidden, inter)
    xq = oracle.quantize_q8_1(synth.activation(synth.rng(5, 0), hidden))
    got = run_ffn(wg, wu, wd, oracle.q8_1_to_bytes(xq), hidden, inter)
    assert np.all(got["u"] == 0) and np.all(got["h"] == 0)
    assert not got["hq"].any() and np.all(got["y"] == 0)


def test_swiglu_optional_gu_pointer():
    banner("swiglu without gu")
    hidden, inter = 1024, 2048
    wg = synth.q4k_weights(synth.rng(6, 1), inter, hidden)
    wu = synth.q4k_weights(synth.rng(6, 2), inter, hidden)
    wd = synth.q4k_weights(synth.rng(6, 3), hidden, inter)
    xb = oracle.q8_1_to_bytes(oracle.quantize_q8_1(synth.activation(synth.rng(6, 0), hidden)))
    a = run_ffn(wg, wu, wd, xb, hidden, inter, with_gu=True)
    b = run_ffn(wg, wu, wd, xb, hidden, inter, with_gu=False)
    assert np.array_equal(a["h"], b["h"]) and np.array_equal(a["hq"], b["hq"])
    assert np.array_equal(a["y"], b["y"])


# ------------------------------------------------------------------ RMSNorm -> Q8_1
def gpu_rmsnorm_q8(x, gamma, eps, n_padded, with_normed=True):
    x2 = x if x.ndim == 2 else x[None, :]
    nt, n = x2.shape
    normed = empty_f32(nt * n) if with_normed else None
    xq = empty_bytes(rz.q8_1_nbytes(n_padded, nt))
    rz.rz_rmsnorm_q8_1(dev_f32(x2), dev_f32(gamma), eps, n, n_padded, nt, normed, xq)
    q = q8_host_bytes(xq, nt * n_padded // 32).reshape(nt, n_padded // 32, 40)
    return (host(normed).reshape(nt, n) if with_normed else None), q


def _norm_chain(n_padded):
    """Longest chain of dependent fp32 additions in the kernel's sum of squares.
    Rows of up to 16384 values: 4 values per 1024-value pass in each of 256
    threads, then 6 DPP levels inside a wave and 2 over the 4 wave sums; longer
    rows: 4 values per 4096-value pass in each of 1024 threads, 6 + 4 levels."""
    if n_padded <= 16384:
        return 4 * -(-n_padded // 1024) + 8
    return 4 * -(-n_padded // 4096) + 10


@pytest.mark.parametrize("n,n_padded,nt,scale", [
    (4096, 4096, 1, 1.0),       # the attention-projection input
    (896, 1024, 1, 1.0),        # 896-wide hidden state, padded
    (4096, 4096, 8, 1.0),       # 8 tokens
    (14336, 14336, 1, 1.0),
    (1000, 1024, 3, 1.0),       # ragged tail inside a block
    (1, 32, 1, 1.0),
    (33, 64, 2, 1.0),
    (20000, 20480, 1, 1.0),     # several 32-block passes
    (4096, 4096, 2, 1e-4),      # eps comparable to the mean square
    (4096, 4096, 1, 1e15),      # large values: the sum of squares near 1e34
])
def test_rmsnorm_q8_1_matches_oracle(n, n_padded, nt, scale):
    """Stage by stage: the normed values within the fp32 rounding bound of the
    float64 definition; the Q8_1 blocks byte-equal to the oracle's quantize of
    the GPU's own normed values; against the oracle's blocks of its own normed
    values, d within the propagated bound and every code within one step."""
    banner("rmsnorm_q8_1", n, n_padded, nt, scale)
    g = np.random.default_rng(n * 7 + nt)
    x = (synth.activation(g, n, nt) * np.float32(scale)).astype(np.float32)
    gamma = synth.norm_weights(np.random.default_rng(n + 1), n)
    eps = 1e-5
    normed, q = gpu_rmsnorm_q8(x, gamma, eps, n_padded)
    ref = oracle.rmsnorm(x, gamma, eps)
    tol = oracle.rmsnorm_tolerance(ref, _norm_chain(n_padded))
    err = np.abs(normed.astype(np.float64) - ref)
    assert np.all(err <= tol), "normed: %d outside, worst ratio %.3g" % (
        int((err > tol).sum()), float(np.max(err / tol)))
    # byte-exact: the oracle's Q8_1 of the GPU's own normed values
    want_gpu = oracle.q8_1_to_bytes(oracle.quantize_q8_1(normed, n_padded)).reshape(q.shape)
    bad = first_mismatch(q, want_gpu)
    assert bad is None, "Q8_1 differs from the oracle's quantize of the GPU's normed values: %r" % (bad,)
    # against the oracle's quantize of its own (float64 -> fp32) normed values
    want = oracle.quantize_q8_1(ref.astype(np.float32), n_padded)
    d_gpu = q[..., 0:4].copy().view("<f4")[..., 0].astype(np.float64).reshape(-1)
    q_gpu = q[..., 8:40].copy().view(np.int8).astype(np.int64).reshape(-1, 32)
    d_ref = want.d.astype(np.float64).reshape(-1)
    q_ref = want.q.astype(np.int64).reshape(-1, 32)
    tol_pad = np.zeros((nt, n_padded))
    tol_pad[:, :n] = tol + np.abs(ref) * 2.0 ** -24
    amax_tol = np.max(tol_pad.reshape(-1, 32), axis=1)
    assert np.all(np.abs(d_gpu - d_ref) <= amax_tol / 127 + 2 * 2.0 ** -24 * d_ref)
    assert np.all(np.abs(q_gpu - q_ref) <= 1)


def test_rmsnorm_q8_1_tokens_independent_and_optional_output():
    """Each token is normalised on its own (a batch equals its tokens one at a
    time, bit for bit), and skipping the normed output changes nothing."""
    banner("rmsnorm tokens")
    n = 4096
    x = synth.activation(np.random.default_rng(11), n, 5)
    gamma = synth.norm_weights(np.random.default_rng(12), n)
    normed, q = gpu_rmsnorm_q8(x, gamma, 1e-5, n)
    _, q_skip = gpu_rmsnorm_q8(x, gamma, 1e-5, n, with_normed=False)
    assert np.array_equal(q, q_skip)
    for t in (4, 0, 2):
        nt_, qt = gpu_rmsnorm_q8(x[t], gamma, 1e-5, n)
        assert np.array_equal(nt_[0], normed[t]) and np.array_equal(qt[0], q[t])


def test_rmsnorm_q8_1_degenerate_inputs():
    """All-zero tokens give zero values and all-zero blocks; a zero weight zeroes
    its value; a constant token of c gives c / sqrt(c^2 + eps) * gamma."""
    banner("rmsnorm degenerate")
    n = 512
    x = np.zeros((3, n), np.float32)
    x[1] = 3.0
    x[2] = synth.activation(np.random.default_rng(13), n)
    gamma = synth.norm_weights(np.random.default_rng(14), n)
    gamma[::7] = 0.0
    normed, q = gpu_rmsnorm_q8(x, gamma, 1e-5, n)
    assert np.all(normed[0] == 0) and not q[0].any()
    assert np.all(normed[1:, ::7] == 0)
    ref = oracle.rmsnorm(x[1], gamma, 1e-5)
    closed = 3.0 / np.sqrt(9.0 + 1e-5) * gamma.astype(np.float64)
    assert np.allclose(ref, closed, rtol=1e-15, atol=0)
    assert np.all(np.abs(normed[1] - closed) <= oracle.rmsnorm_tolerance(closed, _norm_chain(n)))


# ------------------------------------------------------------------ residual-add epilogue
def _one_pass(n_tokens, in_dim):
    """The row fits one pass of the kernel (so y = fl32(W x + r) exactly)."""
    return in_dim <= (16384 if n_tokens <= 2 else 4096)


def gpu_q4k_add(blob, xq_bytes, r, n_tokens, in_place=False):
    out_dim = blob.shape[0]
    rd = dev_f32(r.reshape(-1))
    y = rd if in_place else empty_f32(out_dim * n_tokens)
    rz.rz_q4k_q8_gemv_add(dev_bytes(blob), dev_bytes(xq_bytes), rd, y, out_dim,
                          blob.shape[1] * 256, n_tokens)
    return host(y).reshape(n_tokens, out_dim)


@pytest.mark.parametrize("out_dim,in_dim,nt", [
    (4096, 4096, 1),      # O projection of the attention workload
    (4096, 14336, 1),     # FFN down projection
    (300, 1024, 1),
    (37, 2048, 2),
    (100, 20480, 1),      # two column passes
    (513, 4096, 3),       # matrix cores, one pass
    (14336, 4096, 8),
    (1000, 14336, 8),     # matrix cores, four passes
])
def test_q4k_gemv_add(out_dim, in_dim, nt):
    """y = W x + r: bit-equal to fl32(rz_q4k_q8_gemv + r) when one pass covers
    the row, the same in place (r is y), and within the GEMV bound of the
    oracle with the residual counted as one more term."""
    banner("gemv_add", out_dim, in_dim, nt)
    cid = 40 + nt
    blob = synth.q4k_weights(synth.rng(cid, synth.T_W0), out_dim, in_dim)
    x = synth.activation(synth.rng(cid, synth.T_ACT), in_dim, nt)
    xq = oracle.quantize_q8_1(x, in_dim)
    xb = oracle.q8_1_to_bytes(xq)
    r = (synth.activation(synth.rng(cid, 7), out_dim, nt) * np.float32(3.0)).astype(np.float32)
    y = gpu_q4k_add(blob, xb, r, nt)
    y_in_place = gpu_q4k_add(blob, xb, r, nt, in_place=True)
    assert np.array_equal(y, y_in_place)
    if _one_pass(nt, in_dim):
        plain = gpu_q4k(blob, xb, nt)
        assert np.array_equal(y, (plain + r).astype(np.float32))
    y_ref, terms = oracle_q4k(blob, xq, nt)
    for t in range(nt):
        assert_within(y[t], oracle.residual_add(r[t], y_ref[t]), terms[t] + np.abs(r[t]),
                      "gemv_add token %d" % t)


def test_swiglu_ffn_add():
    """The FFN with the residual: h and h_q8 as without it, y bit-equal to
    fl32(y + r) of the plain chain (one pass: inter 14336), and in place."""
    hidden, inter = 4096, 14336
    banner("swiglu_add", hidden, inter)
    cid = 2
    wg = synth.q4k_weights(synth.rng(cid, synth.T_W0), inter, hidden)
    wu = synth.q4k_weights(synth.rng(cid, synth.T_W0 + 1), inter, hidden)
    wd = synth.q4k_weights(synth.rng(cid, synth.T_W0 + 2), hidden, inter)
    xb = oracle.q8_1_to_bytes(oracle.quantize_q8_1(synth.activation(synth.rng(cid, synth.T_ACT),
                                                                    hidden)))
    r = synth.activation(synth.rng(cid, 7), hidden)
    plain = run_ffn(wg, wu, wd, xb, hidden, inter, with_gu=False)
    dw = [dev_bytes(a) for a in (wg, wu, wd, xb)]
    for in_place in (False, True):
        h = empty_f32(inter)
        hq = empty_bytes(rz.q8_1_nbytes(inter))
        rd = dev_f32(r)
        y = rd if in_place else empty_f32(hidden)
        rz.rz_swiglu_ffn_q4k_add(*dw, h, hq, rd, y, None, hidden, inter)
        assert np.array_equal(host(h), plain["h"])
        assert np.array_equal(q8_host_bytes(hq, inter // 32), plain["hq"])
        assert np.array_equal(host(y), (plain["y"] + r).astype(np.float32))


# ------------------------------------------------------------------ Q4_K x fp32 activation
def gpu_q4k_xf32(blob, x, n=None):
    out_dim, nsb, _ = blob.shape
    n = x.shape[0] if n is None else n
    y = empty_f32(out_dim)
    rz.rz_q4k_gemv(dev_bytes(blob), dev_f32(x[:n]), n, y, out_dim, nsb * 256)
    return host(y)


def _padded(x, in_dim):
    xp = np.zeros(in_dim, np.float32)
    xp[:x.shape[0]] = x
    return xp


@pytest.mark.parametrize("out_dim,n,in_dim", [
    (1, 256, 256), (3, 200, 256), (64, 512, 512), (257, 1024, 1024), (300, 896, 1024),
    (37, 2048, 2048), (100, 4096, 4096), (65, 5000, 5120), (33, 14335, 14336),
    (8, 20480, 20480), (14336, 4096, 4096), (4096, 14336, 14336),
])
def test_q4k_gemv_xf32_matches_oracle(out_dim, n, in_dim):
    """rz_q4k_gemv within 1e-5 * terms + 1e-6 of the float64 definition, terms
    being the factored form's summands; one to five column chunks, ragged n
    (16-byte and dword activation loads), the full gate and down shapes."""
    banner("q4k_gemv_xf32", out_dim, n, in_dim)
    cid = 80 + in_dim // 256
    blob = synth.q4k_weights(synth.rng(cid, synth.T_W0), out_dim, in_dim)
    x = synth.activation(synth.rng(cid, synth.T_ACT), n)
    y = gpu_q4k_xf32(blob, x)
    y_ref, terms = oracle.gemv_q4k_f32(blob, _padded(x, in_dim))
    assert_within(y, y_ref, terms, "q4k_gemv fp32 x")


def _wide_activation(seed, n):
    """N(0,1) values scaled by 2^k, k uniform in -20..20, about 6% exact zeros."""
    g = np.random.default_rng(seed)
    x = g.standard_normal(n) * np.exp2(g.integers(-20, 21, n).astype(np.float64))
    x[g.random(n) < 0.06] = 0.0
    return x.astype(np.float32)


@pytest.mark.parametrize("out_dim,in_dim", [(300, 4096), (33, 14336), (1024, 1024)])
def test_q4k_gemv_xf32_wide_range_activation(out_dim, in_dim):
    """Activations spanning 2^-20 .. 2^20 with zeros: the 4-bit weights enter
    the fmas as fp16 denormals (q * 2^-24, high nibbles as 16 q * 2^-24 against
    activations prescaled by 2^-4), exact in this range; every output stays
    within the bound of the float64 definition."""
    banner("q4k_gemv_xf32 wide range", out_dim, in_dim)
    blob = synth.q4k_weights(synth.rng(96, in_dim), out_dim, in_dim)
    x = _wide_activation(97 + in_dim, in_dim)
    y = gpu_q4k_xf32(blob, x)
    y_ref, terms = oracle.gemv_q4k_f32(blob, x)
    assert_within(y, y_ref, terms, "q4k_gemv fp32 x, wide range")


@pytest.mark.parametrize("out_dim,in_dim", [(257, 1024), (9, 10240), (130, 4096)])
def test_q4_0_fp32_wide_range_activation(out_dim, in_dim):
    """The Q4_0 fp32-activation path on activations spanning 2^-20 .. 2^20 with
    zeros (its nibbles also enter the fmas as fp16 denormals, with the staged
    high-nibble activations prescaled by 2^-4): within the bound of the
    float64 definition."""
    banner("q4_0 fp32 wide range", out_dim, in_dim)
    blob = synth.q4_0_weights(synth.rng(98, in_dim), out_dim, in_dim)
    x = _wide_activation(99 + in_dim, in_dim)
    y = gpu_q4_0(blob, x, 0)
    y_ref, terms = oracle.gemv_q4_0_f32(blob, x)
    assert_within(y, y_ref, terms, "q4_0 fp32 x, wide range")


@pytest.mark.parametrize("out_dim,in_dim", [(5, 256), (64, 1024), (300, 4096), (40, 14336)])
def test_q4k_gemv_xf32_integer_exact_bit_exact(out_dim, in_dim):
    """d = dmin = 1 and small integer activations: every product and partial sum
    is an integer below 2**24, so the fp32 path must match the oracle exactly;
    this pins the element order of the fp32 activation on the GPU."""
    banner("q4k_gemv_xf32 integer", out_dim, in_dim)
    blob = synth.q4k_weights(synth.rng(90, 1), out_dim, in_dim, d_fixed=1.0, dmin_fixed=1.0)
    x = np.random.default_rng(91).integers(-8, 9, in_dim).astype(np.float32)
    y = gpu_q4k_xf32(blob, x)
    y_ref, _ = oracle.gemv_q4k_f32(blob, x)
    assert np.all(np.abs(y_ref) < 2 ** 24)
    mm = first_mismatch(y.astype(np.float64), y_ref)
    assert mm is None, "row %s gpu=%r oracle=%r (%d rows differ)" % mm


def test_q4k_gemv_xf32_padding_invariance():
    """Values past n read as zero: the same y as an explicitly zero-padded x,
    whatever the weight bytes in the padding hold."""
    banner("q4k_gemv_xf32 padding")
    blob = synth.q4k_weights(synth.rng(92, 1), 129, 1024)
    x = synth.activation(synth.rng(92, 0), 896)
    y1 = gpu_q4k_xf32(blob, x)
    y2 = gpu_q4k_xf32(blob, _padded(x, 1024))
    b2 = blob.copy()
    b2[:, 3, 16 + 64:] = np.random.default_rng(7).integers(0, 256, (129, 64), dtype=np.uint8)
    y3 = gpu_q4k_xf32(b2, x)
    assert np.array_equal(y1, y2) and np.array_equal(y1, y3)


def test_q4k_gemv_xf32_is_more_accurate_than_q8_1():
    """The comparison the fp32 path exists for, at 4096 -> 14336 against the
    float64 definition on the unquantized activation: the fp32 path is within
    its rounding bound, the Q8_1 path carries the activation's quantization
    error, which is far larger."""
    banner("fp32 vs Q8_1 accuracy")
    blob = synth.q4k_weights(synth.rng(2, synth.T_W0), 14336, 4096)
    x = synth.activation(synth.rng(2, synth.T_ACT), 4096)
    y_def, terms = oracle.gemv_q4k_f32(blob, x)
    y32 = gpu_q4k_xf32(blob, x)
    y8 = gpu_q4k(blob, gpu_quantize(x, 4096)[0])[0]
    e32 = np.abs(y32 - y_def) / terms
    e8 = np.abs(y8 - y_def) / terms
    print("[accuracy] max |y - y_def| / terms: fp32 x %.3g, Q8_1 x %.3g; median %.3g / %.3g"
          % (e32.max(), e8.max(), np.median(e32), np.median(e8)), flush=True)
    assert e32.max() <= 1e-5 and e8.max() > 10 * e32.max()


def run_ffn_f32(wg, wu, wd, x, hidden, inter, with_gu=True):
    h = empty_f32(inter)
    y = empty_f32(hidden)
    gu = empty_f32(2 * inter) if with_gu else None
    rz.rz_swiglu_ffn_q4k_f32(dev_bytes(wg), dev_bytes(wu), dev_bytes(wd), dev_f32(x), h, y, gu,
                             hidden, inter)
    out = dict(h=host(h), y=host(y))
    if with_gu:
        g_u = host(gu)
        out["g"], out["u"] = g_u[:inter], g_u[inter:]
    return out


@pytest.mark.parametrize("hidden,inter", [(256, 512), (512, 768), (1024, 2816), (4096, 14336)])
def test_swiglu_ffn_f32_chain(hidden, inter):
    """Stage by stage, as for the Q8_1 chain: g and u within the GEMV bound; h
    within the bound propagated through silu(g) * u; y bit-equal to rz_q4k_gemv
    over the GPU's own h, the standalone down GEMV over the oracle's h within
    the GEMV bound, and the chain's y within that bound plus |W| . |h_gpu - h|."""
    banner("swiglu fp32", hidden, inter)
    cid = 2 if (hidden, inter) == (4096, 14336) else 30 + hidden // 256
    wg = synth.q4k_weights(synth.rng(cid, synth.T_W0), inter, hidden)
    wu = synth.q4k_weights(synth.rng(cid, synth.T_W0 + 1), inter, hidden)
    wd = synth.q4k_weights(synth.rng(cid, synth.T_W0 + 2), hidden, inter)
    x = synth.activation(synth.rng(cid, synth.T_ACT), hidden)
    st = oracle.ffn_swiglu_q4k_f32(wg, wu, wd, x)
    got = run_ffn_f32(wg, wu, wd, x, hidden, inter)
    assert_within(got["g"], st["g"], st["g_terms"], "gate")
    assert_within(got["u"], st["u"], st["u_terms"], "up")
    tol_h = oracle.h_tolerance(st["g"], st["u"], st["tol_g"], st["tol_u"], st["h"])
    err_h = np.abs(got["h"].astype(np.float64) - st["h"])
    assert np.all(err_h <= tol_h), "h: %d outside, worst ratio %.3g" % (
        int((err_h > tol_h).sum()), float(np.max(err_h / tol_h)))
    assert np.array_equal(got["y"], gpu_q4k_xf32(wd, got["h"]))
    assert_within(gpu_q4k_xf32(wd, st["h32"]), st["y"], st["y_terms"], "down over oracle h")
    w_abs = np.abs(oracle.dequantize_q4k(wd))
    extra = w_abs @ np.abs(got["h"].astype(np.float64) - st["h32"].astype(np.float64))
    assert_within(got["y"], st["y"], st["y_terms"] + extra / oracle.GEMV_REL, "chain y")


def test_swiglu_ffn_f32_optional_gu_and_y_on_x():
    """Skipping gu changes nothing, and y may overwrite x."""
    banner("swiglu fp32 options")
    hidden, inter = 1024, 2048
    wg = synth.q4k_weights(synth.rng(33, 1), inter, hidden)
    wu = synth.q4k_weights(synth.rng(33, 2), inter, hidden)
    wd = synth.q4k_weights(synth.rng(33, 3), hidden, inter)
    x = synth.activation(synth.rng(33, 0), hidden)
    a = run_ffn_f32(wg, wu, wd, x, hidden, inter, with_gu=True)
    b = run_ffn_f32(wg, wu, wd, x, hidden, inter, with_gu=False)
    assert np.array_equal(a["h"], b["h"]) and np.array_equal(a["y"], b["y"])
    xd = dev_f32(x)
    h = empty_f32(inter)
    rz.rz_swiglu_ffn_q4k_f32(dev_bytes(wg), dev_bytes(wu), dev_bytes(wd), xd, h, xd, None,
                             hidden, inter)
    assert np.array_equal(host(xd), a["y"])


# ------------------------------------------------------------------ LM head epilogue
def gpu_lm_head(blob, x, x_format, bias, argmax=True):
    """(logits, idx, val) from rz_lm_head_q4_0; idx/val None without argmax."""
    torch = __import__("torch")
    out_dim, nb, _ = blob.shape
    in_dim = nb * 32
    logits = empty_f32(out_dim)
    xd = dev_f32(x) if x_format == 0 else dev_bytes(x)
    bd = dev_f32(bias) if bias is not None else None
    idx = torch.full((1,), -7, dtype=torch.int32, device="cuda") if argmax else None
    val = empty_f32(1) if argmax else None
    ws = None
    if argmax:
        ws = empty_bytes(rz.rz_lm_head_q4_0_workspace_bytes(out_dim, in_dim, x_format))
    rz.rz_lm_head_q4_0(dev_bytes(blob), xd, x_format, bd, logits, out_dim, in_dim, idx, val, ws)
    lg = host(logits)
    if not argmax:
        return lg, None, None
    return lg, int(host(idx)[0]), host(val)[0]


def _q4_0_one_pass(in_dim, x_format):
    """The row fits one column pass of the Q4_0 kernel (224 block pairs for fp32
    x, 256 for Q8_1 x), so the bias store gives fl32(W x + bias) exactly."""
    return in_dim <= (16384 if x_format == 1 else 14336)


def _check_lm_head(blob, x, x_format, bias, x_oracle):
    lg, idx, val = gpu_lm_head(blob, x, x_format, bias)
    # logits: fl32(plain GEMV + bias) for one pass (a longer row adds the bias
    # to its first pass), and the oracle bound with |bias| as a term
    plain = gpu_q4_0(blob, x, x_format)
    if bias is None or _q4_0_one_pass(blob.shape[1] * 32, x_format):
        want = plain if bias is None else (plain + bias).astype(np.float32)
        mm = first_mismatch(lg, want)
        assert mm is None, "logit %s fused=%r plain+bias=%r (%d differ)" % mm
    y_ref, terms = oracle.lm_head_q4_0(blob, x_oracle, bias, x_format)
    assert_within(lg, y_ref, terms, "lm head logits")
    # the greedy token: unique on the GPU's own logits (same fp32 values, same tie rule)
    assert idx == oracle.argmax_first(lg)
    assert np.float32(val).tobytes() == np.float32(lg[idx]).tobytes()
    # and a valid choice against the exact logits: within both tolerances of the true maximum
    tol = oracle.gemv_tolerance(terms)
    best = oracle.argmax_first(y_ref)
    assert y_ref[idx] >= y_ref[best] - tol[idx] - tol[best]
    return lg, idx


@pytest.mark.parametrize("fmt", [0, 1])
def test_lm_head_full_with_bias(fmt):
    """151936 x 1024 with an N(0, 1) output bias."""
    banner("lm head full", fmt)
    w = synth.WORKLOADS["lm_head_q4_0"]
    blob = synth.q4_0_weights(synth.rng(3, synth.T_W0), w["out_dim"], w["in_dim"])
    x = _padded(synth.activation(synth.rng(3, synth.T_ACT), w["n"]), w["in_dim"])
    bias = synth.activation(synth.rng(3, 8), w["out_dim"])
    if fmt == 0:
        _check_lm_head(blob, x, 0, bias, x)
    else:
        xq = oracle.quantize_q8_1(x)
        _check_lm_head(blob, oracle.q8_1_to_bytes(xq), 1, bias, xq)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("out_dim,in_dim", [(1, 64), (17, 64), (1000, 1024), (4097, 2048),
                                            (77, 8192), (300, 10240),   # fp32: 8-wave workgroups
                                            (3000, 16384), (50, 32768)])
def test_lm_head_shapes(fmt, out_dim, in_dim):
    """Ragged row counts, one and several column passes (the epilogue runs in
    the last), with and without bias."""
    banner("lm head", fmt, out_dim, in_dim)
    g = np.random.default_rng(out_dim + in_dim)
    blob = synth.q4_0_weights(synth.rng(60, 1), out_dim, in_dim)
    x = synth.activation(g, in_dim)
    bias = None if out_dim % 2 else synth.activation(g, out_dim)
    if fmt == 0:
        _check_lm_head(blob, x, 0, bias, x)
    else:
        xq = oracle.quantize_q8_1(x)
        _check_lm_head(blob, oracle.q8_1_to_bytes(xq), 1, bias, xq)


def test_lm_head_ties_and_negative_logits():
    """Zero weights make the logits equal to the bias exactly: equal largest
    values at rows 5000 and 100000 give 5000; an all-equal bias gives 0; all
    negative logits still give the largest."""
    banner("lm head ties")
    rows, in_dim = 151936, 1024
    blob = synth.q4_0_weights(synth.rng(61, 1), rows, in_dim, d_fixed=0.0)
    x = synth.activation(synth.rng(61, 0), in_dim)
    bias = -np.abs(synth.activation(synth.rng(61, 2), rows)) - 1.0
    bias[100000] = bias[5000] = -0.25
    lg, idx, val = gpu_lm_head(blob, x, 0, bias)
    assert np.array_equal(lg, bias) and idx == 5000 and val == np.float32(-0.25)
    lg, idx, val = gpu_lm_head(blob, x, 0, np.full(rows, 3.5, np.float32))
    assert idx == 0 and val == np.float32(3.5)
    lg, idx, val = gpu_lm_head(blob, x, 0, None)
    assert idx == 0 and np.all(lg == 0)


def test_lm_head_optional_outputs_and_workspace_reuse():
    """Only the index, only the value, no argmax at all, and one workspace used
    by two calls of different sizes in a row (it holds no state)."""
    banner("lm head options")
    torch = __import__("torch")
    blob = synth.q4_0_weights(synth.rng(62, 1), 20000, 1024)
    x = synth.activation(synth.rng(62, 0), 1024)
    lg_full, idx_full, val_full = gpu_lm_head(blob, x, 0, None)
    ws = empty_bytes(rz.rz_lm_head_q4_0_workspace_bytes(20000, 1024, 0))
    xd, wd = dev_f32(x), dev_bytes(blob)
    logits = empty_f32(20000)
    idx = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    val = empty_f32(1)
    rz.rz_lm_head_q4_0(wd, xd, 0, None, logits, 20000, 1024, idx, None, ws)
    assert int(host(idx)[0]) == idx_full
    rz.rz_lm_head_q4_0(wd, xd, 0, None, logits, 20000, 1024, None, val, ws)
    assert host(val)[0] == val_full
    small = blob[:777]
    rz.rz_lm_head_q4_0(dev_bytes(small), xd, 0, None, logits, 777, 1024, idx, val, ws)
    assert int(host(idx)[0]) == oracle.argmax_first(host(logits)[:777])
    rz.rz_lm_head_q4_0(wd, xd, 0, None, logits, 20000, 1024, None, None, None)
    assert np.array_equal(host(logits), lg_full)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("out_dim,in_dim", [(300, 1024), (50, 32768), (129, 20480)])
def test_lm_head_bias_is_logits(fmt, out_dim, in_dim):
    """The bias may be the logits buffer itself: the same logits and greedy
    token as with a separate bias, bit for bit, with one column pass and with
    several (the bias enters the first pass, before the buffer is written)."""
    banner("lm head bias aliased", fmt, out_dim, in_dim)
    torch = __import__("torch")
    blob = synth.q4_0_weights(synth.rng(63, in_dim), out_dim, in_dim)
    x = synth.activation(synth.rng(63, 1), in_dim)
    xin = x if fmt == 0 else oracle.q8_1_to_bytes(oracle.quantize_q8_1(x))
    bias = synth.activation(synth.rng(63, 2), out_dim)
    lg, idx, val = gpu_lm_head(blob, xin, fmt, bias)
    wd = dev_bytes(blob)
    xd = dev_f32(xin) if fmt == 0 else dev_bytes(xin)
    both = dev_f32(bias)
    i2 = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    v2 = empty_f32(1)
    ws = empty_bytes(rz.rz_lm_head_q4_0_workspace_bytes(out_dim, in_dim, fmt))
    rz.rz_lm_head_q4_0(wd, xd, fmt, both, both, out_dim, in_dim, i2, v2, ws)
    assert np.array_equal(host(both).view(np.uint32), lg.view(np.uint32))
    assert int(host(i2)[0]) == idx and host(v2)[0] == val


# ------------------------------------------------------------------ top-k
def gpu_topk(values, k, want_idx=True, want_val=True):
    torch = __import__("torch")
    n = values.size
    idx = torch.full((k,), -7, dtype=torch.int32, device="cuda") if want_idx else None
    val = empty_f32(k) if want_val else None
    ws = empty_bytes(rz.rz_topk_f32_workspace_bytes(n, k))
    rz.rz_topk_f32(dev_f32(values), n, k, idx, val, ws)
    return (host(idx) if want_idx else None), (host(val) if want_val else None)


def _topk_values(kind, n, seed):
    g = np.random.default_rng(seed)
    if kind == "normal":        # logits-like, all distinct with high probability
        return g.standard_normal(n).astype(np.float32)
    if kind == "ties":          # seven values only: long runs of equal values
        return g.integers(-3, 4, n).astype(np.float32)
    if kind == "zeros":         # -0 and +0 mixed under a few negatives: ties across signs
        v = np.where(g.random(n) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        v[g.random(n) < 0.1] = -1.0
        return v
    if kind == "ulps":          # 1 + j ulp, j < 4096: keys differ in their low 12 bits only
        return (1.0 + g.integers(0, 4096, n) * 2.0 ** -23).astype(np.float32)
    if kind == "ascending":     # the largest values in the last slice
        return np.arange(n, dtype=np.float32) * np.float32(0.5)
    if kind == "descending":
        return -np.arange(n, dtype=np.float32)
    raise ValueError(kind)


def _check_topk(values, k):
    idx, val = gpu_topk(values, k)
    want_i, want_v = oracle.topk_first(values, k)
    mm = first_mismatch(idx, want_i.astype(np.int32))
    assert mm is None, "topk index %s gpu=%r oracle=%r (%d differ)" % mm
    # the values bit for bit (the sign of a zero included)
    assert np.array_equal(val.view(np.uint32), want_v.astype(np.float32).view(np.uint32))


_TOPK_CASES = [(n, k) for n in (1, 7, 128, 1000, 2048, 2049, 4097, 20000, 151936, 262144)
               for k in (1, 5, 40, 128) if k <= n]
# the merge's shape changes at 2048, 4096 and 8192 candidates (slices x k):
# exactly each, and one slice more
_TOPK_CASES += [(n, 128) for n in (32768, 32769, 65536, 65537, 131072, 131073)]


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "ulps", "ascending", "descending"])
@pytest.mark.parametrize("n,k", _TOPK_CASES)
def test_topk_matches_oracle(kind, n, k):
    """One slice (n up to 2048, padded), several slices with a ragged last one,
    128 slices of 2048 at k = 128 (16384 candidates, the merge's capacity),
    and candidate counts on both sides of each change of the merge's shape:
    indices and values equal to the oracle's."""
    banner("topk", kind, n, k)
    _check_topk(_topk_values(kind, n, n * 131 + k), k)


def _topk_random_cases(count=40, seed=2024):
    g = np.random.default_rng(seed)
    kinds = ("normal", "ties", "zeros", "ulps", "ascending", "descending", "heavy")
    cases = []
    while len(cases) < count:
        n = int(np.exp(g.uniform(0, np.log(200000))))
        k = int(g.integers(1, min(n, 128) + 1))
        if rz.rz_topk_f32_workspace_bytes(n, k) == 0:
            continue
        cases.append((n, k, kinds[int(g.integers(len(kinds)))], int(g.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("n,k,kind,seed", _topk_random_cases())
def test_topk_random_shapes(n, k, kind, seed):
    """Seeded random sizes (log-uniform n up to 200000, k up to 128) and value
    patterns, including heavy-tailed values (a Cauchy draw, so the keys span
    many binades) and many equal values: indices and values equal to the
    oracle's."""
    banner("topk random", n, k, kind, seed)
    if kind == "heavy":
        v = np.random.default_rng(seed).standard_cauchy(n).astype(np.float32)
        v[~np.isfinite(v)] = 0.0
    else:
        v = _topk_values(kind, n, seed)
    _check_topk(v, k)


def test_topk_optional_outputs_and_workspace_reuse():
    """Only indices, only values, and one workspace used by calls of different
    sizes in a row (it holds no state)."""
    banner("topk options")
    torch = __import__("torch")
    v = _topk_values("normal", 151936, 70)
    want_i, want_v = oracle.topk_first(v, 40)
    i_only, _ = gpu_topk(v, 40, want_val=False)
    _, v_only = gpu_topk(v, 40, want_idx=False)
    assert np.array_equal(i_only, want_i) and np.array_equal(v_only, want_v)
    ws = empty_bytes(rz.rz_topk_f32_workspace_bytes(262144, 128))
    idx = torch.full((128,), -7, dtype=torch.int32, device="cuda")
    for n, k in ((262144, 128), (5000, 3), (151936, 40)):
        vals = _topk_values("ties", n, n)
        rz.rz_topk_f32(dev_f32(vals), n, k, idx, None, ws)
        assert np.array_equal(host(idx)[:k], oracle.topk_first(vals, k)[0])


@pytest.mark.parametrize("n,k", [(524288, 64), (1 << 20, 32), (1 << 24, 1), (1 << 24, 2)])
def test_topk_planted_at_largest_sizes(n, k):
    """Sizes the oracle's sort would take minutes over: values drawn from
    [-1, 1), then k entries set above 1 at spread-out positions (two of them
    equal, so their order is by index).  The top k are exactly those entries,
    largest first."""
    banner("topk planted", n, k)
    g = np.random.default_rng(n + k)
    v = (g.random(n, dtype=np.float32) * 2 - 1).astype(np.float32)
    pos = np.sort(g.choice(n, size=k, replace=False))
    planted = 2.0 + np.arange(k, dtype=np.float32)
    planted[-1] = planted[0] if k > 1 else planted[-1]   # a tie between the first and last position
    v[pos] = planted
    order = sorted(range(k), key=lambda j: (-float(planted[j]), int(pos[j])))
    want_i = pos[order].astype(np.int32)
    idx, val = gpu_topk(v, k)
    assert np.array_equal(idx, want_i), (idx[:8], want_i[:8])
    assert np.array_equal(val, v[want_i])


def test_topk_merge_capacity_boundaries():
    """The largest n the merge takes at k = 128 and 64 (16384 candidates) and
    the rejection one value beyond."""
    banner("topk capacity")
    for n, k in ((262144, 128), (524288, 64)):
        assert rz.rz_topk_f32_workspace_bytes(n, k) == 16384 * 8
        assert rz.rz_topk_f32_workspace_bytes(n + 1, k) == 0
        with pytest.raises(rz.RzError):
            rz.rz_topk_f32(dev_f32(np.zeros(n + 1, np.float32)), n + 1, k,
                           empty_f32(k), None, empty_bytes(1 << 17))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("out_dim,in_dim,k", [(7, 64, 7), (1000, 1024, 40), (3000, 16384, 128),
                                              (4100, 32768, 5)])
def test_lm_head_topk_shapes(fmt, out_dim, in_dim, k):
    """Small vocabularies (k = out_dim), one column pass and several (the
    selection runs on the finished logits): logits bit-equal to
    rz_lm_head_q4_0's, the top k equal to the oracle's selection over them."""
    banner("lm head topk", fmt, out_dim, in_dim, k)
    torch = __import__("torch")
    blob = synth.q4_0_weights(synth.rng(64, in_dim), out_dim, in_dim)
    x = synth.activation(synth.rng(64, 1), in_dim)
    xin = x if fmt == 0 else oracle.q8_1_to_bytes(oracle.quantize_q8_1(x))
    bias = synth.activation(synth.rng(64, 2), out_dim)
    lg, _, _ = gpu_lm_head(blob, xin, fmt, bias)
    xd = dev_f32(xin) if fmt == 0 else dev_bytes(xin)
    logits = empty_f32(out_dim)
    idx = torch.full((k,), -7, dtype=torch.int32, device="cuda")
    val = empty_f32(k)
    ws = empty_bytes(rz.rz_topk_f32_workspace_bytes(out_dim, k))
    rz.rz_lm_head_q4_0_topk(dev_bytes(blob), xd, fmt, dev_f32(bias), logits, out_dim, in_dim, k,
                            idx, val, ws)
    got = host(logits)
    assert np.array_equal(got.view(np.uint32), lg.view(np.uint32))
    want_i, want_v = oracle.topk_first(got, k)
    assert np.array_equal(host(idx), want_i.astype(np.int32))
    assert np.array_equal(host(val).view(np.uint32), want_v.view(np.uint32))


@pytest.mark.parametrize("fmt", [0, 1])
def test_lm_head_topk_full(fmt):
    """151936 x 1024 with bias: the logits bit-equal to rz_lm_head_q4_0's, the
    top 40 equal to the oracle's selection over those logits, and k = 1 the
    greedy token."""
    banner("lm head topk", fmt)
    torch = __import__("torch")
    w = synth.WORKLOADS["lm_head_q4_0"]
    out_dim, in_dim = w["out_dim"], w["in_dim"]
    blob = synth.q4_0_weights(synth.rng(3, synth.T_W0), out_dim, in_dim)
    x = _padded(synth.activation(synth.rng(3, synth.T_ACT), w["n"]), in_dim)
    xin = x if fmt == 0 else oracle.q8_1_to_bytes(oracle.quantize_q8_1(x))
    bias = synth.activation(synth.rng(3, 8), out_dim)
    lg, best, best_v = gpu_lm_head(blob, xin, fmt, bias)
    wd, bd = dev_bytes(blob), dev_f32(bias)
    xd = dev_f32(xin) if fmt == 0 else dev_bytes(xin)
    for k in (1, 40, 128):
        logits = empty_f32(out_dim)
        idx = torch.full((k,), -7, dtype=torch.int32, device="cuda")
        val = empty_f32(k)
        ws = empty_bytes(rz.rz_topk_f32_workspace_bytes(out_dim, k))
        rz.rz_lm_head_q4_0_topk(wd, xd, fmt, bd, logits, out_dim, in_dim, k, idx, val, ws)
        got = host(logits)
        assert np.array_equal(got.view(np.uint32), lg.view(np.uint32))
        want_i, want_v = oracle.topk_first(got, k)
        assert np.array_equal(host(idx), want_i.astype(np.int32))
        assert np.array_equal(host(val).view(np.uint32), want_v.view(np.uint32))
        assert int(host(idx)[0]) == best and host(val)[0] == best_v


@pytest.mark.parametrize("hidden,inter", [(256, 16384), (16384, 256)])
def test_gelu_ffn_bias_is_output(hidden, inter):
    """up_bias may be h and down_bias may be y: the same h and y as with
    separate biases, bit for bit, also where the projection runs in two column
    passes (inter 16384 for the down projection, hidden 16384 for the up)."""
    banner("gelu ffn bias aliased", hidden, inter)
    wu = synth.q4_0_weights(synth.rng(64, 1), inter, hidden)
    wd = synth.q4_0_weights(synth.rng(64, 2), hidden, inter)
    x = synth.activation(synth.rng(64, 0), hidden)
    ub = synth.activation(synth.rng(64, 3), inter)
    db = synth.activation(synth.rng(64, 4), hidden)
    dwu, dwd, xd = dev_bytes(wu), dev_bytes(wd), dev_f32(x)
    h, y = empty_f32(inter), empty_f32(hidden)
    rz.rz_gelu_ffn_q4_0(dwu, dwd, xd, dev_f32(ub), dev_f32(db), h, y, hidden, inter)
    h2, y2 = dev_f32(ub), dev_f32(db)
    rz.rz_gelu_ffn_q4_0(dwu, dwd, xd, h2, y2, h2, y2, hidden, inter)
    assert np.array_equal(host(h2).view(np.uint32), host(h).view(np.uint32)), "h"
    assert np.array_equal(host(y2).view(np.uint32), host(y).view(np.uint32)), "y"
    st = oracle.ffn_gelu_q4_0(wu, wd, x, ub, db)
    tol_h = oracle.gelu_h_tolerance(st["u"], st["tol_u"], st["h"])
    assert np.all(np.abs(host(h).astype(np.float64) - st["h"]) <= tol_h)


# ------------------------------------------------------------------ GELU FFN (Q4_0)
def gpu_q4_0_bias(blob, x, bias):
    """W x + bias through rz_lm_head_q4_0 (no argmax): the GEMV and bias stage
    the GELU FFN runs, for the staged checks."""
    out_dim, nb, _ = blob.shape
    y = empty_f32(out_dim)
    rz.rz_lm_head_q4_0(dev_bytes(blob), dev_f32(x), 0, dev_f32(bias) if bias is not None else None,
                       y, out_dim, nb * 32)
    return host(y)


@pytest.mark.parametrize("hidden,inter,biases", [(64, 64, True), (256, 512, False),
                                                 (1024, 4096, True), (512, 16384, True),
                                                 (2560, 10240, True)])
def test_gelu_ffn_chain(hidden, inter, biases):
    """Stage by stage: h within the bound propagated through GELU from the up
    projection's GEMV bound; y bit-equal to the same GEMV + bias over the GPU's
    own h; that GEMV over the oracle's h within the bound; the chain's y within
    the bound plus |W| . |h_gpu - h|."""
    banner("gelu ffn", hidden, inter, biases)
    cid = 5 if (hidden, inter) == (2560, 10240) else 40 + hidden // 64
    wu = synth.q4_0_weights(synth.rng(cid, synth.T_W0), inter, hidden)
    wd = synth.q4_0_weights(synth.rng(cid, synth.T_W0 + 1), hidden, inter)
    x = synth.activation(synth.rng(cid, synth.T_ACT), hidden)
    ub = synth.activation(synth.rng(cid, 7), inter) if biases else None
    db = synth.activation(synth.rng(cid, 8), hidden) if biases else None
    st = oracle.ffn_gelu_q4_0(wu, wd, x, ub, db)
    h = empty_f32(inter)
    y = empty_f32(hidden)
    rz.rz_gelu_ffn_q4_0(dev_bytes(wu), dev_bytes(wd), dev_f32(x),
                        dev_f32(ub) if biases else None, dev_f32(db) if biases else None,
                        h, y, hidden, inter)
    h_gpu, y_gpu = host(h), host(y)
    assert_within(gpu_q4_0_bias(wu, x, ub), st["u"], st["u_terms"], "up + bias")
    tol_h = oracle.gelu_h_tolerance(st["u"], st["tol_u"], st["h"])
    err_h = np.abs(h_gpu.astype(np.float64) - st["h"])
    assert np.all(err_h <= tol_h), "h: %d outside, worst ratio %.3g" % (
        int((err_h > tol_h).sum()), float(np.max(err_h / tol_h)))
    assert np.array_equal(y_gpu, gpu_q4_0_bias(wd, h_gpu, db))
    assert_within(gpu_q4_0_bias(wd, st["h32"], db), st["y"], st["y_terms"], "down over oracle h")
    extra = np.abs(oracle.dequantize_q4_0(wd)) @ np.abs(h_gpu.astype(np.float64) -
                                                       st["h32"].astype(np.float64))
    assert_within(y_gpu, st["y"], st["y_terms"] + extra / oracle.GEMV_REL, "chain y")


def _rand_cases(seed, count, draw):
    g = np.random.default_rng(seed)
    return [draw(g) for _ in range(count)]


def _draw_swiglu(g):
    while True:
        hidden, inter = 256 * int(g.integers(1, 17)), 256 * int(g.integers(1, 41))
        if hidden * inter <= 8_000_000:
            return hidden, inter


@pytest.mark.parametrize("hidden,inter", _rand_cases(91, 10, _draw_swiglu))
def test_swiglu_ffn_chain_random_shapes(hidden, inter):
    """The staged SwiGLU checks of test_swiglu_ffn_chain on seeded random
    hidden and intermediate sizes."""
    test_swiglu_ffn_chain(hidden, inter)


def _draw_rmsnorm(g):
    n = int(np.exp(g.uniform(0, np.log(20480))))
    n_padded = 32 * ((n + 31) // 32) + 32 * int(g.integers(0, 3))
    return n, min(n_padded, 20480), int(g.integers(1, 5)), float(10.0 ** g.integers(-3, 4))


@pytest.mark.parametrize("n,n_padded,nt,scale", _rand_cases(92, 12, _draw_rmsnorm))
def test_rmsnorm_q8_1_random_shapes(n, n_padded, nt, scale):
    """The checks of test_rmsnorm_q8_1_matches_oracle on seeded random lengths,
    paddings, token counts and scales."""
    test_rmsnorm_q8_1_matches_oracle(n, n_padded, nt, scale)


def _draw_gelu(g):
    while True:
        hidden, inter = 64 * int(g.integers(1, 41)), 64 * int(g.integers(1, 257))
        if hidden * inter <= 8_000_000:
            return hidden, inter, bool(g.integers(0, 2))


@pytest.mark.parametrize("hidden,inter,biases", _rand_cases(93, 10, _draw_gelu))
def test_gelu_ffn_chain_random_shapes(hidden, inter, biases):
    """The staged GELU FFN checks of test_gelu_ffn_chain on seeded random sizes,
    with and without biases."""
    test_gelu_ffn_chain(hidden, inter, biases)


def _draw_multi(g):
    k = int(g.integers(1, 9))
    in_dim = 256 * int(g.integers(1, 65))
    outs = [int(np.exp(g.uniform(0, np.log(700)))) for _ in range(k)]
    return int(g.integers(1, 3)), outs, in_dim


@pytest.mark.parametrize("n_tokens,out_dims,in_dim", _rand_cases(94, 12, _draw_multi))
def test_q4k_multi_random_shapes(n_tokens, out_dims, in_dim):
    """The checks of test_q4k_multi_matches_single_calls on seeded random
    matrix counts, row counts and row lengths."""
    test_q4k_multi_matches_single_calls(n_tokens, out_dims, in_dim)


def _draw_lm_head(g):
    while True:
        out_dim = int(np.exp(g.uniform(0, np.log(30000))))
        in_dim = 64 * int(g.integers(1, 401))
        if out_dim * in_dim <= 12_000_000:
            return out_dim, in_dim, int(g.integers(0, 2)), bool(g.integers(0, 2)), int(g.integers(1 << 30))


@pytest.mark.parametrize("out_dim,in_dim,fmt,with_bias,seed", _rand_cases(95, 14, _draw_lm_head))
def test_lm_head_random_shapes(out_dim, in_dim, fmt, with_bias, seed):
    """The LM head with and without bias, both activation formats, on seeded
    random vocabulary sizes and row lengths (up to 25600 values: several
    column passes): logits and greedy token as in test_lm_head_shapes."""
    banner("lm head random", fmt, out_dim, in_dim, with_bias)
    g = np.random.default_rng(seed)
    blob = synth.q4_0_weights(synth.rng(96, seed), out_dim, in_dim)
    x = synth.activation(g, in_dim)
    bias = synth.activation(g, out_dim) if with_bias else None
    if fmt == 0:
        _check_lm_head(blob, x, 0, bias, x)
    else:
        xq = oracle.quantize_q8_1(x)
        _check_lm_head(blob, oracle.q8_1_to_bytes(xq), 1, bias, xq)


def test_gelu_ffn_zero_up_weights():
    """Zero up weights: h = gelu(up_bias) exactly as the oracle rounds it, up to
    the device exp; with no up bias h is exactly 0 and y is the down bias."""
    banner("gelu ffn zero up")
    hidden, inter = 256, 1024
    wu = synth.q4_0_weights(synth.rng(45, 1), inter, hidden, d_fixed=0.0)
    wd = synth.q4_0_weights(synth.rng(45, 2), hidden, inter)
    x = synth.activation(synth.rng(45, 0), hidden)
    db = synth.activation(synth.rng(45, 3), hidden)
    h = empty_f32(inter)
    y = empty_f32(hidden)
    rz.rz_gelu_ffn_q4_0(dev_bytes(wu), dev_bytes(wd), dev_f32(x), None, dev_f32(db), h, y,
                        hidden, inter)
    assert np.all(host(h) == 0) and np.array_equal(host(y), db)
    ub = (4.0 * synth.activation(synth.rng(45, 4), inter)).astype(np.float32)
    rz.rz_gelu_ffn_q4_0(dev_bytes(wu), dev_bytes(wd), dev_f32(x), dev_f32(ub), dev_f32(db), h, y,
                        hidden, inter)
    ref = oracle.gelu(ub.astype(np.float64))
    assert np.all(np.abs(host(h) - ref) <= 8 * 2.0 ** -24 * np.abs(ref) + 1e-6)


# ------------------------------------------------------------------ errors on device tensors
def test_binding_errors_on_gpu():
    banner("binding errors")
    t = dev_f32(np.zeros(64, np.float32))
    with pytest.raises(rz.RzError):
        rz.rz_q4k_q8_gemv(t, t, t, 1, 100, 1)
    with pytest.raises(ValueError):
        rz.rz_q4k_q8_gemv(t, t, t, 1, 256, 1)     # buffers too small for the shape


# ------------------------------------------------------------------ minimum alignments
def _at(arr_or_n, shift: int, dtype="f32"):
    """A device buffer whose first byte sits `shift` bytes past a 256-byte
    boundary: a copy of a numpy array, or (given a size) an output filled
    with a marker.  Its neighbours inside the backing allocation are never
    touched by a correct kernel."""
    import torch
    if isinstance(arr_or_n, int):
        n = arr_or_n
        src = None
    else:
        src = np.ascontiguousarray(arr_or_n)
        n = src.size if dtype == "f32" else src.nbytes
    esize = 4 if dtype == "f32" else 1
    nbytes = n * esize
    raw = torch.full((nbytes + 512,), 0xA5, dtype=torch.uint8, device="cuda")
    base = (-raw.data_ptr()) % 256
    view = raw[base + shift: base + shift + nbytes]
    if dtype == "f32":
        view = view.view(torch.float32)
    if src is not None:
        host_t = torch.from_numpy(src.reshape(-1).view(np.uint8).copy() if dtype != "f32"
                                  else src.astype(np.float32).reshape(-1).copy())
        view.copy_(host_t.to("cuda"))
    else:
        if dtype == "f32":
            view.fill_(float("nan"))
    assert view.data_ptr() % 256 == shift
    return view


def _bits(t):
    return host(t).view(np.uint8).copy()


def _run_both(call, aligned_args, shifted_args, outs_a, outs_s, what):
    call(*aligned_args)
    call(*shifted_args)
    for k, (a, b) in enumerate(zip(outs_a, outs_s)):
        assert np.array_equal(_bits(a), _bits(b)), "%s: output %d differs at minimum alignment" % (what, k)


def test_minimum_alignments_bit_identical():
    """Every entry point on buffers at exactly the alignments include/rz.h
    requires (Q4_K and Q8_1 16 bytes, Q4_0 4, fp32 4 -- 16 for the Q4_0 and
    GELU activations) gives the same bytes as on 256-byte aligned buffers."""
    banner("minimum alignments")
    g = synth.rng(70, 1)
    # Q8_1 quantize and RMSNorm
    x = synth.activation(synth.rng(70, 0), 4096, 2)
    gam = synth.norm_weights(synth.rng(70, 2), 4096)
    qa, qs = _at(2 * 128 * 40, 0, "u8"), _at(2 * 128 * 40, 16, "u8")
    _run_both(lambda xx, q: rz.rz_q8_1_quantize(xx, 4096, 4096, 2, q),
              (_at(x, 0), qa), (_at(x, 4), qs), [qa], [qs], "quantize")
    na, ns = _at(2 * 4096, 0), _at(2 * 4096, 4)
    qa, qs = _at(2 * 128 * 40, 0, "u8"), _at(2 * 128 * 40, 16, "u8")
    _run_both(lambda xx, gg, nn, q: rz.rz_rmsnorm_q8_1(xx, gg, 1e-5, 4096, 4096, 2, nn, q),
              (_at(x, 0), _at(gam, 0), na, qa), (_at(x, 4), _at(gam, 4), ns, qs),
              [na, qa], [ns, qs], "rmsnorm")
    # Q4_K x Q8_1 GEMV: two-slot rows, seven-slot rows, two tokens, eight tokens (matrix cores)
    for out_dim, in_dim, nt in [(1000, 4096, 1), (300, 14336, 1), (129, 4096, 2), (77, 4096, 8)]:
        w = synth.q4k_weights(synth.rng(71, out_dim), out_dim, in_dim)
        xq = oracle.q8_1_to_bytes(oracle.quantize_q8_1(synth.activation(synth.rng(71, 0), in_dim, nt), in_dim))
        ya, ys = _at(nt * out_dim, 0), _at(nt * out_dim, 4)
        _run_both(lambda ww, q, yy: rz.rz_q4k_q8_gemv(ww, q, yy, out_dim, in_dim, nt),
                  (_at(w, 0, "u8"), _at(xq, 0, "u8"), ya), (_at(w, 16, "u8"), _at(xq, 16, "u8"), ys),
                  [ya], [ys], "gemv %dx%d nt %d" % (out_dim, in_dim, nt))
        r = synth.activation(synth.rng(71, 5), out_dim, nt)
        ya, ys = _at(nt * out_dim, 0), _at(nt * out_dim, 4)
        _run_both(lambda ww, q, rr, yy: rz.rz_q4k_q8_gemv_add(ww, q, rr, yy, out_dim, in_dim, nt),
                  (_at(w, 0, "u8"), _at(xq, 0, "u8"), _at(r, 0), ya),
                  (_at(w, 16, "u8"), _at(xq, 16, "u8"), _at(r, 4), ys), [ya], [ys], "gemv add")
    # fused quantize + GEMV (16-byte and dword activation loads) and the fp32-x GEMV
    w = synth.q4k_weights(synth.rng(72, 1), 500, 4096)
    xf = synth.activation(synth.rng(72, 0), 4096)
    for n in (4096, 4093):
        ya, ys = _at(500, 0), _at(500, 4)
        qa, qs = _at(128 * 40, 0, "u8"), _at(128 * 40, 16, "u8")
        _run_both(lambda ww, xx, q, yy: rz.rz_q4k_q8_gemv_f32(ww, xx, n, q, yy, 500, 4096),
                  (_at(w, 0, "u8"), _at(xf[:n], 0), qa, ya), (_at(w, 16, "u8"), _at(xf[:n], 4), qs, ys),
                  [ya, qa], [ys, qs], "fused n %d" % n)
        ya, ys = _at(500, 0), _at(500, 4)
        _run_both(lambda ww, xx, yy: rz.rz_q4k_gemv(ww, xx, n, yy, 500, 4096),
                  (_at(w, 0, "u8"), _at(xf[:n], 0), ya), (_at(w, 16, "u8"), _at(xf[:n], 4), ys),
                  [ya], [ys], "fp32-x gemv n %d" % n)
    # several matrices in one launch
    shapes = [(300, 4096), (64, 4096), (129, 4096)]
    ws = [synth.q4k_weights(synth.rng(73, k), o, i) for k, (o, i) in enumerate(shapes)]
    xq = oracle.q8_1_to_bytes(oracle.quantize_q8_1(synth.activation(synth.rng(73, 9), 4096), 4096))
    yas = [_at(o, 0) for o, _ in shapes]
    yss = [_at(o, 4) for o, _ in shapes]
    rz.rz_q4k_q8_gemv_multi([_at(w_, 0, "u8") for w_ in ws], _at(xq, 0, "u8"), yas, [o for o, _ in shapes], 4096)
    rz.rz_q4k_q8_gemv_multi([_at(w_, 16, "u8") for w_ in ws], _at(xq, 16, "u8"), yss, [o for o, _ in shapes], 4096)
    for a_, b_ in zip(yas, yss):
        assert np.array_equal(_bits(a_), _bits(b_)), "multi differs at minimum alignment"
    # SwiGLU chains
    hid, inter = 1024, 2816
    wg, wu = (synth.q4k_weights(synth.rng(74, k), inter, hid) for k in (1, 2))
    wd = synth.q4k_weights(synth.rng(74, 3), hid, inter)
    xf = synth.activation(synth.rng(74, 0), hid)
    xq = oracle.q8_1_to_bytes(oracle.quantize_q8_1(xf, hid))
    outs = {}
    for sh in (0, 1):
        h, hq, y = _at(inter, 4 * sh), _at(inter // 32 * 40, 16 * sh, "u8"), _at(hid, 4 * sh)
        rz.rz_swiglu_ffn_q4k(_at(wg, 16 * sh, "u8"), _at(wu, 16 * sh, "u8"), _at(wd, 16 * sh, "u8"),
                             _at(xq, 16 * sh, "u8"), h, hq, y, None, hid, inter)
        h2, y2 = _at(inter, 4 * sh), _at(hid, 4 * sh)
        rz.rz_swiglu_ffn_q4k_f32(_at(wg, 16 * sh, "u8"), _at(wu, 16 * sh, "u8"), _at(wd, 16 * sh, "u8"),
                                 _at(xf, 4 * sh), h2, y2, None, hid, inter)
        outs[sh] = [_bits(t) for t in (h, hq, y, h2, y2)]
    for k in range(5):
        assert np.array_equal(outs[0][k], outs[1][k]), "swiglu output %d differs at minimum alignment" % k
    # Q4_0: GEMV (fp32 and Q8_1 x; 16-pair and 160-pair rows), LM head with argmax, GELU FFN
    for out_dim, in_dim in [(1000, 1024), (9, 10240)]:
        w0 = synth.q4_0_weights(synth.rng(75, in_dim), out_dim, in_dim)
        xf = synth.activation(synth.rng(75, 0), in_dim)
        xq = oracle.q8_1_to_bytes(oracle.quantize_q8_1(xf, in_dim))
        for fmt, xx in ((0, xf), (1, xq)):
            dt = "f32" if fmt == 0 else "u8"
            ya, ys = _at(out_dim, 0), _at(out_dim, 4)
            _run_both(lambda ww, x_, yy: rz.rz_q4_0_gemv(ww, x_, fmt, yy, out_dim, in_dim),
                      (_at(w0, 0, "u8"), _at(xx, 0, dt), ya), (_at(w0, 4, "u8"), _at(xx, 16, dt), ys),
                      [ya], [ys], "q4_0 %dx%d fmt %d" % (out_dim, in_dim, fmt))
            need = rz.rz_lm_head_q4_0_workspace_bytes(out_dim, in_dim, fmt)
            bias = synth.activation(synth.rng(75, 7), out_dim)
            res = []
            for sh in (0, 1):
                lg, idx, val = _at(out_dim, 4 * sh), _at(1, 4 * sh, "u8"), _at(1, 4 * sh)
                idx = _at(4, 4 * sh, "u8")
                ws_ = _at(need, 4 * sh, "u8")
                rz.rz_lm_head_q4_0(_at(w0, 4 * sh, "u8"), _at(xx, 16 * sh, dt), fmt, _at(bias, 4 * sh),
                                   lg, out_dim, in_dim, idx, val, ws_)
                res.append([_bits(lg), _bits(idx), _bits(val)])
            for k in range(3):
                assert np.array_equal(res[0][k], res[1][k]), "lm head output %d differs" % k
    hid, inter = 2560, 10240
    wup = synth.q4_0_weights(synth.rng(76, 1), inter, hid)
    wdn = synth.q4_0_weights(synth.rng(76, 2), hid, inter)
    xf = synth.activation(synth.rng(76, 0), hid)
    ub, db = synth.activation(synth.rng(76, 3), inter), synth.activation(synth.rng(76, 4), hid)
    res = []
    for sh in (0, 1):
        h, y = _at(inter, 16 * sh), _at(hid, 4 * sh)
        rz.rz_gelu_ffn_q4_0(_at(wup, 4 * sh, "u8"), _at(wdn, 4 * sh, "u8"), _at(xf, 16 * sh),
                            _at(ub, 4 * sh), _at(db, 4 * sh), h, y, hid, inter)
        res.append([_bits(h), _bits(y)])
    for k in range(2):
        assert np.array_equal(res[0][k], res[1][k]), "gelu output %d differs" % k


# ------------------------------------------------------------------ HIP graph capture
@pytest.mark.parametrize("fused", [False, True])
def test_graph_replays_match_eager(fused):
    """A decode-layer-shaped sequence -- RMSNorm + Q8_1, the attention
    projections in one launch, the O projection with its residual, RMSNorm
    again, the SwiGLU chain with its residual, the LM head with bias and
    greedy token, and the top 40 of its logits -- captured in one HIP graph
    and replayed three times, with
    eager work and synchronisations between replays, gives every replay the
    bytes of the eager run.  Nothing in the library records memsets or
    allocations, so the graph has kernel nodes only.  `fused`: the RMSNorm runs
    inside the Q/K/V launch and the gate/up launch, and the O projection
    quantizes its input itself; every output but the shared Q8_1 buffer then
    also equals the unfused sequence's bytes."""
    import torch
    banner("graph replays", "fused" if fused else "separate")
    H, KV, I, V = 4096, 1024, 2816, 5000      # two-slot rows: the LDS-staged activation path
    g = lambda k: synth.rng(80, k)
    wq, wk, wv, wo = (dev_bytes(synth.q4k_weights(g(k), o, H)) for k, o in ((1, H), (2, KV), (3, KV), (4, H)))
    wg, wu = (dev_bytes(synth.q4k_weights(g(k), I, H)) for k in (5, 6))
    wd = dev_bytes(synth.q4k_weights(g(7), H, I))
    wl = dev_bytes(synth.q4_0_weights(g(8), V, H))
    gam1, gam2 = dev_f32(synth.norm_weights(g(9), H)), dev_f32(synth.norm_weights(g(10), H))
    bias = dev_f32(synth.activation(g(11), V))
    x0 = dev_f32(synth.activation(g(0), H))
    hidden = torch.empty(H, dtype=torch.float32, device="cuda")
    xq = torch.empty(rz.q8_1_nbytes(H), dtype=torch.uint8, device="cuda")
    q, k_, v = (torch.empty(o, dtype=torch.float32, device="cuda") for o in (H, KV, KV))
    h = torch.empty(I, dtype=torch.float32, device="cuda")
    hq = torch.empty(rz.q8_1_nbytes(I), dtype=torch.uint8, device="cuda")
    logits = torch.empty(V, dtype=torch.float32, device="cuda")
    idx = torch.empty(1, dtype=torch.int32, device="cuda")
    val = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(rz.rz_lm_head_q4_0_workspace_bytes(V, H, 0), dtype=torch.uint8, device="cuda")
    tk_idx = torch.empty(40, dtype=torch.int32, device="cuda")
    tk_val = torch.empty(40, dtype=torch.float32, device="cuda")
    tk_ws = torch.empty(rz.rz_topk_f32_workspace_bytes(V, 40), dtype=torch.uint8, device="cuda")
    outs = (hidden, xq, q, k_, v, h, hq, logits, idx, val, tk_idx, tk_val)

    def layer(fused):
        hidden.copy_(x0)
        if fused:
            # the Q8_1 side output keeps xq an output of the fused sequence too
            rz.rz_rmsnorm_q4k_q8_gemv_multi([wq, wk, wv], hidden, gam1, 1e-5, H, xq, [q, k_, v],
                                            [H, KV, KV], H)
        else:
            rz.rz_rmsnorm_q8_1(hidden, gam1, 1e-5, H, H, 1, None, xq)
            rz.rz_q4k_q8_gemv_multi([wq, wk, wv], xq, [q, k_, v], [H, KV, KV], H)
        # the attention output stands in as q; quantize it for the O projection
        if fused:
            rz.rz_q4k_q8_gemv_f32_add(wo, q, H, None, hidden, hidden, H, H)
        else:
            rz.rz_q8_1_quantize(q, H, H, 1, xq)
            rz.rz_q4k_q8_gemv_add(wo, xq, hidden, hidden, H, H, 1)
        if fused:
            rz.rz_rmsnorm_swiglu_ffn_q4k_add(wg, wu, wd, hidden, gam2, 1e-5, h, hq, hidden, None,
                                             H, I)
        else:
            rz.rz_rmsnorm_q8_1(hidden, gam2, 1e-5, H, H, 1, None, xq)
            rz.rz_swiglu_ffn_q4k_add(wg, wu, wd, xq, h, hq, hidden, hidden, None, H, I)
        rz.rz_lm_head_q4_0(wl, hidden, 0, bias, logits, V, H, idx, val, ws)
        rz.rz_topk_f32(logits, V, 40, tk_idx, tk_val, tk_ws)

    layer(False)
    torch.cuda.synchronize()
    separate = [_bits(t) for t in outs]
    if fused:
        layer(True)
        torch.cuda.synchronize()
    eager = [_bits(t) for t in outs]
    for k, t in enumerate(outs):
        if t is not xq:
            assert np.array_equal(eager[k], separate[k]), "output %d: fused differs from separate" % k
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(fused)                              # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        layer(fused)
    for rep in range(3):
        for t in outs:                            # eager work between replays
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, t in enumerate(outs):
            assert np.array_equal(_bits(t), eager[k]), "replay %d: output %d differs from eager" % (rep, k)


def test_library_loaded_before_torch():
    """A process that loads librz.so before importing torch (here through a
    size query, which touches no device) still runs kernels on torch's
    tensors: the binding imports torch first, so both use one HIP runtime."""
    import subprocess
    import sys
    banner("library before torch")
    child = (
        "import sys; sys.path.insert(0, %r)\n"
        "import q4_q8_integer_quantize_amd as rz\n"
        "assert rz.rz_topk_f32_workspace_bytes(3824, 12) > 0\n"
        "import torch\n"
        "v = torch.arange(3824, dtype=torch.float32, device='cuda')\n"
        "i = torch.empty(12, dtype=torch.int32, device='cuda')\n"
        "ws = torch.empty(rz.rz_topk_f32_workspace_bytes(3824, 12), dtype=torch.uint8, device='cuda')\n"
        "rz.rz_topk_f32(v, 3824, 12, i, None, ws)\n"
        "assert i.cpu().tolist() == list(range(3823, 3811, -1)), i.cpu().tolist()\n"
        "print('ok')\n" % str(__import__("pathlib").Path(__file__).resolve().parents[1]))
    res = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, timeout=100)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stderr[-2000:]


def test_c_consumer_without_python():
    """tests/native/abi_consumer (built by the package build from plain C
    against include/rz.h, librz.so and the HIP runtime, no torch) quantizes,
    multiplies the hand-worked Q4_K super-blocks of the golden fixture
    (43600, 90064, 46464, exact) and takes their top 2 on device 0."""
    import subprocess
    banner("C consumer")
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_consumer")
    assert os.path.exists(exe), "tests/native/abi_consumer is not built (run the package build)"
    res = subprocess.run([exe, "gpu"], capture_output=True, text=True, timeout=100)
    assert res.returncode == 0 and "passed: 0 failure(s)" in res.stdout, res.stdout + res.stderr


def test_concurrent_streams_match_sequential():
    """The library keeps no state between calls: three independent call chains
    issued on three streams (default priority) at once -- quantize + GEMV with
    the Q8_1 side output, the SwiGLU chain with its residual, and the LM head
    with bias and its top 40 -- repeated with no synchronisation between the
    rounds, give every round the bytes of the same chains run one after
    another on one stream."""
    import torch
    banner("concurrent streams")
    H, I, V = 4096, 2816, 20000
    g = lambda k: synth.rng(90, k)
    w1 = dev_bytes(synth.q4k_weights(g(1), 14336, H))
    wg, wu = (dev_bytes(synth.q4k_weights(g(k), I, H)) for k in (2, 3))
    wd = dev_bytes(synth.q4k_weights(g(4), H, I))
    wl = dev_bytes(synth.q4_0_weights(g(5), V, H))
    x1, x2, x3 = (dev_f32(synth.activation(g(10 + k), H)) for k in range(3))
    bias = dev_f32(synth.activation(g(14), V))

    def buffers():
        return dict(xq1=torch.empty(rz.q8_1_nbytes(H), dtype=torch.uint8, device="cuda"),
                    y1=torch.empty(14336, dtype=torch.float32, device="cuda"),
                    xq2=torch.empty(rz.q8_1_nbytes(H), dtype=torch.uint8, device="cuda"),
                    h=torch.empty(I, dtype=torch.float32, device="cuda"),
                    hq=torch.empty(rz.q8_1_nbytes(I), dtype=torch.uint8, device="cuda"),
                    hid=torch.empty(H, dtype=torch.float32, device="cuda"),
                    logits=torch.empty(V, dtype=torch.float32, device="cuda"),
                    ti=torch.empty(40, dtype=torch.int32, device="cuda"),
                    tv=torch.empty(40, dtype=torch.float32, device="cuda"),
                    ws=torch.empty(rz.rz_topk_f32_workspace_bytes(V, 40), dtype=torch.uint8,
                                   device="cuda"))

    def chain(b, which, stream):
        if which == 0:
            rz.rz_q4k_q8_gemv_f32(w1, x1, H, b["xq1"], b["y1"], 14336, H, stream=stream)
        elif which == 1:
            b["hid"].copy_(x2)
            rz.rz_q8_1_quantize(x2, H, H, 1, b["xq2"], stream=stream)
            rz.rz_swiglu_ffn_q4k_add(wg, wu, wd, b["xq2"], b["h"], b["hq"], b["hid"], b["hid"],
                                     None, H, I, stream=stream)
        else:
            rz.rz_lm_head_q4_0_topk(wl, x3, 0, bias, b["logits"], V, H, 40, b["ti"], b["tv"],
                                    b["ws"], stream=stream)

    ref = buffers()
    for which in range(3):
        chain(ref, which, None)
    torch.cuda.synchronize()
    want = {k: _bits(t) for k, t in ref.items() if k != "ws"}
    streams = [torch.cuda.Stream() for _ in range(3)]
    rounds = [buffers() for _ in range(4)]
    torch.cuda.synchronize()
    for b in rounds:
        for which, st in enumerate(streams):
            with torch.cuda.stream(st):
                chain(b, which, st)
    torch.cuda.synchronize()
    for n, b in enumerate(rounds):
        for k, t in b.items():
            if k != "ws":
                assert np.array_equal(_bits(t), want[k]), "round %d: %s differs" % (n, k)


# ------------------------------------------------------------------ RMSNorm fused into the GEMV
@pytest.mark.parametrize("in_dim,n,out_dims", [
    (1024, 1000, [300, 64]),               # four teams a row
    (2048, 2047, [33, 65, 17]),            # dword activation loads
    (4096, 4096, [4096, 1024, 1024]),      # the Q, K, V projections
    (5120, 4999, [700, 128]),              # three slots, ragged n
    (16384, 16384, [129]),
    (4096, 4096, [2048, 1024, 1024]),      # 2048 row groups: 2 groups a wave
    (4096, 4000, [3000, 2000, 1000]),      # 3000 row groups: 3 groups a wave
    (4096, 4096, [4096, 4096, 8192]),      # 8192 row groups: 4 groups a wave
    (1024, 1024, [30000, 100]),            # 7525 row groups: 8 groups a wave
])
def test_rmsnorm_q4k_q8_gemv_multi_bit_identical(in_dim, n, out_dims):
    """One launch (RMSNorm + Q8_1 in every workgroup, then the GEMVs) equals
    rz_rmsnorm_q8_1 followed by rz_q4k_q8_gemv_multi bit for bit (the outputs
    and the Q8_1 side output), and against the oracle: the side output is the
    oracle's Q8_1 of the GPU's normed values, byte for byte, and every output
    is within the GEMV bound of the oracle's product over those blocks."""
    banner("rmsnorm multi", in_dim, n, out_dims)
    x = synth.activation(synth.rng(81, in_dim), n)
    gam = synth.norm_weights(synth.rng(81, 1), n)
    blobs = [synth.q4k_weights(synth.rng(82, k), o, in_dim) for k, o in enumerate(out_dims)]
    ws = [dev_bytes(b) for b in blobs]
    xd, gd = dev_f32(x), dev_f32(gam)
    xq_ref = empty_bytes(rz.q8_1_nbytes(in_dim))
    normed = empty_f32(n)
    rz.rz_rmsnorm_q8_1(xd, gd, 1e-5, n, in_dim, 1, normed, xq_ref)
    y_ref = [empty_f32(o) for o in out_dims]
    rz.rz_q4k_q8_gemv_multi(ws, xq_ref, y_ref, out_dims, in_dim)
    xq = empty_bytes(rz.q8_1_nbytes(in_dim))
    y = [empty_f32(o) for o in out_dims]
    rz.rz_rmsnorm_q4k_q8_gemv_multi(ws, xd, gd, 1e-5, n, xq, y, out_dims, in_dim)
    assert np.array_equal(host(xq), host(xq_ref)), "Q8_1 side output differs"
    for m, (a_, b_) in enumerate(zip(y, y_ref)):
        assert np.array_equal(host(a_).view(np.uint32), host(b_).view(np.uint32)), "matrix %d" % m
    y2 = [empty_f32(o) for o in out_dims]
    rz.rz_rmsnorm_q4k_q8_gemv_multi(ws, xd, gd, 1e-5, n, None, y2, out_dims, in_dim)
    for a_, b_ in zip(y2, y_ref):
        assert np.array_equal(host(a_).view(np.uint32), host(b_).view(np.uint32))
    # against the oracle: the normed values within the fp32 bound of the float64
    # RMSNorm, the fused launch's Q8_1 side output byte-equal to the oracle's
    # quantize of those values, every output within the GEMV bound of the
    # oracle's integer form over those blocks
    nv = host(normed)
    ref = oracle.rmsnorm(x, gam, 1e-5)
    assert np.all(np.abs(nv.astype(np.float64) - ref) <= oracle.rmsnorm_tolerance(ref, _norm_chain(in_dim)))
    xq_o = oracle.quantize_q8_1(nv, in_dim)
    bad = first_mismatch(q8_host_bytes(xq, in_dim // 32), oracle.q8_1_to_bytes(xq_o))
    assert bad is None, "fused Q8_1 side output differs from the oracle: %r" % (bad,)
    for m, (b_, y_) in enumerate(zip(blobs, y)):
        y_o, t_o = oracle.gemv_q4k_q8_int(b_, xq_o)
        assert_within(host(y_), y_o, t_o, "rmsnorm multi matrix %d" % m)


@pytest.mark.parametrize("hidden,inter", [
    (1024, 2816),
    (2048, 5632),
    (4096, 14336),       # the 8B FFN block
    (16384, 256),        # the widest hidden state, one pass of gate/up rows
])
def test_rmsnorm_swiglu_ffn_add_bit_identical(hidden, inter):
    """The pre-norm FFN block in two launches (RMSNorm + Q8_1 in every gate/up
    workgroup, then down + residual) equals rz_rmsnorm_q8_1 followed by
    rz_swiglu_ffn_q4k_add with r = x, bit for bit: h, h_q8, gu and y, also
    with y written over x."""
    banner("rmsnorm swiglu add", hidden, inter)
    x = synth.activation(synth.rng(83, hidden), hidden)
    gam = synth.norm_weights(synth.rng(83, 1), hidden)
    blobs = [synth.q4k_weights(synth.rng(84, k), o, i)
             for k, (o, i) in enumerate(((inter, hidden), (inter, hidden), (hidden, inter)))]
    ws = [dev_bytes(b) for b in blobs]
    xd, gd = dev_f32(x), dev_f32(gam)
    xq = empty_bytes(rz.q8_1_nbytes(hidden))
    normed = empty_f32(hidden)
    rz.rz_rmsnorm_q8_1(xd, gd, 1e-5, hidden, hidden, 1, normed, xq)
    h_ref, hq_ref = empty_f32(inter), empty_bytes(rz.q8_1_nbytes(inter))
    gu_ref, y_ref = empty_f32(2 * inter), empty_f32(hidden)
    rz.rz_swiglu_ffn_q4k_add(*ws[:3], xq, h_ref, hq_ref, xd, y_ref, gu_ref, hidden, inter)
    bits = lambda t: host(t).view(np.uint32)
    for in_place in (False, True):
        xd2 = dev_f32(x)
        h, hq = empty_f32(inter), empty_bytes(rz.q8_1_nbytes(inter))
        gu = empty_f32(2 * inter)
        y = xd2 if in_place else empty_f32(hidden)
        rz.rz_rmsnorm_swiglu_ffn_q4k_add(*ws[:3], xd2, gd, 1e-5, h, hq, y, gu, hidden, inter)
        assert np.array_equal(bits(gu), bits(gu_ref)), "gate/up"
        assert np.array_equal(bits(h), bits(h_ref)), "h"
        assert np.array_equal(host(hq), host(hq_ref)), "h_q8"
        assert np.array_equal(bits(y), bits(y_ref)), "y (in place: %s)" % in_place
    y2 = empty_f32(hidden)
    rz.rz_rmsnorm_swiglu_ffn_q4k_add(*ws[:3], xd, gd, 1e-5, h, hq, y2, None, hidden, inter)
    assert np.array_equal(bits(y2), bits(y_ref)), "without gu"
    # against the oracle, stage by stage on the fused launch's outputs (h, h_q8,
    # gu and y above are those of the fused launch, bit for bit): the activation
    # blocks are the oracle's Q8_1 of the GPU's normed values; g and u within the
    # GEMV bound; h within the bound propagated through silu(g) * u; h_q8 the
    # oracle's Q8_1 of the GPU's h, byte for byte; y within the GEMV bound of the
    # oracle's down projection over those blocks plus the residual x
    nv = host(normed)
    ref = oracle.rmsnorm(x, gam, 1e-5)
    assert np.all(np.abs(nv.astype(np.float64) - ref) <= oracle.rmsnorm_tolerance(ref, _norm_chain(hidden)))
    xq_o = oracle.quantize_q8_1(nv, hidden)
    assert first_mismatch(q8_host_bytes(xq, hidden // 32), oracle.q8_1_to_bytes(xq_o)) is None
    g_o, tg = oracle.gemv_q4k_q8_int(blobs[0], xq_o)
    u_o, tu = oracle.gemv_q4k_q8_int(blobs[1], xq_o)
    gu_h = host(gu)
    assert_within(gu_h[:inter], g_o, tg, "rmsnorm swiglu gate")
    assert_within(gu_h[inter:], u_o, tu, "rmsnorm swiglu up")
    h_o = oracle.swiglu(g_o, u_o)
    tol_h = oracle.h_tolerance(g_o, u_o, oracle.gemv_tolerance(tg), oracle.gemv_tolerance(tu), h_o)
    h_h = host(h)
    assert np.all(np.abs(h_h.astype(np.float64) - h_o) <= tol_h), "rmsnorm swiglu h"
    hq_o = oracle.quantize_q8_1(h_h, inter)
    bad = first_mismatch(q8_host_bytes(hq, inter // 32), oracle.q8_1_to_bytes(hq_o))
    assert bad is None, "h_q8 differs from the oracle's quantize of the GPU's h: %r" % (bad,)
    y_o, ty = oracle.gemv_q4k_q8_int(blobs[2], hq_o)
    assert_within(host(y2), oracle.residual_add(x, y_o), ty + np.abs(x), "rmsnorm swiglu y")


@pytest.mark.parametrize("out_dim,n,in_dim", [
    (4096, 4096, 4096),      # the O projection of the attention workload
    (14336, 4096, 4096),
    (300, 1000, 1024),       # ragged n, ragged rows
    (65, 16384, 16384),
])
def test_q4k_q8_gemv_f32_add_bit_identical(out_dim, n, in_dim):
    """Quantize + GEMV + residual in one launch equals rz_q8_1_quantize followed
    by rz_q4k_q8_gemv_add bit for bit (y out of place and in place, r is y, and
    the Q8_1 side output), the side output is the oracle's Q8_1 of x byte for
    byte, and y is within the GEMV bound of the oracle plus r."""
    banner("f32 add", out_dim, n, in_dim)
    x = synth.activation(synth.rng(85, in_dim), n)
    r = synth.activation(synth.rng(85, 1), out_dim)
    blob = synth.q4k_weights(synth.rng(86, out_dim), out_dim, in_dim)
    w = dev_bytes(blob)
    xd = dev_f32(x)
    xq_ref = empty_bytes(rz.q8_1_nbytes(in_dim))
    rz.rz_q8_1_quantize(xd, n, in_dim, 1, xq_ref)
    y_ref = empty_f32(out_dim)
    rz.rz_q4k_q8_gemv_add(w, xq_ref, dev_f32(r), y_ref, out_dim, in_dim, 1)
    bits = lambda t: host(t).view(np.uint32)
    xq = empty_bytes(rz.q8_1_nbytes(in_dim))
    y = empty_f32(out_dim)
    rz.rz_q4k_q8_gemv_f32_add(w, xd, n, xq, dev_f32(r), y, out_dim, in_dim)
    assert np.array_equal(host(xq), host(xq_ref)), "Q8_1 side output"
    assert np.array_equal(bits(y), bits(y_ref)), "out of place"
    yr = dev_f32(r)
    rz.rz_q4k_q8_gemv_f32_add(w, xd, n, None, yr, yr, out_dim, in_dim)
    assert np.array_equal(bits(yr), bits(y_ref)), "in place"
    # against the oracle: the side output is the oracle's Q8_1 of x byte for
    # byte, and y is within the GEMV bound of the integer form plus r
    xq_o = oracle.quantize_q8_1(x, in_dim)
    bad = first_mismatch(q8_host_bytes(xq, in_dim // 32), oracle.q8_1_to_bytes(xq_o))
    assert bad is None, "Q8_1 side output differs from the oracle: %r" % (bad,)
    y_o, t_o = oracle.gemv_q4k_q8_int(blob, xq_o)
    assert_within(host(y), oracle.residual_add(r, y_o), t_o + np.abs(r), "f32 add y")


def _draw_add(g):
    while True:
        nt = int(g.integers(1, 9))
        in_dim = 256 * int(g.integers(1, 81))
        out_dim = int(np.exp(g.uniform(0, np.log(3000))))
        if out_dim * in_dim * nt <= 24_000_000:
            return out_dim, in_dim, nt


@pytest.mark.parametrize("out_dim,in_dim,nt", _rand_cases(97, 12, _draw_add))
def test_q4k_gemv_add_random_shapes(out_dim, in_dim, nt):
    """The residual checks of test_q4k_gemv_add on seeded random shapes and
    token counts (1-2 on the dot4 kernel, 3-8 on the matrix cores, column
    passes past the register window)."""
    test_q4k_gemv_add(out_dim, in_dim, nt)


def _draw_fused(g):
    while True:
        in_dim = 256 * int(g.integers(1, 65))
        n = int(g.integers(max(1, in_dim - 255), in_dim + 1))
        out_dim = int(np.exp(g.uniform(0, np.log(6000))))
        if out_dim * in_dim <= 24_000_000:
            return out_dim, n, in_dim


@pytest.mark.parametrize("out_dim,n,in_dim", _rand_cases(98, 10, _draw_fused))
def test_q4k_gemv_f32_two_step_random_shapes(out_dim, n, in_dim):
    """The checks of test_q4k_gemv_f32_matches_two_step_and_oracle (bit-equal
    to quantize then GEMV, side output equal to the oracle's bytes) on seeded
    random shapes and ragged activation lengths."""
    test_q4k_gemv_f32_matches_two_step_and_oracle(out_dim, n, in_dim)


@pytest.mark.parametrize("out_dim,n,in_dim", _rand_cases(99, 8, _draw_fused))
def test_q4k_q8_gemv_f32_add_random_shapes(out_dim, n, in_dim):
    """The checks of test_q4k_q8_gemv_f32_add_bit_identical on seeded random
    shapes."""
    test_q4k_q8_gemv_f32_add_bit_identical(out_dim, n, in_dim)


def _draw_norm_ffn(g):
    while True:
        hidden, inter = 256 * int(g.integers(1, 33)), 256 * int(g.integers(1, 41))
        if hidden * inter <= 12_000_000:
            return hidden, inter


@pytest.mark.parametrize("hidden,inter", _rand_cases(100, 8, _draw_norm_ffn))
def test_rmsnorm_swiglu_ffn_add_random_shapes(hidden, inter):
    """The checks of test_rmsnorm_swiglu_ffn_add_bit_identical on seeded
    random sizes."""
    test_rmsnorm_swiglu_ffn_add_bit_identical(hidden, inter)


@pytest.mark.parametrize("hidden,inter", _rand_cases(101, 8, _draw_swiglu))
def test_swiglu_ffn_f32_chain_random_shapes(hidden, inter):
    """The staged checks of test_swiglu_ffn_f32_chain on seeded random sizes."""
    test_swiglu_ffn_f32_chain(hidden, inter)


def _draw_norm_multi(g):
    k = int(g.integers(1, 9))
    in_dim = 256 * int(g.integers(1, 65))
    n = int(g.integers(max(1, in_dim - 255), in_dim + 1))
    outs = [int(np.exp(g.uniform(0, np.log(2000)))) for _ in range(k)]
    return in_dim, n, outs


@pytest.mark.parametrize("in_dim,n,out_dims", _rand_cases(102, 10, _draw_norm_multi))
def test_rmsnorm_q4k_q8_gemv_multi_random_shapes(in_dim, n, out_dims):
    """The checks of test_rmsnorm_q4k_q8_gemv_multi_bit_identical on seeded
    random matrix sets, row lengths and ragged activation lengths."""
    test_rmsnorm_q4k_q8_gemv_multi_bit_identical(in_dim, n, out_dims)


def test_minimum_alignments_fused_entries():
    """The RMSNorm-prologue entries and quantize + GEMV + residual on buffers
    at exactly the alignments include/rz.h requires (Q4_K and Q8_1 16 bytes,
    fp32 4) give the same bytes as on 256-byte aligned buffers."""
    banner("minimum alignments, fused entries")
    H, I = 1024, 2816
    gam = synth.norm_weights(synth.rng(76, 2), H)
    shapes = [(300, H), (64, H)]
    ws = [synth.q4k_weights(synth.rng(76, 10 + k), o, H) for k, (o, _) in enumerate(shapes)]
    for n in (H, H - 3):           # 16-byte and dword activation loads
        x = synth.activation(synth.rng(76, n), n)
        res = []
        for sh in (0, 1):
            ys = [_at(o, 4 * sh) for o, _ in shapes]
            q = _at(H // 32 * 40, 16 * sh, "u8")
            rz.rz_rmsnorm_q4k_q8_gemv_multi([_at(w_, 16 * sh, "u8") for w_ in ws], _at(x, 4 * sh),
                                            _at(gam[:n], 4 * sh), 1e-5, n, q, ys,
                                            [o for o, _ in shapes], H)
            res.append([_bits(t) for t in ys + [q]])
        for k, (a_, b_) in enumerate(zip(*res)):
            assert np.array_equal(a_, b_), "rmsnorm multi n %d output %d" % (n, k)
    wg, wu = (synth.q4k_weights(synth.rng(77, k), I, H) for k in (1, 2))
    wd = synth.q4k_weights(synth.rng(77, 3), H, I)
    x = synth.activation(synth.rng(77, 0), H)
    res = []
    for sh in (0, 1):
        h, hq, y, gu = _at(I, 4 * sh), _at(I // 32 * 40, 16 * sh, "u8"), _at(H, 4 * sh), _at(2 * I, 4 * sh)
        rz.rz_rmsnorm_swiglu_ffn_q4k_add(_at(wg, 16 * sh, "u8"), _at(wu, 16 * sh, "u8"),
                                         _at(wd, 16 * sh, "u8"), _at(x, 4 * sh), _at(gam, 4 * sh),
                                         1e-5, h, hq, y, gu, H, I)
        res.append([_bits(t) for t in (h, hq, y, gu)])
    for k, (a_, b_) in enumerate(zip(*res)):
        assert np.array_equal(a_, b_), "rmsnorm swiglu output %d" % k
    w = synth.q4k_weights(synth.rng(78, 1), 500, 4096)
    r = synth.activation(synth.rng(78, 2), 500)
    for n in (4096, 4093):
        xf = synth.activation(synth.rng(78, n), n)
        res = []
        for sh in (0, 1):
            y, q = _at(500, 4 * sh), _at(128 * 40, 16 * sh, "u8")
            rz.rz_q4k_q8_gemv_f32_add(_at(w, 16 * sh, "u8"), _at(xf, 4 * sh), n, q, _at(r, 4 * sh), y,
                                      500, 4096)
            res.append([_bits(y), _bits(q)])
        for k, (a_, b_) in enumerate(zip(*res)):
            assert np.array_equal(a_, b_), "f32 add n %d output %d" % (n, k)
