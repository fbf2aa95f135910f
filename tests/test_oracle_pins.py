"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-worked blocks (tests/golden/), closed forms, exact-integer cases, the
dequantize-then-dot identity, padding invariance and symmetry properties.

A plausible slip in the oracle -- a wrong nibble order, 6-bit unpack, rounding
mode, dropped min term, sign or transposed operand -- fails at least one test.
"""
import numpy as np
import pytest

import oracle
import synth
from golden_io import floats, hexbytes, ints, load, pairs

U32 = 2.0 ** -24   # fp32 unit roundoff


# ----------------------------------------------------------------- helpers
def _q8_block_input(fx, key):
    x = np.zeros(32, np.float32)
    vals = floats(fx[key + ".x"])
    x[:len(vals)] = vals
    return x


def _ones_q8(nblocks):
    return oracle.Q8Blocks(np.ones(nblocks, np.float32), np.full(nblocks, 32.0, np.float32),
                           np.ones((nblocks, 32), np.int8))


def _onehot_q8(nblocks, k):
    d = np.zeros(nblocks, np.float32)
    s = np.zeros(nblocks, np.float32)
    q = np.zeros((nblocks, 32), np.int8)
    d[k // 32] = 1.0
    s[k // 32] = 1.0
    q[k // 32, k % 32] = 1
    return oracle.Q8Blocks(d, s, q)


def _pack_uniform_scales(S, M):
    """12 scale bytes with every 6-bit scale = S and every min = M (the test's own
    encoding of the packing read in q4k_superblock.txt)."""
    lo_s = (S & 63) | ((S >> 4) << 6)
    lo_m = (M & 63) | ((M >> 4) << 6)
    hi = (S & 15) | ((M & 15) << 4)
    return bytes([lo_s] * 4 + [lo_m] * 4 + [hi] * 4)


def _f16le(v):
    return np.array([v], np.float16).tobytes()


# ----------------------------------------------------------------- Q8_1
@pytest.mark.parametrize("key", ["A", "B", "C", "D"])
def test_q8_1_hand_worked_blocks(key):
    fx = load("q8_1_blocks.txt")
    blk = oracle.quantize_q8_1(_q8_block_input(fx, key))
    q_exp = np.zeros(32, np.int64)
    qv = ints(fx[key + ".q"])
    q_exp[:len(qv)] = qv
    assert blk.d[0] == np.float32(float(fx[key + ".d"]))
    assert blk.s[0] == np.float32(float(fx[key + ".s"]))
    assert np.array_equal(blk.q[0].astype(np.int64), q_exp)


def test_q8_1_bytes_layout():
    fx = load("q8_1_blocks.txt")
    raw = oracle.q8_1_to_bytes(oracle.quantize_q8_1(_q8_block_input(fx, "B")))
    assert raw.shape == (1, 40)
    assert raw[0, 0:4].tobytes() == np.float32(0.25).tobytes()
    assert raw[0, 4:8].tobytes() == np.float32(32.25).tobytes()
    assert raw[0, 8] == 127 and raw[0, 11] == 0xFE  # -2 as int8
    back = oracle.q8_1_from_bytes(raw)
    assert back.d[0] == np.float32(0.25) and back.q[0, 4] == -4


def test_q8_1_padding_tail_is_zero_blocks():
    x = synth.activation(synth.rng(0, 0), 896)
    blk = oracle.quantize_q8_1(x, 1024)
    assert blk.n_blocks == 32
    assert np.all(blk.d[28:] == 0) and np.all(blk.s[28:] == 0) and np.all(blk.q[28:] == 0)
    same = oracle.quantize_q8_1(np.concatenate([x, np.zeros(128, np.float32)]), 1024)
    assert np.array_equal(oracle.q8_1_to_bytes(blk), oracle.q8_1_to_bytes(same))


@pytest.mark.parametrize("seed", range(4))
def test_q8_1_properties(seed):
    g = np.random.default_rng(100 + seed)
    x = (g.standard_normal(32 * 16) * np.exp(g.uniform(-8, 8, 32 * 16))).astype(np.float32)
    blk = oracle.quantize_q8_1(x)
    xb = x.reshape(16, 32).astype(np.float64)
    d = blk.d.astype(np.float64)
    q = blk.q.astype(np.int64)
    # codes inside the int8 range, and the largest magnitude maps to +-127
    assert np.all(np.abs(q) <= 127)
    amax_idx = np.argmax(np.abs(xb), axis=1)
    assert np.all(np.abs(q[np.arange(16), amax_idx]) == 127)
    # d is amax/127 up to one fp32 rounding
    amax = np.abs(xb).max(axis=1)
    assert np.all(np.abs(d - amax / 127) <= U32 * amax / 127)
    # reconstruction error of a nearest rounding: at most d/2 (plus fp32 slack)
    assert np.all(np.abs(xb - d[:, None] * q) <= d[:, None] * (0.5 + 1e-5))
    # s is d * sum(q) up to one fp32 rounding
    exact = d * q.sum(axis=1)
    assert np.all(np.abs(blk.s - exact) <= U32 * np.abs(exact))


@pytest.mark.parametrize("seed", range(3))
def test_q8_1_sign_and_power_of_two_symmetry(seed):
    x = synth.activation(np.random.default_rng(7 + seed), 256)
    a = oracle.quantize_q8_1(x)
    neg = oracle.quantize_q8_1(-x)
    assert np.array_equal(neg.q, -a.q) and np.array_equal(neg.d, a.d) and np.array_equal(neg.s, -a.s)
    for k in (-3, 5):
        sc = oracle.quantize_q8_1((x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(sc.q, a.q)
        assert np.array_equal(sc.d, (a.d * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(sc.s, (a.s * np.float32(2.0 ** k)).astype(np.float32))


def _units(vals, e):
    """float32 values k * 2^e for the integers or halves k (exact, denormals included)."""
    return np.array([np.ldexp(v, e) for v in vals], np.float64).astype(np.float32)


def test_q8_1_denormal_blocks():
    """Blocks of denormals, worked by hand in units of 2^-149 and 2^-140.
    amax = 63 units: amax/127 < 2^-150 rounds to 0, and the block is zeros.
    amax = 64 units: amax/127 = 0.504 units rounds to d = 2^-149, so every code
    is the value in units.  amax = 190 units: d = 2^-149 again and the clamp
    binds.  amax = 127 * 2^-140: d = 2^-140 exactly, and halves of d round to
    even."""
    x = np.zeros(32, np.float32)
    x[:3] = _units([63, -5, 1], -149)
    blk = oracle.quantize_q8_1(x)
    assert blk.d[0] == 0 and blk.s[0] == 0 and not blk.q.any()

    x = np.zeros(32, np.float32)
    ks = [64, -63, 1, -1, 0, 32, 7, -40]
    x[:8] = _units(ks, -149)
    blk = oracle.quantize_q8_1(x)
    assert blk.d[0] == np.float32(np.ldexp(1.0, -149))
    assert list(blk.q[0, :8]) == ks and not blk.q[0, 8:].any()
    assert blk.s[0] == np.float32(np.ldexp(sum(ks), -149))

    # amax = 190 units: 190/127 = 1.496 rounds down to d = 2^-149, so 190 and
    # -190 units quotient to +-190 and the clamp to [-127, 127] binds
    x = np.zeros(32, np.float32)
    x[:3] = _units([190, 100, -190], -149)
    blk = oracle.quantize_q8_1(x)
    assert blk.d[0] == np.float32(np.ldexp(1.0, -149))
    assert list(blk.q[0, :3]) == [127, 100, -127] and not blk.q[0, 3:].any()
    assert blk.s[0] == np.float32(np.ldexp(100, -149))

    x = np.zeros(32, np.float32)
    x[:6] = _units([127, 0.5, 1.5, 2.5, -0.5, -1.5], -140)
    blk = oracle.quantize_q8_1(x)
    assert blk.d[0] == np.float32(np.ldexp(1.0, -140))
    assert list(blk.q[0, :6]) == [127, 0, 2, 2, 0, -2]
    assert blk.s[0] == np.float32(np.ldexp(129, -140))


def test_q8_1_batch_is_per_token():
    X = synth.activation(synth.rng(4, 0), 256, n_tokens=3)
    b = oracle.quantize_q8_1(X)
    for t in range(3):
        one = oracle.quantize_q8_1(X[t])
        assert np.array_equal(oracle.q8_1_to_bytes(b.token(t)), oracle.q8_1_to_bytes(one))


# ----------------------------------------------------------------- Q4_K
def _fixture_superblock():
    fx = load("q4k_superblock.txt")
    raw = hexbytes(fx["header_hex"]) + hexbytes(fx["qs_fill_hex"]) * 128
    return fx, np.frombuffer(raw, np.uint8).reshape(1, 1, 144).copy()


def test_q4k_hand_worked_superblock():
    fx, blob = _fixture_superblock()
    d, dmin, sc, m, q = oracle.q4k_fields(blob)
    assert d[0, 0] == 1.0 and dmin[0, 0] == 0.5
    assert sc[0, 0].tolist() == ints(fx["sc"])
    assert m[0, 0].tolist() == ints(fx["m"])
    w = oracle.dequantize_q4k(blob).reshape(8, 32)
    w_sub = floats(fx["w_sub"])
    for j in range(8):
        assert np.all(w[j] == w_sub[j])
    ones = _ones_q8(8)
    y_int, _ = oracle.gemv_q4k_q8_int(blob, ones)
    y_def = oracle.gemv_q4k_q8_def(blob, ones)
    assert y_int[0] == float(fx["y_ones"]) and y_def[0] == float(fx["y_ones"])


def test_q4k_hand_worked_nibble_order():
    fx = load("q4k_nibble_order.txt")
    raw = bytearray(hexbytes(fx["header_hex"]) + bytes(128))
    for k, v in pairs(fx["qs_set"], int, lambda s: int(s, 16)):
        raw[16 + k] = v
    blob = np.frombuffer(bytes(raw), np.uint8).reshape(1, 1, 144).copy()
    w = oracle.dequantize_q4k(blob)[0]
    for idx, val in pairs(fx["w_at"]):
        assert w[idx] == val, (idx, w[idx], val)
    x = _onehot_q8(8, 32)
    assert oracle.gemv_q4k_q8_int(blob, x)[0][0] == float(fx["y_onehot32"])
    assert oracle.gemv_q4k_q8_def(blob, x)[0] == float(fx["y_onehot32"])


def test_q4k_f32_hand_worked_superblock():
    """fp32 activation of all ones: y and the factored-form terms as worked by hand."""
    fx, blob = _fixture_superblock()
    y, terms = oracle.gemv_q4k_f32(blob, np.ones(256, np.float32))
    assert y[0] == float(fx["y_ones"])
    assert terms[0] == float(fx["terms_f32_ones"])


def test_q4k_f32_unit_vectors_pick_the_fixture_elements():
    """x = e_k returns weight k of the super-block: the element order of the fp32
    path against the hand-worked positions (an interleaved nibble order or an
    off-by-one chunk fails here)."""
    fx = load("q4k_nibble_order.txt")
    raw = bytearray(hexbytes(fx["header_hex"]) + bytes(128))
    for k, v in pairs(fx["qs_set"], int, lambda s: int(s, 16)):
        raw[16 + k] = v
    blob = np.frombuffer(bytes(raw), np.uint8).reshape(1, 1, 144).copy()
    for idx, val in pairs(fx["w_at"]):
        x = np.zeros(256, np.float32)
        x[idx] = 1.0
        assert oracle.gemv_q4k_f32(blob, x)[0][0] == val, idx
    x = np.zeros(256, np.float32)
    x[32] = 1.0
    assert oracle.gemv_q4k_f32(blob, x)[0][0] == float(fx["y_onehot32"])


@pytest.mark.parametrize("qn,S,M,v", [(3, 5, 9, 0.75), (15, 63, 63, -2.5), (0, 40, 17, 1.0),
                                      (9, 18, 0, -0.125)])
def test_q4k_f32_closed_form(qn, S, M, v):
    """All nibbles qn, scales S, mins M, every activation value v:
    y = in_dim * v * (d*S*qn - dmin*M) and terms = in_dim * |v| * (d*S*qn + dmin*M)."""
    d, dmin, nsb = 0.0078125, 0.001953125, 3
    sb = _f16le(d) + _f16le(dmin) + _pack_uniform_scales(S, M) + bytes([qn | (qn << 4)] * 128)
    blob = np.frombuffer(sb * nsb, np.uint8).reshape(1, nsb, 144).copy()
    y, terms = oracle.gemv_q4k_f32(blob, np.full(nsb * 256, v, np.float32))
    n = nsb * 256
    assert y[0] == pytest.approx(n * v * (d * S * qn - dmin * M), rel=1e-13, abs=1e-12)
    assert terms[0] == pytest.approx(n * abs(v) * (d * S * qn + dmin * M), rel=1e-13)


@pytest.mark.parametrize("out_dim,in_dim,seed", [(1, 256, 0), (7, 512, 1), (65, 1024, 2),
                                                 (40, 4096, 3)])
def test_q4k_f32_equals_integer_form_on_exact_activations(out_dim, in_dim, seed):
    """x = D * q with D a power of two and int8 codes q is exact in fp32 and is
    its own Q8_1 dequantization (d = D, s = D * sum q exactly): the fp32 path and
    the integer form (exact int64 sums, separate code) must agree to float64
    rounding.  Also terms >= sum |w x| >= |y|."""
    g = np.random.default_rng(70 + seed)
    blob = synth.q4k_weights(synth.rng(70 + seed, 1), out_dim, in_dim)
    D = 2.0 ** -5
    q = g.integers(-127, 128, (in_dim // 32, 32)).astype(np.int8)
    x = (D * q.astype(np.float64)).astype(np.float32).reshape(-1)
    xq = oracle.Q8Blocks(np.full(in_dim // 32, D, np.float32),
                         (D * q.astype(np.int64).sum(axis=1)).astype(np.float32), q)
    y, terms = oracle.gemv_q4k_f32(blob, x)
    y_int, _ = oracle.gemv_q4k_q8_int(blob, xq)
    assert np.all(np.abs(y - y_int) <= 1e-12 * terms)
    direct = np.abs(oracle.dequantize_q4k(blob)) @ np.abs(x.astype(np.float64))
    assert np.all(terms >= direct * (1 - 1e-12)) and np.all(direct >= np.abs(y) * (1 - 1e-12))


def test_q4k_f32_padding_invariance():
    """Zero activation values make their weights irrelevant, whatever the bytes."""
    blob = synth.q4k_weights(synth.rng(75, 1), 33, 1024)
    x = np.zeros(1024, np.float32)
    x[:896] = synth.activation(synth.rng(75, 0), 896)
    y1, t1 = oracle.gemv_q4k_f32(blob, x)
    b2 = blob.copy()
    b2[:, 3, 16 + 64:] = np.random.default_rng(3).integers(0, 256, (33, 64), dtype=np.uint8)
    y2, t2 = oracle.gemv_q4k_f32(b2, x)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("qn,S,M,Q,D", [(3, 5, 9, 7, 0.25), (15, 63, 63, -127, 0.5),
                                        (0, 40, 17, 100, 2.0), (9, 18, 0, -3, 1.0)])
def test_q4k_closed_form(qn, S, M, Q, D):
    """All nibbles qn, all scales S, all mins M, all activation codes Q with scale D:
    y = n_sub * 32 * Q * D * (d*S*qn - dmin*M)."""
    d, dmin, nsb = 0.0078125, 0.001953125, 3       # exact fp16 values
    sb = _f16le(d) + _f16le(dmin) + _pack_uniform_scales(S, M) + bytes([qn | (qn << 4)] * 128)
    blob = np.frombuffer(sb * nsb, np.uint8).reshape(1, nsb, 144).copy()
    nb = nsb * 8
    x = oracle.Q8Blocks(np.full(nb, D, np.float32), np.full(nb, 32 * Q * D, np.float32),
                        np.full((nb, 32), Q, np.int8))
    expect = nb * 32 * Q * D * (d * S * qn - dmin * M)
    y_int, _ = oracle.gemv_q4k_q8_int(blob, x)
    y_def = oracle.gemv_q4k_q8_def(blob, x)
    assert y_int[0] == pytest.approx(expect, rel=1e-13, abs=1e-12)
    assert y_def[0] == pytest.approx(expect, rel=1e-13, abs=1e-12)


@pytest.mark.parametrize("out_dim,in_dim,seed", [(1, 256, 0), (3, 512, 1), (65, 256, 2),
                                                 (257, 1024, 3), (40, 4096, 4)])
def test_q4k_integer_form_equals_definition(out_dim, in_dim, seed):
    """Dequantize-then-dot equals the integer formulation; the only gap is the
    fp32 rounding of s, at most 2**-24 * sum dmin*m*|s| (plus float64 slack)."""
    blob = synth.q4k_weights(synth.rng(50 + seed, 1), out_dim, in_dim)
    x = oracle.quantize_q8_1(synth.activation(synth.rng(50 + seed, 0), in_dim))
    y_int, terms = oracle.gemv_q4k_q8_int(blob, x)
    y_def = oracle.gemv_q4k_q8_def(blob, x)
    d, dmin, sc, m, q = oracle.q4k_fields(blob)
    min_mass = (dmin[..., None] * m * np.abs(x.s.astype(np.float64)).reshape(-1, 8)[None]).sum(axis=(1, 2))
    assert np.all(np.abs(y_int - y_def) <= U32 * min_mass + 1e-12 * terms)


def test_q4k_integer_exact_inputs():
    """d = dmin = 1, activation scale 1, codes in [-8, 8]: every term is an integer
    below 2**24, so the int form is exact and equals the definition exactly."""
    blob = synth.q4k_weights(synth.rng(60, 1), 37, 2048, d_fixed=1.0, dmin_fixed=1.0)
    g = np.random.default_rng(61)
    q = g.integers(-8, 9, size=(64, 32)).astype(np.int8)
    x = oracle.Q8Blocks(np.ones(64, np.float32), q.sum(axis=1).astype(np.float32), q)
    y_int, _ = oracle.gemv_q4k_q8_int(blob, x)
    y_def = oracle.gemv_q4k_q8_def(blob, x)
    assert np.array_equal(y_int, y_def)
    assert np.all(y_int == np.round(y_int)) and np.all(np.abs(y_int) < 2 ** 24)


def test_q4k_padding_invariance():
    """in_dim 896 padded to 1024: the last super-block's sub-blocks 4..7 meet zero
    activation blocks, so re-randomising their nibbles and 6-bit fields leaves y
    unchanged, and y equals the product over the first 896 values only."""
    n, in_dim, rows = 896, 1024, 64
    blob = synth.q4k_weights(synth.rng(0, 1), rows, in_dim)
    x = synth.activation(synth.rng(0, 0), n)
    xq = oracle.quantize_q8_1(x, in_dim)
    y, _ = oracle.gemv_q4k_q8_int(blob, xq)
    g = np.random.default_rng(99)
    b2 = blob.copy()
    b2[:, -1, 16 + 64:144] = g.integers(0, 256, (rows, 64), dtype=np.uint8)   # chunks 2,3
    # keep the low 6 bits of scale bytes 0..7 (sc/m of sub-blocks 0..3); their top
    # two bits and bytes 8..11 belong to sub-blocks 4..7 only
    r = g.integers(0, 256, (rows, 12), dtype=np.uint8)
    b2[:, -1, 4:12] = (blob[:, -1, 4:12] & 63) | (r[:, 0:8] & 0xC0)
    b2[:, -1, 12:16] = r[:, 8:12]
    sc0, m0 = oracle.q4k_unpack_scales(blob[:, -1, 4:16])
    sc1, m1 = oracle.q4k_unpack_scales(b2[:, -1, 4:16])
    assert np.array_equal(sc0[:, :4], sc1[:, :4]) and np.array_equal(m0[:, :4], m1[:, :4])
    assert not np.array_equal(sc0[:, 4:], sc1[:, 4:])
    y2, _ = oracle.gemv_q4k_q8_int(b2, xq)
    assert np.array_equal(y, y2)
    w = oracle.dequantize_q4k(blob)[:, :n]
    xh = oracle.dequantize_q8_1(xq)[:n]
    assert np.allclose(y, w @ xh, rtol=0, atol=1e-9 * np.abs(w).sum())


def test_q4k_row_permutation_and_scaling():
    blob = synth.q4k_weights(synth.rng(70, 1), 33, 512)
    xq = oracle.quantize_q8_1(synth.activation(synth.rng(70, 0), 512))
    y, _ = oracle.gemv_q4k_q8_int(blob, xq)
    perm = np.random.default_rng(1).permutation(33)
    yp, _ = oracle.gemv_q4k_q8_int(blob[perm], xq)
    assert np.array_equal(yp, y[perm])
    x2 = oracle.Q8Blocks(xq.d * np.float32(2), xq.s * np.float32(2), xq.q)
    y2, _ = oracle.gemv_q4k_q8_int(blob, x2)
    assert np.array_equal(y2, 2 * y)


def test_q4k_isum_brute_force_tiny():
    """Sub-block sums against a scalar loop over the bytes of one row."""
    blob = synth.q4k_weights(synth.rng(80, 1), 2, 256)
    xq = oracle.quantize_q8_1(synth.activation(synth.rng(80, 0), 256))
    _, _, isum = oracle.gemv_q4k_q8_int(blob, xq, return_isum=True)
    for r in range(2):
        qs = blob[r, 0, 16:144]
        for j in range(8):
            acc = 0
            for l in range(32):
                byte = int(qs[32 * (j // 2) + l])
                nib = byte & 0xF if j % 2 == 0 else byte >> 4
                acc += nib * int(xq.q[j, l])
            assert isum[r, 0, j] == acc


# ----------------------------------------------------------------- Q4_0
def _q4_0_fixture():
    fx = load("q4_0_block.txt")
    blob = np.frombuffer(hexbytes(fx["block_hex"]), np.uint8).reshape(1, 1, 18).copy()
    return fx, blob


def test_q4_0_hand_worked_block():
    fx, blob = _q4_0_fixture()
    w = oracle.dequantize_q4_0(blob)[0]
    for idx, val in pairs(fx["w_at"]):
        assert w[idx] == val
    for k, key in ((0, "y_onehot0"), (16, "y_onehot16")):
        x = np.zeros(32, np.float32)
        x[k] = 1.0
        assert oracle.gemv_q4_0_f32(blob, x)[0][0] == float(fx[key])
        assert oracle.gemv_q4_0_q8_int(blob, _onehot_q8(1, k))[0][0] == float(fx[key])


@pytest.mark.parametrize("qn,d", [(0, 0.5), (15, 0.0078125), (8, 1.0), (3, 2.0)])
def test_q4_0_closed_form(qn, d):
    nb = 5
    blob = np.frombuffer((_f16le(d) + bytes([qn | (qn << 4)] * 16)) * nb, np.uint8).reshape(1, nb, 18).copy()
    x = synth.activation(np.random.default_rng(qn), nb * 32)
    y, _ = oracle.gemv_q4_0_f32(blob, x)
    assert y[0] == pytest.approx(d * (qn - 8) * x.astype(np.float64).sum(), rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("rows,in_dim,seed", [(7, 64, 0), (130, 1024, 1)])
def test_q4_0_q8_variant_matches_fp32_on_dequantized_activation(rows, in_dim, seed):
    """Q4_0 x Q8_1 (integer form) equals dequantized weights times d*q."""
    blob = synth.q4_0_weights(synth.rng(90 + seed, 1), rows, in_dim)
    xq = oracle.quantize_q8_1(synth.activation(synth.rng(90 + seed, 0), in_dim))
    y8, t8 = oracle.gemv_q4_0_q8_int(blob, xq)
    w = oracle.dequantize_q4_0(blob)
    xh = oracle.dequantize_q8_1(xq)          # exact in float64
    assert np.all(np.abs(y8 - w @ xh) <= 1e-12 * t8)


def test_q4_0_padding_invariance():
    rows, n, in_dim = 16, 896, 1024
    blob = synth.q4_0_weights(synth.rng(3, 1), rows, in_dim)
    x = np.zeros(in_dim, np.float32)
    x[:n] = synth.activation(synth.rng(3, 0), n)
    y, _ = oracle.gemv_q4_0_f32(blob, x)
    b2 = blob.copy()
    # re-randomise the nibbles of the four padded blocks (their fp16 scales stay
    # finite: a padded weight is an ordinary finite weight meeting a zero value)
    b2[:, 28:, 2:18] = np.random.default_rng(5).integers(0, 256, (rows, 4, 16), dtype=np.uint8)
    y2, _ = oracle.gemv_q4_0_f32(b2, x)
    assert np.array_equal(y, y2)


# ----------------------------------------------------------------- SwiGLU
def test_silu_textbook_values():
    # silu(1) = sigma(1) = 1/(1+e^-1); silu(0) = 0; silu(x) -> x for large x, -> 0 for very negative x
    assert oracle.silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(50.0) == pytest.approx(50.0, rel=1e-15)
    assert abs(oracle.silu(-800.0)) == 0.0
    g = np.linspace(-20, 20, 81)
    assert np.allclose(oracle.silu(-g), oracle.silu(g) - g, rtol=0, atol=1e-12)


def test_silu_grad_by_finite_difference():
    g = np.linspace(-12, 12, 97)
    h = 1e-6
    fd = (oracle.silu(g + h) - oracle.silu(g - h)) / (2 * h)
    assert np.allclose(oracle.silu_grad(g), fd, rtol=0, atol=1e-8)
    from oracle.swiglu import SILU_CURV_MAX, SILU_GRAD_MAX
    dense = np.linspace(-30, 30, 60001)
    assert np.max(np.abs(oracle.silu_grad(dense))) <= SILU_GRAD_MAX
    curv = np.gradient(oracle.silu_grad(dense), dense)
    assert np.max(np.abs(curv)) <= SILU_CURV_MAX + 1e-6


def test_silu_curvature_by_finite_difference_and_bounds():
    """silu'' against a central difference of silu', at the textbook point
    silu''(0) = 1/2 and on a grid, also where sigma(g) rounds to 1; its sup and
    the Lipschitz constant of its second factor hold on a dense grid; and the
    interval bound used by the h bound is above a brute-force maximum of
    |silu''| over random intervals (and within a hair of it)."""
    from oracle.swiglu import SILU_A_LIP, SILU_CURV_MAX, silu_curv_bound
    assert oracle.silu_curv(0.0) == 0.5
    g = np.linspace(-40, 40, 161)
    h = 1e-5
    fd = (oracle.silu_grad(g + h) - oracle.silu_grad(g - h)) / (2 * h)
    assert np.allclose(oracle.silu_curv(g), fd, rtol=1e-5, atol=1e-9)
    dense = np.linspace(-80, 80, 1600001)
    assert np.max(np.abs(oracle.silu_curv(dense))) <= SILU_CURV_MAX
    a = 2.0 - dense * np.tanh(0.5 * dense)
    lip = np.max(np.abs(np.gradient(a, dense)))
    assert 1.19 < lip <= SILU_A_LIP
    rng = np.random.default_rng(3)
    gg = rng.uniform(-60, 60, 4000)
    r = 10.0 ** rng.uniform(-6, 0.3, 4000)
    xs = gg[:, None] + r[:, None] * np.linspace(-1, 1, 401)[None, :]
    sup = np.max(np.abs(oracle.silu_curv(xs)), axis=1)
    bound = silu_curv_bound(gg, r)
    assert np.all(sup <= bound * (1 + 1e-12))
    assert np.median(sup / bound) > 0.5



def _uniform_q4k(nsb, rows, qn, S, M, d=0.0078125, dmin=0.001953125):
    sb = _f16le(d) + _f16le(dmin) + _pack_uniform_scales(S, M) + bytes([qn | (qn << 4)] * 128)
    return np.frombuffer(sb * (nsb * rows), np.uint8).reshape(rows, nsb, 144).copy()


def test_ffn_chain_f32_closed_form():
    """Uniform gate, up and down matrices and a constant activation v: every g is
    gw*H*v, every u is uw*H*v (gw, uw the uniform weights), h = silu(g)*u in
    every row, and y = dw*I*fp32(h).  Gate and up differ, so swapping them (silu
    on the up projection) changes h."""
    H, I = 512, 768
    wg = _uniform_q4k(H // 256, I, 11, 30, 7)
    wu = _uniform_q4k(H // 256, I, 4, 9, 50)
    wd = _uniform_q4k(I // 256, H, 6, 20, 12)
    v = 2.0 ** -8                                            # g, u of order 1
    d, dmin = 0.0078125, 0.001953125
    gw, uw, dw = d * 30 * 11 - dmin * 7, d * 9 * 4 - dmin * 50, d * 20 * 6 - dmin * 12
    g, u = gw * H * v, uw * H * v
    h = g / (1.0 + np.exp(-g)) * u
    assert abs(h - u / (1.0 + np.exp(-u)) * g) > 0.1          # the swap is visible
    st = oracle.ffn_swiglu_q4k_f32(wg, wu, wd, np.full(H, v, np.float32))
    assert np.allclose(st["g"], g, rtol=1e-13) and np.allclose(st["u"], u, rtol=1e-13)
    assert np.allclose(st["h"], h, rtol=1e-13)
    assert np.allclose(st["y"], dw * I * float(np.float32(h)), rtol=1e-13)


def test_ffn_chain_zero_up_gives_zero():
    """u = 0 (all up scales zero) gives h = 0, all-zero Q8_1 blocks and y = 0."""
    hidden, inter = 256, 512
    wg = synth.q4k_weights(synth.rng(2, 1), inter, hidden)
    wu = synth.q4k_weights(synth.rng(2, 2), inter, hidden, d_fixed=0.0, dmin_fixed=0.0)
    wd = synth.q4k_weights(synth.rng(2, 3), hidden, inter)
    xq = oracle.quantize_q8_1(synth.activation(synth.rng(2, 0), hidden))
    st = oracle.ffn_swiglu_q4k(wg, wu, wd, xq)
    assert np.all(st["u"] == 0) and np.all(st["h"] == 0)
    assert np.all(st["h_q8"].d == 0) and np.all(st["h_q8"].q == 0) and np.all(st["h_q8"].s == 0)
    assert np.all(st["y"] == 0)


def test_ffn_chain_stages_compose():
    hidden, inter = 256, 512
    wg = synth.q4k_weights(synth.rng(2, 1), inter, hidden)
    wu = synth.q4k_weights(synth.rng(2, 2), inter, hidden)
    wd = synth.q4k_weights(synth.rng(2, 3), hidden, inter)
    xq = oracle.quantize_q8_1(synth.activation(synth.rng(2, 0), hidden))
    st = oracle.ffn_swiglu_q4k(wg, wu, wd, xq)
    assert np.array_equal(st["h"], oracle.silu(st["g"]) * st["u"])
    # the down projection of the fp64 h (no requantization) agrees with y to the
    # Q8_1 quantization error sum_k |w_k| * d_k / 2
    w = oracle.dequantize_q4k(wd)
    d_blocks = np.repeat(st["h_q8"].d.astype(np.float64), 32)
    assert np.all(np.abs(st["y"] - w @ st["h"]) <= np.abs(w) @ (d_blocks / 2) * (1 + 1e-6) + 1e-9)


def test_h_tolerance_covers_perturbations():
    g = np.random.default_rng(0).normal(0, 40, 4096)
    u = np.random.default_rng(1).normal(0, 40, 4096)
    tg = np.full_like(g, 0.01)
    tu = np.full_like(u, 0.01)
    h = oracle.swiglu(g, u)
    tol = oracle.h_tolerance(g, u, tg, tu, h)
    for sg, su in ((1, 1), (1, -1), (-1, 1), (-1, -1)):
        hp = oracle.swiglu(g + sg * tg, u + su * tu)
        assert np.all(np.abs(hp - h) <= tol)


def _swiglu_gpu_scale():
    """g, u and their GEMV bounds at the scale of the 4096 -> 14336 gate/up
    projections the GPU test checks (N(0, 1) activation through Q4_K weights
    drawn as the workload draws them; 512 rows keep this fast)."""
    import synth
    wg = synth.q4k_weights(synth.rng(2, synth.T_W0), 512, 4096)
    wu = synth.q4k_weights(synth.rng(2, synth.T_W0 + 1), 512, 4096)
    xq = oracle.quantize_q8_1(synth.activation(synth.rng(2, synth.T_ACT), 4096))
    g, tg = oracle.gemv_q4k_q8_int(wg, xq)
    u, tu = oracle.gemv_q4k_q8_int(wu, xq)
    return g, u, oracle.gemv_tolerance(tg), oracle.gemv_tolerance(tu)


def test_h_tolerance_rejects_planted_mistakes():
    """At the GPU test's scales the bound separates the SwiGLU definition from
    plausible mistakes in it: SiLU on the up projection instead of the gate,
    the SiLU dropped (h = g * u), SiLU with exp(+g), the up factor dropped.
    Some rows cannot show a mistake (silu(x) is about x for large positive x
    and about 0 for large negative x, so with g and u both large and of one
    sign the swap of g and u changes nothing), but each planted h falls
    outside the bound on more than a quarter of the rows, so the GPU check
    (every row within the bound) fails on any of them."""
    g, u, tg, tu = _swiglu_gpu_scale()
    h = oracle.swiglu(g, u)
    tol = oracle.h_tolerance(g, u, tg, tu, h)
    with np.errstate(over="ignore"):
        planted = {
            "silu on up": oracle.silu(u) * g,
            "no silu": g * u,
            "silu with exp(+g)": g / (1.0 + np.exp(g)) * u,
            "up dropped": oracle.silu(g),
        }
    for name, hp in planted.items():
        outside = np.abs(hp - h) > tol
        assert outside.mean() > 0.25, "%s: only %.3f of rows outside" % (name, outside.mean())


def test_h_tolerance_is_not_loose():
    """The bound stays within a small factor of what it bounds: the largest
    change of silu(g) * u when g and u move by their GEMV bounds (all four sign
    combinations) plus the fp32 rounding allowance, also where silu saturates
    (there the curvature bound decays with sigma'); a bound ten times looser
    fails this."""
    g, u, tg, tu = _swiglu_gpu_scale()
    h = oracle.swiglu(g, u)
    tol = oracle.h_tolerance(g, u, tg, tu, h)
    worst = np.zeros_like(h)
    for sg, su in ((1, 1), (1, -1), (-1, 1), (-1, -1)):
        worst = np.maximum(worst, np.abs(oracle.swiglu(g + sg * tg, u + su * tu) - h))
    worst = worst + 8.0 * 2.0 ** -24 * np.abs(h) + 1e-6
    # where silu is linear the bound equals the change exactly, up to float64 rounding
    assert np.all(tol >= worst * (1.0 - 1e-9))
    ratio = tol / worst
    assert np.median(ratio) < 1.5 and np.percentile(ratio, 99) < 3.0, (np.median(ratio),
                                                                      np.percentile(ratio, 99))
    assert np.median(10 * tol / worst) > 3.0       # what a ten-times looser bound would give


# ------------------------------------------------------------------ RMSNorm, residual
# using.rs rms_norm_inplace: RMS = sqrt(mean(x^2) + eps); x * (1 / RMS) * weight.

def test_rmsnorm_hand_worked():
    # [3, 4]: mean of squares 12.5 (a sum of 25 would give [0.6, 0.8]; no root, [0.24, 0.32])
    y = oracle.rmsnorm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert np.allclose(y, [3 / np.sqrt(12.5), 4 / np.sqrt(12.5)], rtol=0, atol=1e-15)
    assert abs(y[0] - 0.848528137423857) < 1e-14 and abs(y[1] - 1.131370849898476) < 1e-14


def test_rmsnorm_eps_inside_the_root():
    # mean 1, eps 3: RMS = sqrt(4) = 2 (eps added after the root would give 4)
    assert np.array_equal(oracle.rmsnorm(np.ones(4), np.ones(4), 3.0), np.full(4, 0.5))
    # all-zero input: the eps keeps it finite, and the output is zero
    assert np.array_equal(oracle.rmsnorm(np.zeros(8), np.ones(8), 1e-5), np.zeros(8))


def test_rmsnorm_weight_is_per_element():
    assert np.array_equal(oracle.rmsnorm(np.array([2.0, 2.0]), np.array([1.0, 3.0]), 0.0),
                          np.array([1.0, 3.0]))
    g = np.random.default_rng(5)
    x, w = g.normal(size=64), g.normal(1, 0.1, 64)
    assert np.array_equal(oracle.rmsnorm(x, 2 * w, 1e-5), 2 * oracle.rmsnorm(x, w, 1e-5))


def test_rmsnorm_unit_rms_and_scale_invariance():
    g = np.random.default_rng(6)
    x = g.normal(size=4096)
    y = oracle.rmsnorm(x, np.ones(4096), 0.0)
    assert abs(np.mean(y * y) - 1.0) < 1e-12
    for k in (0.25, 8.0, 2.0 ** -20):   # powers of two: exact with eps = 0
        assert np.array_equal(oracle.rmsnorm(k * x, np.ones(4096), 0.0), y)


def test_rmsnorm_rows_are_independent():
    g = np.random.default_rng(7)
    X = g.normal(size=(3, 96)) * np.array([[1.0], [100.0], [1e-3]])
    w = g.normal(1, 0.1, 96)
    Y = oracle.rmsnorm(X, w, 1e-5)
    for t in range(3):
        assert np.array_equal(Y[t], oracle.rmsnorm(X[t], w, 1e-5))


@pytest.mark.parametrize("n", [32, 896, 4096, 16384])
def test_rmsnorm_tolerance_covers_fp32_evaluations(n):
    """fp32 evaluations of the same formula -- a sequential sum as the pages
    write it, and numpy's blocked pairwise sum -- stay within the bound for
    their summation chains."""
    g = np.random.default_rng(n)
    x = g.normal(size=n).astype(np.float32)
    w = g.normal(1, 0.1, n).astype(np.float32)
    ref = oracle.rmsnorm(x, w, 1e-5)
    f = np.float32
    seq = f(0)
    for v in x:
        seq = f(seq + f(v * v))
    pair = np.sum(x * x, dtype=np.float32)
    for ss, chain in ((seq, n), (pair, 128 + int(np.ceil(np.log2(max(n / 128, 1)))) + 1)):
        scale = f(f(1) / f(np.sqrt(f(f(ss / f(n)) + f(1e-5)))))
        y32 = (x * scale) * w
        assert np.all(np.abs(y32.astype(np.float64) - ref) <= oracle.rmsnorm_tolerance(ref, chain))


def test_rmsnorm_tolerance_rejects_planted_mistakes():
    """At the chain length of a tree-shaped sum over 4096 values (24 dependent
    additions), the bound is tight enough to reject a dropped eps, a mean over
    n - 1 values and eps added after the root (each evaluated exactly, so only
    the mistake separates it from the definition)."""
    g = np.random.default_rng(9)
    n = 4096
    x = g.normal(size=n)
    w = g.normal(1, 0.1, n)
    eps = 1e-5
    ref = oracle.rmsnorm(x, w, eps)
    tol = oracle.rmsnorm_tolerance(ref, 24)
    ms = np.mean(x * x)
    planted = {
        "eps dropped": x / np.sqrt(ms) * w,
        "mean over n-1": x / np.sqrt(np.sum(x * x) / (n - 1) + eps) * w,
        "eps after the root": x / (np.sqrt(ms) + eps) * w,
    }
    for name, y in planted.items():
        assert np.all(np.abs(y - ref) > tol), name


def test_residual_add():
    r = np.array([1.0, -2.0, 0.5])
    assert np.array_equal(oracle.residual_add(r, np.array([0.25, 2.0, -0.5])), [1.25, 0.0, 0.0])


# ----------------------------------------------------------------- LM head
def test_argmax_first_tie_rule_and_special_cases():
    assert oracle.argmax_first([1.0]) == 0
    assert oracle.argmax_first([3.0, 7.0, 7.0, -1.0]) == 1          # first of equal maxima
    assert oracle.argmax_first([-5.0, -2.0, -3.0]) == 1              # all negative
    assert oracle.argmax_first([0.0, -0.0, 0.0]) == 0                # signed zeros are equal
    assert oracle.argmax_first([-0.0, 0.0]) == 0
    assert oracle.argmax_first(np.full(17, 2.5)) == 0
    assert oracle.argmax_first([1.0, 2.0, 3.0, 3.0000002]) == 3


def test_argmax_first_matches_numpy_on_random_ties():
    g = np.random.default_rng(1)
    for _ in range(50):
        v = g.integers(-3, 4, g.integers(1, 40)).astype(np.float32)   # many ties
        assert oracle.argmax_first(v) == int(np.argmax(v))


def test_topk_first_hand_worked():
    # [3, 1, 3, -0.0, +0.0, 2]: the two 3s in index order, then 2, 1, then the
    # signed zeros (equal) in index order
    v = np.array([3.0, 1.0, 3.0, -0.0, 0.0, 2.0], np.float32)
    idx, val = oracle.topk_first(v, 4)
    assert idx.tolist() == [0, 2, 5, 1] and val.tolist() == [3.0, 3.0, 2.0, 1.0]
    idx, _ = oracle.topk_first(v, 6)
    assert idx.tolist() == [0, 2, 5, 1, 3, 4]
    idx, _ = oracle.topk_first(np.full(9, -1.5, np.float32), 3)
    assert idx.tolist() == [0, 1, 2]


def test_topk_first_by_repeated_argmax():
    """Against an independent definition: the first of the top k is the greedy
    token; remove it and the next is the greedy token of the rest; and so on.
    Random small arrays with many ties (integers, both signed zeros)."""
    g = np.random.default_rng(7)
    for _ in range(60):
        n = int(g.integers(1, 40))
        v = g.integers(-3, 4, n).astype(np.float32)
        v[g.random(n) < 0.2] = -0.0
        k = int(g.integers(1, n + 1))
        idx, val = oracle.topk_first(v, k)
        rest = list(range(n))
        want = []
        for _ in range(k):
            j = rest[oracle.argmax_first(v[rest])]
            want.append(j)
            rest.remove(j)
        assert idx.tolist() == want
        assert np.array_equal(val, v[want])


def test_topk_first_k1_and_full_order():
    g = np.random.default_rng(8)
    v = g.standard_normal(1000).astype(np.float32)
    v[::7] = v[3]                                   # ties
    idx, _ = oracle.topk_first(v, 1)
    assert idx.tolist() == [oracle.argmax_first(v)]
    idx, val = oracle.topk_first(v, v.size)
    assert sorted(idx.tolist()) == list(range(v.size))             # a permutation
    assert np.all(val[:-1] >= val[1:])                            # descending
    eq = val[:-1] == val[1:]
    assert np.all(idx[:-1][eq] < idx[1:][eq])                     # ties by index


def test_lm_head_bias_closed_form():
    """Uniform Q4_0 weights w and activation v give v*in_dim*w in every row; the
    bias shifts each row by its own value, and it moves the greedy token."""
    d, qn, in_dim, rows = 0.0078125, 11, 128, 5
    blk = np.array([d], np.float16).tobytes() + bytes([qn | (qn << 4)] * 16)
    blob = np.frombuffer(blk * (rows * in_dim // 32), np.uint8).reshape(rows, in_dim // 32, 18).copy()
    x = np.full(in_dim, 0.5, np.float32)
    base = 0.5 * in_dim * (qn - 8) * d
    bias = np.array([0.0, 1.0, -1.0, 2.0, 1.5], np.float32)
    y, terms = oracle.lm_head_q4_0(blob, x, bias)
    assert np.allclose(y, base + bias.astype(np.float64), rtol=0, atol=1e-12)
    y0, t0 = oracle.lm_head_q4_0(blob, x)
    assert np.allclose(terms - t0, np.abs(bias.astype(np.float64)), rtol=0, atol=1e-12)
    assert oracle.argmax_first(y0) == 0 and oracle.argmax_first(y) == 3


# ----------------------------------------------------------------- GELU FFN
def test_gelu_against_the_erf_definition():
    """The tanh form stays within 5e-4 of x * Phi(x) (scipy's erf, an independent
    routine); a wrong constant or a missing sqrt(2/pi) moves it much further."""
    from scipy.special import erf
    u = np.linspace(-10, 10, 200001)
    exact = 0.5 * u * (1.0 + erf(u / np.sqrt(2.0)))
    assert np.max(np.abs(oracle.gelu(u) - exact)) < 5e-4
    wrong_c = 0.5 * u * (1.0 + np.tanh(np.sqrt(2 / np.pi) * (u + 0.44715 * u ** 3)))
    wrong_k = 0.5 * u * (1.0 + np.tanh(u + 0.044715 * u ** 3))
    assert np.max(np.abs(wrong_c - exact)) > 1e-2 and np.max(np.abs(wrong_k - exact)) > 1e-2


def test_gelu_identities_and_limits():
    u = np.linspace(-30, 30, 6001)
    # gelu(u) - gelu(-u) = u, and the sigmoid form used on the device is the same function
    assert np.allclose(oracle.gelu(u) - oracle.gelu(-u), u, rtol=0, atol=1e-12)
    z = np.sqrt(2 / np.pi) * (u + 0.044715 * u ** 3)
    with np.errstate(over="ignore"):
        sig_form = u / (1.0 + np.exp(-2.0 * z))
    # the tanh form cancels for negative u (1 + tanh z), so compare with an
    # allowance of a few float64 ulps of |u|
    assert np.all(np.abs(sig_form - oracle.gelu(u)) <= 1e-13 * np.abs(sig_form) + 1e-15 * np.abs(u))
    assert oracle.gelu(0.0) == 0.0
    assert oracle.gelu(10.0) == pytest.approx(10.0, rel=1e-15)
    assert abs(oracle.gelu(-10.0)) < 1e-40


def test_gelu_grad_by_finite_difference_and_bounds():
    from oracle.gelu import GELU_CURV_MAX, GELU_GRAD_MAX
    u = np.linspace(-8, 8, 1601)
    h = 1e-6
    fd = (oracle.gelu(u + h) - oracle.gelu(u - h)) / (2 * h)
    assert np.allclose(oracle.gelu_grad(u), fd, rtol=0, atol=1e-8)
    dense = np.linspace(-12, 12, 1200001)
    g = oracle.gelu_grad(dense)
    assert np.max(np.abs(g)) <= GELU_GRAD_MAX
    assert np.max(np.abs(np.gradient(g, dense))) <= GELU_CURV_MAX


def _uniform_q4_0(rows, in_dim, qn, d):
    blk = np.array([d], np.float16).tobytes() + bytes([qn | (qn << 4)] * 16)
    return np.frombuffer(blk * (rows * in_dim // 32), np.uint8).reshape(rows, in_dim // 32, 18).copy()


def test_ffn_gelu_chain_closed_form():
    """Zero up weights make u the up bias exactly; uniform down weights w make
    every y equal w * sum(fp32(gelu(b))) + down bias.  Biases on both sides are
    exercised, and the order (bias before GELU) is visible."""
    H, I = 128, 192
    wu = _uniform_q4_0(I, H, 5, 0.0)
    d, qn = 0.0078125, 13
    wd = _uniform_q4_0(H, I, qn, d)
    g = np.random.default_rng(2)
    x = g.standard_normal(H).astype(np.float32)
    ub = g.standard_normal(I).astype(np.float32)
    db = g.standard_normal(H).astype(np.float32)
    st = oracle.ffn_gelu_q4_0(wu, wd, x, ub, db)
    assert np.array_equal(st["u"], ub.astype(np.float64))
    h32 = oracle.gelu(ub.astype(np.float64)).astype(np.float32)
    assert np.array_equal(st["h32"], h32)
    w = (qn - 8) * d
    assert np.allclose(st["y"], w * h32.astype(np.float64).sum() + db, rtol=1e-13, atol=1e-12)
    # GELU of (0 + bias) differs from GELU(0) + bias
    assert not np.allclose(oracle.gelu(ub), ub)


def _gelu_gpu_scale():
    """The GELU FFN's up projection at the phi-2 size the GPU test checks
    (2560 -> 10240, Q4_0 weights, N(0, 1) activation and bias; 1024 rows)."""
    import synth
    w = synth.q4_0_weights(synth.rng(5, 1), 1024, 2560)
    x = synth.activation(synth.rng(5, synth.T_ACT), 2560)
    b = synth.activation(synth.rng(5, 7), 1024).astype(np.float64)
    u0, tu = oracle.gemv_q4_0_f32(w, x)
    return u0, b, u0 + b, oracle.gemv_tolerance(tu + np.abs(b))


def _gelu_device_form_f32(u):
    """GELU the way the device evaluates it, in fp32 throughout:
    u / (1 + exp(-2 sqrt(2/pi) (u + 0.044715 u^3)))."""
    u = np.asarray(u, np.float32)
    k2 = np.float32(2.0 * np.sqrt(2.0 / np.pi))
    c = np.float32(0.044715)
    with np.errstate(over="ignore"):
        z = (-k2 * (u + c * u * u * u)).astype(np.float32)
        return (u / (np.float32(1.0) + np.exp(z).astype(np.float32))).astype(np.float32)


def test_gelu_h_tolerance_covers_device_form_and_perturbations():
    """The bound covers (a) an fp32 evaluation of the device's sigmoid form of
    GELU on the oracle's exact pre-activations, and (b) GELU of the
    pre-activation moved by its GEMV bound either way."""
    _, _, u, tol_u = _gelu_gpu_scale()
    h = oracle.gelu(u)
    tol = oracle.gelu_h_tolerance(u, tol_u, h)
    dev = _gelu_device_form_f32(u.astype(np.float32)).astype(np.float64)
    # the fp32 cast of u is itself a perturbation well inside tol_u
    assert np.all(np.abs(u.astype(np.float32).astype(np.float64) - u) <= tol_u)
    assert np.all(np.abs(dev - h) <= tol)
    for sgn in (1.0, -1.0):
        assert np.all(np.abs(oracle.gelu(u + sgn * tol_u) - h) <= tol)


def test_gelu_h_tolerance_rejects_planted_mistakes():
    """At the GPU test's scales the bound rejects plausible mistakes in the GELU
    stage: the cubic term dropped, its coefficient off by a decimal place, 2/pi
    for sqrt(2/pi), the bias added after GELU instead of before, and the exact
    erf form of GELU in place of the tanh form taken here.  Each falls outside
    the bound on more than a quarter of the rows (near u = 0 and for large |u|
    the forms agree), so the GPU check (every row within the bound) fails on
    any of them."""
    from scipy.special import erf
    u0, b, u, tol_u = _gelu_gpu_scale()
    h = oracle.gelu(u)
    tol = oracle.gelu_h_tolerance(u, tol_u, h)
    k = np.sqrt(2.0 / np.pi)

    def tanh_gelu(v, kk, cc):
        return 0.5 * v * (1.0 + np.tanh(kk * (v + cc * v ** 3)))
    planted = {
        "cubic term dropped": tanh_gelu(u, k, 0.0),
        "0.44715 for 0.044715": tanh_gelu(u, k, 0.44715),
        "2/pi for sqrt(2/pi)": tanh_gelu(u, 2.0 / np.pi, 0.044715),
        "bias after GELU": oracle.gelu(u0) + b,
        "erf form": 0.5 * u * (1.0 + erf(u / np.sqrt(2.0))),
    }
    for name, hp in planted.items():
        outside = np.abs(hp - h) > tol
        assert outside.mean() > 0.25, "%s: only %.3f of rows outside" % (name, outside.mean())


def test_gelu_h_tolerance_is_not_loose():
    """The bound stays within a small factor of the change of GELU over the
    pre-activation's GEMV bound plus the fp32 rounding allowance (a bound ten
    times looser fails this), away from the stationary point of GELU near
    u = -0.75 where its slope vanishes."""
    _, _, u, tol_u = _gelu_gpu_scale()
    h = oracle.gelu(u)
    tol = oracle.gelu_h_tolerance(u, tol_u, h)
    worst = np.maximum(np.abs(oracle.gelu(u + tol_u) - h), np.abs(oracle.gelu(u - tol_u) - h))
    worst = worst + 8.0 * 2.0 ** -24 * np.abs(h) + 1e-6
    assert np.all(tol >= worst * (1.0 - 1e-9))
    away = np.abs(oracle.gelu_grad(u)) > 0.05
    ratio = tol[away] / worst[away]
    assert np.median(ratio) < 1.5 and np.percentile(ratio, 99) < 3.0, (np.median(ratio),
                                                                      np.percentile(ratio, 99))
