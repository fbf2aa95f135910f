"""GPU test of rz_lm_head_q4_0_noalloc, the LM head whose argmax pairs live in
the library's fixed per-GPU array (for callers that cannot allocate), against
rz_lm_head_q4_0 with a caller workspace: calls in a row on one GPU, each
smaller than the one before, logits and greedy token bit for bit.

The first call's largest logit is planted far above anything later calls can
produce, so a later call that read a pair left over from an earlier one would
return the planted row instead of its own."""
import numpy as np
import pytest

import oracle
import synth
import q4_q8_integer_quantize_amd as rz
from gpu_util import banner, dev_bytes, dev_f32, empty_bytes, empty_f32, host

pytestmark = pytest.mark.gpu


def _heads(blob, x, fmt, bias):
    """(logits, idx, val) from the workspace entry and from the no-alloc entry."""
    torch = __import__("torch")
    out_dim, nb, _ = blob.shape
    in_dim = nb * 32
    wd = dev_bytes(blob)
    xd = dev_f32(x) if fmt == 0 else dev_bytes(x)
    bd = dev_f32(bias) if bias is not None else None
    res = []
    for noalloc in (False, True):
        logits = empty_f32(out_dim)
        idx = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        val = empty_f32(1)
        if noalloc:
            rz.rz_lm_head_q4_0_noalloc(wd, xd, fmt, bd, logits, out_dim, in_dim, idx, val)
        else:
            ws = empty_bytes(rz.rz_lm_head_q4_0_workspace_bytes(out_dim, in_dim, fmt))
            rz.rz_lm_head_q4_0(wd, xd, fmt, bd, logits, out_dim, in_dim, idx, val, ws)
        res.append((host(logits), int(host(idx)[0]), host(val)[0]))
    return res


@pytest.mark.parametrize("fmt", [0, 1])
def test_noalloc_lm_head_equals_workspace_entry_in_a_row(fmt):
    banner("noalloc lm head", fmt)
    calls = [(151936, 1024, True), (20000, 1024, False), (777, 2048, True)]
    planted = 151000
    for k, (out_dim, in_dim, with_bias) in enumerate(calls):
        blob = synth.q4_0_weights(synth.rng(90 + k, 1), out_dim, in_dim)
        x = synth.activation(synth.rng(90 + k, 0), in_dim)
        xin = x if fmt == 0 else oracle.q8_1_to_bytes(oracle.quantize_q8_1(x))
        bias = synth.activation(synth.rng(90 + k, 2), out_dim) if with_bias else None
        if k == 0:
            bias[planted] = np.float32(1.0e6)
        (lg_ws, i_ws, v_ws), (lg_na, i_na, v_na) = _heads(blob, xin, fmt, bias)
        assert np.array_equal(lg_na.view(np.uint32), lg_ws.view(np.uint32)), "call %d logits" % k
        assert i_na == i_ws and np.float32(v_na).tobytes() == np.float32(v_ws).tobytes(), \
            "call %d: greedy token %d (%r) against %d (%r)" % (k, i_na, v_na, i_ws, v_ws)
        assert i_na == oracle.argmax_first(lg_na)
        if k == 0:
            assert i_na == planted
        else:
            assert i_na < out_dim


def test_noalloc_lm_head_without_argmax():
    """Without argmax outputs the call does not use the array and gives the
    same logits as the workspace entry; a call with the argmax right after
    still agrees with it."""
    banner("noalloc lm head, no argmax")
    blob = synth.q4_0_weights(synth.rng(95, 1), 4096, 1024)
    x = synth.activation(synth.rng(95, 0), 1024)
    wd, xd = dev_bytes(blob), dev_f32(x)
    a, b = empty_f32(4096), empty_f32(4096)
    rz.rz_lm_head_q4_0(wd, xd, 0, None, a, 4096, 1024)
    rz.rz_lm_head_q4_0_noalloc(wd, xd, 0, None, b, 4096, 1024)
    assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32))
    (lg_ws, i_ws, _), (lg_na, i_na, _) = _heads(blob, x, 0, None)
    assert np.array_equal(lg_na.view(np.uint32), lg_ws.view(np.uint32)) and i_na == i_ws
