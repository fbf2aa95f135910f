"""Host-only checks of the C ABI: librz.so loads, exports every function that
include/rz.h declares, and rejects bad arguments before any HIP call.

The rejection calls pass made-up device addresses, so they run in a child
process that sees no GPU (ROCR_VISIBLE_DEVICES=-1): should a case ever pass
validation by mistake, its launch fails for want of a device instead of
touching memory.  Such a case shows up as RZ_ELAUNCH and fails its test."""
import ctypes
import json
import os
import re
import subprocess
import sys

import pytest

import q4_q8_integer_quantize_amd as rz

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rz.h")

# plausible-looking device addresses; validation never dereferences them
P = 0x7f0000000000
P_ODD = P + 2


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s*(rz_\w+)\s*\(", text,
                                 re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rz.library_path()):
        pytest.skip("librz.so not built")
    return rz.load_library()


def test_header_declares_the_four_operations():
    syms = declared_symbols()
    for name in ("rz_q8_1_quantize", "rz_q4k_q8_gemv", "rz_q4k_q8_gemv_f32", "rz_q4_0_gemv",
                 "rz_swiglu_ffn_q4k", "rz_q4k_q8_gemv_multi", "rz_rmsnorm_q8_1",
                 "rz_q4k_q8_gemv_add", "rz_swiglu_ffn_q4k_add", "rz_q4k_gemv",
                 "rz_rmsnorm_q4k_q8_gemv_multi", "rz_rmsnorm_swiglu_ffn_q4k_add",
                 "rz_q4k_q8_gemv_f32_add",
                 "rz_swiglu_ffn_q4k_f32", "rz_lm_head_q4_0", "rz_lm_head_q4_0_workspace_bytes",
                 "rz_lm_head_q4_0_noalloc", "rz_gelu_ffn_q4_0",
                 "rz_topk_f32", "rz_topk_f32_workspace_bytes", "rz_lm_head_q4_0_topk",
                 "rz_last_error",
                 "rz_abi_version"):
        assert name in syms


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(rz.library_path())
    for name in declared_symbols():
        assert hasattr(raw, name), name


def test_abi_version(lib):
    assert rz.rz_abi_version() == 100


_CHILD = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import q4_q8_integer_quantize_amd as rz
lib = rz.load_library(preload_torch=False)   # no kernel runs here
out = []
import ctypes
def conv(a):
    # {"p": [...]} -> a host array of pointers, {"i": [...]} -> a host int array
    if isinstance(a, dict) and "p" in a:
        return (ctypes.c_void_p * max(1, len(a["p"])))(*a["p"])
    if isinstance(a, dict) and "i" in a:
        return (ctypes.c_int * max(1, len(a["i"])))(*a["i"])
    return a
for fn, args in json.loads(sys.stdin.read()):
    rc = getattr(lib, fn)(*[conv(a) for a in args])
    out.append([rc, rz.rz_last_error()])
print(json.dumps(out))
"""


def run_isolated(calls):
    """[(fn, args)] -> [(rc, message)], executed in a GPU-less child process."""
    env = dict(os.environ, ROCR_VISIBLE_DEVICES="-1", HIP_VISIBLE_DEVICES="-1")
    res = subprocess.run([sys.executable, "-c", _CHILD, ROOT], input=json.dumps(calls),
                         capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stderr
    return [tuple(x) for x in json.loads(res.stdout.strip().splitlines()[-1])]


def _rc(fn, *args):
    rc, msg = run_isolated([(fn, list(args))])[0]
    _rc.last = msg
    return rc


@pytest.mark.parametrize("args,code", [
    ((None, 896, 1024, 1, P, None), rz.RZ_EINVAL),          # null x
    ((P, 896, 1024, 1, None, None), rz.RZ_EINVAL),          # null out
    ((P, 896, 1024, 0, P, None), rz.RZ_EINVAL),             # n_tokens 0
    ((P, 896, 1024, 9, P, None), rz.RZ_EINVAL),             # n_tokens 9
    ((P, 896, 1000, 1, P, None), rz.RZ_EDIM),               # n_padded % 32
    ((P, 1025, 1024, 1, P, None), rz.RZ_EDIM),              # n > n_padded
    ((P, 0, 1024, 1, P, None), rz.RZ_EDIM),                 # n == 0
    ((P, 896, 0, 1, P, None), rz.RZ_EDIM),                  # n_padded == 0
    ((P_ODD, 896, 1024, 1, P, None), rz.RZ_EALIGN),         # x not 4-aligned
    ((P, 896, 1024, 1, P + 4, None), rz.RZ_EALIGN),         # x_q8 not 16-aligned
    ((P, 896, 1024, 1, P + 8, None), rz.RZ_EALIGN),
])
def test_q8_1_quantize_rejects(lib, args, code):
    assert _rc("rz_q8_1_quantize", *args) == code
    assert _rc.last.startswith("rz_q8_1_quantize")


@pytest.mark.parametrize("args,code", [
    ((None, P, P, 14336, 4096, 1, None), rz.RZ_EINVAL),
    ((P, None, P, 14336, 4096, 1, None), rz.RZ_EINVAL),
    ((P, P, None, 14336, 4096, 1, None), rz.RZ_EINVAL),
    ((P, P, P, 14336, 4096, 0, None), rz.RZ_EINVAL),
    ((P, P, P, 14336, 4096, 9, None), rz.RZ_EINVAL),
    ((P, P, P, 14336, 896, 1, None), rz.RZ_EDIM),           # unpadded in_dim
    ((P, P, P, 14336, 0, 1, None), rz.RZ_EDIM),
    ((P, P, P, 0, 4096, 1, None), rz.RZ_EDIM),
    ((P, P, P, -5, 4096, 1, None), rz.RZ_EDIM),
    ((P, P, P, 14336, 1 << 25, 1, None), rz.RZ_EDIM),
    ((P + 8, P, P, 14336, 4096, 1, None), rz.RZ_EALIGN),    # weights need 16
    ((P, P + 4, P, 14336, 4096, 1, None), rz.RZ_EALIGN),
    ((P, P + 8, P, 14336, 4096, 1, None), rz.RZ_EALIGN),    # Q8_1 activations need 16
    ((P, P, P_ODD, 14336, 4096, 1, None), rz.RZ_EALIGN),
])
def test_q4k_q8_gemv_rejects(lib, args, code):
    assert _rc("rz_q4k_q8_gemv", *args) == code
    assert "rz_q4k_q8_gemv" in _rc.last


def _m(ws, ys, ods):
    return {"p": ws}, {"p": ys}, {"i": ods}


@pytest.mark.parametrize("args,code", [
    ((3,) + _m([P, P, P], [P, P, P], [4096, 1024, 1024]) + (P, 4096, 9, None), rz.RZ_EINVAL),
    ((0,) + _m([P], [P], [4096]) + (P, 4096, 1, None), rz.RZ_EINVAL),          # n_mats 0
    ((9,) + _m([P] * 9, [P] * 9, [16] * 9) + (P, 4096, 1, None), rz.RZ_EINVAL),  # n_mats 9
    ((2,) + _m([P, 0], [P, P], [16, 16]) + (P, 4096, 1, None), rz.RZ_EINVAL),  # null entry
    ((2,) + _m([P, P], [P, 0], [16, 16]) + (P, 4096, 1, None), rz.RZ_EINVAL),
    ((2,) + _m([P, P], [P, P], [16, 16]) + (None, 4096, 1, None), rz.RZ_EINVAL),
    ((2,) + _m([P, P], [P, P], [16, 0]) + (P, 4096, 1, None), rz.RZ_EDIM),     # empty matrix
    ((2,) + _m([P, P], [P, P], [16, 16]) + (P, 4000, 1, None), rz.RZ_EDIM),
    ((2,) + _m([P, P + 8], [P, P], [16, 16]) + (P, 4096, 1, None), rz.RZ_EALIGN),
    ((2,) + _m([P, P], [P, P_ODD], [16, 16]) + (P, 4096, 1, None), rz.RZ_EALIGN),
    ((2,) + _m([P, P], [P, P], [16, 16]) + (P + 4, 4096, 1, None), rz.RZ_EALIGN),
    ((1,) + _m([P], [P], [1 << 20]) + (P, 1 << 14, 1, None), rz.RZ_EDIM),      # > 2 GiB
])
def test_q4k_q8_gemv_multi_rejects(lib, args, code):
    assert _rc("rz_q4k_q8_gemv_multi", *args) == code
    assert _rc.last.startswith("rz_q4k_q8_gemv_multi")


@pytest.mark.parametrize("args,code", [
    ((None, P, 4096, P, P, 14336, 4096, None), rz.RZ_EINVAL),
    ((P, None, 4096, P, P, 14336, 4096, None), rz.RZ_EINVAL),
    ((P, P, 4096, P, None, 14336, 4096, None), rz.RZ_EINVAL),
    ((P, P, 4096, P, P, 14336, 4000, None), rz.RZ_EDIM),
    ((P, P, 4097, P, P, 14336, 4096, None), rz.RZ_EDIM),     # n > in_dim
    ((P, P, 0, P, P, 14336, 4096, None), rz.RZ_EDIM),
    ((P, P, 20480, P, P, 14336, 20480, None), rz.RZ_EDIM),   # above the fused limit
    ((P, P, 4096, P, P, 0, 4096, None), rz.RZ_EDIM),
    ((P + 8, P, 4096, P, P, 14336, 4096, None), rz.RZ_EALIGN),
    ((P, P_ODD, 4096, P, P, 14336, 4096, None), rz.RZ_EALIGN),
    ((P, P, 4096, P + 4, P, 14336, 4096, None), rz.RZ_EALIGN),
])
def test_q4k_q8_gemv_f32_rejects(lib, args, code):
    assert _rc("rz_q4k_q8_gemv_f32", *args) == code


@pytest.mark.parametrize("args,code", [
    ((None, P, 0, P, 151936, 1024, None), rz.RZ_EINVAL),
    ((P, P, 2, P, 151936, 1024, None), rz.RZ_EINVAL),       # unknown format
    ((P, P, -1, P, 151936, 1024, None), rz.RZ_EINVAL),
    ((P, P, 0, P, 151936, 800, None), rz.RZ_EDIM),          # 800 % 64 != 0
    ((P, P, 0, P, 151936, 32, None), rz.RZ_EDIM),
    ((P, P, 0, P, 0, 1024, None), rz.RZ_EDIM),
    ((P_ODD, P, 0, P, 151936, 1024, None), rz.RZ_EALIGN),
    ((P, P + 8, 0, P, 151936, 1024, None), rz.RZ_EALIGN),   # fp32 x needs 16
    ((P, P + 4, 1, P, 151936, 1024, None), rz.RZ_EALIGN),   # Q8_1 x needs 8
    ((P, P, 0, P_ODD, 151936, 1024, None), rz.RZ_EALIGN),
])
def test_q4_0_gemv_rejects(lib, args, code):
    assert _rc("rz_q4_0_gemv", *args) == code


@pytest.mark.parametrize("args,code", [
    ((None, P, P, P, P, P, P, None, 4096, 14336, None), rz.RZ_EINVAL),
    ((P, P, P, P, None, P, P, None, 4096, 14336, None), rz.RZ_EINVAL),
    ((P, P, P, P, P, P, None, None, 4096, 14336, None), rz.RZ_EINVAL),
    ((P, P, P, P, P, P, P, None, 4000, 14336, None), rz.RZ_EDIM),
    ((P, P, P, P, P, P, P, None, 4096, 14000, None), rz.RZ_EDIM),
    ((P, P, P, P, P, P, P, None, 32768, 14336, None), rz.RZ_EDIM),   # hidden above fused limit
    ((P + 8, P, P, P, P, P, P, None, 4096, 14336, None), rz.RZ_EALIGN),
    ((P, P, P, P + 4, P, P, P, None, 4096, 14336, None), rz.RZ_EALIGN),
    ((P, P, P, P, P, P, P, P_ODD, 4096, 14336, None), rz.RZ_EALIGN),
])
def test_swiglu_ffn_rejects(lib, args, code):
    assert _rc("rz_swiglu_ffn_q4k", *args) == code


@pytest.mark.parametrize("args,code", [
    ((None, P, 1e-5, 4096, 4096, 1, None, P, None), rz.RZ_EINVAL),       # null x
    ((P, None, 1e-5, 4096, 4096, 1, None, P, None), rz.RZ_EINVAL),       # null gamma
    ((P, P, 1e-5, 4096, 4096, 1, None, None, None), rz.RZ_EINVAL),       # null x_q8
    ((P, P, 1e-5, 4096, 4096, 0, None, P, None), rz.RZ_EINVAL),          # n_tokens 0
    ((P, P, 1e-5, 4096, 4096, 9, None, P, None), rz.RZ_EINVAL),          # n_tokens 9
    ((P, P, 0.0, 4096, 4096, 1, None, P, None), rz.RZ_EINVAL),           # eps 0
    ((P, P, -1e-5, 4096, 4096, 1, None, P, None), rz.RZ_EINVAL),         # eps < 0
    ((P, P, float("inf"), 4096, 4096, 1, None, P, None), rz.RZ_EINVAL),  # eps inf
    ((P, P, float("nan"), 4096, 4096, 1, None, P, None), rz.RZ_EINVAL),  # eps NaN
    ((P, P, 1e-5, 896, 1000, 1, None, P, None), rz.RZ_EDIM),             # n_padded % 32
    ((P, P, 1e-5, 1025, 1024, 1, None, P, None), rz.RZ_EDIM),            # n > n_padded
    ((P, P, 1e-5, 0, 1024, 1, None, P, None), rz.RZ_EDIM),               # n == 0
    ((P_ODD, P, 1e-5, 896, 1024, 1, None, P, None), rz.RZ_EALIGN),       # x
    ((P, P_ODD, 1e-5, 896, 1024, 1, None, P, None), rz.RZ_EALIGN),       # gamma
    ((P, P, 1e-5, 896, 1024, 1, P_ODD, P, None), rz.RZ_EALIGN),          # normed
    ((P, P, 1e-5, 896, 1024, 1, None, P + 4, None), rz.RZ_EALIGN),       # x_q8
])
def test_rmsnorm_q8_1_rejects(lib, args, code):
    assert _rc("rz_rmsnorm_q8_1", *args) == code
    assert _rc.last.startswith("rz_rmsnorm_q8_1")


Y = P + (1 << 30)   # a y buffer far from P
@pytest.mark.parametrize("args,code", [
    ((None, P, P, Y, 4096, 4096, 1, None), rz.RZ_EINVAL),
    ((P, None, P, Y, 4096, 4096, 1, None), rz.RZ_EINVAL),
    ((P, P, None, Y, 4096, 4096, 1, None), rz.RZ_EINVAL),          # null r
    ((P, P, P, None, 4096, 4096, 1, None), rz.RZ_EINVAL),
    ((P, P, P, Y, 4096, 4096, 0, None), rz.RZ_EINVAL),
    ((P, P, P, Y, 4096, 4096, 9, None), rz.RZ_EINVAL),
    ((P, P, Y + 4, Y, 4096, 4096, 1, None), rz.RZ_EINVAL),         # r overlaps y, not equal
    ((P, P, Y - 4 * 4095, Y, 4096, 4096, 1, None), rz.RZ_EINVAL),  # overlap by one value
    ((P, P, Y, Y + 4 * 4096 * 2, 4096, 4096, 3, None), rz.RZ_EINVAL),  # 3 tokens: overlaps
    ((P, P, P, Y, 4096, 896, 1, None), rz.RZ_EDIM),
    ((P, P, P, Y, 0, 4096, 1, None), rz.RZ_EDIM),
    ((P + 8, P, P, Y, 4096, 4096, 1, None), rz.RZ_EALIGN),
    ((P, P + 4, P, Y, 4096, 4096, 1, None), rz.RZ_EALIGN),
    ((P, P, P_ODD, Y, 4096, 4096, 1, None), rz.RZ_EALIGN),
    ((P, P, P, Y + 2, 4096, 4096, 1, None), rz.RZ_EALIGN),
])
def test_q4k_q8_gemv_add_rejects(lib, args, code):
    assert _rc("rz_q4k_q8_gemv_add", *args) == code
    assert _rc.last.startswith("rz_q4k_q8_gemv_add")


def test_q4k_q8_gemv_add_accepts_in_place_and_adjacent(lib):
    # r == y and r right after y pass validation; with no device visible the
    # launch itself then fails
    res = run_isolated([("rz_q4k_q8_gemv_add", [P, P, Y, Y, 4096, 4096, 2, None]),
                        ("rz_q4k_q8_gemv_add", [P, P, Y + 4 * 4096 * 2, Y, 4096, 4096, 2, None])])
    assert [rc for rc, _ in res] == [rz.RZ_ELAUNCH, rz.RZ_ELAUNCH]


H = P + (2 << 30)
@pytest.mark.parametrize("args,code", [
    ((P, P, P, P, H, P, None, Y, None, 4096, 14336, None), rz.RZ_EINVAL),        # null r
    ((P, P, P, P, H, P, Y + 4, Y, None, 4096, 14336, None), rz.RZ_EINVAL),       # r overlaps y
    ((P, P, P, P, H, P, H + 64, Y, None, 4096, 14336, None), rz.RZ_EINVAL),      # r inside h
    ((P, P, P, P, H, Y + 65536, Y + 65536 - 400, Y, None, 4096, 14336, None),
     rz.RZ_EINVAL),                                                              # r meets h_q8
    ((P, P, P, P, H, P, H + 4 * 14336, Y, H, 4096, 14336, None), rz.RZ_EINVAL),  # r inside gu
    ((P, P, P, P, H, P, P_ODD, Y, None, 4096, 14336, None), rz.RZ_EALIGN),
    ((P, P, P, P, H, P, Y, Y, None, 4000, 14336, None), rz.RZ_EDIM),
])
def test_swiglu_ffn_add_rejects(lib, args, code):
    assert _rc("rz_swiglu_ffn_q4k_add", *args) == code
    assert _rc.last.startswith("rz_swiglu_ffn_q4k_add")


@pytest.mark.parametrize("args,code", [
    ((None, P, 4096, Y, 14336, 4096, None), rz.RZ_EINVAL),
    ((P, None, 4096, Y, 14336, 4096, None), rz.RZ_EINVAL),
    ((P, P, 4096, None, 14336, 4096, None), rz.RZ_EINVAL),
    ((P, Y + 4, 4096, Y, 14336, 4096, None), rz.RZ_EINVAL),     # x overlaps y
    ((P, P, 4097, Y, 14336, 4096, None), rz.RZ_EDIM),           # n > in_dim
    ((P, P, 0, Y, 14336, 4096, None), rz.RZ_EDIM),
    ((P, P, 896, Y, 14336, 896, None), rz.RZ_EDIM),             # unpadded in_dim
    ((P, P, 4096, Y, 0, 4096, None), rz.RZ_EDIM),
    ((P, P, 4096, Y, 1 << 20, 16384, None), rz.RZ_EDIM),        # matrix >= 2 GiB
    ((P + 8, P, 4096, Y, 14336, 4096, None), rz.RZ_EALIGN),
    ((P, P_ODD, 4096, Y, 14336, 4096, None), rz.RZ_EALIGN),
    ((P, P, 4096, Y + 2, 14336, 4096, None), rz.RZ_EALIGN),
])
def test_q4k_gemv_rejects(lib, args, code):
    assert _rc("rz_q4k_gemv", *args) == code
    assert _rc.last.startswith("rz_q4k_gemv")


@pytest.mark.parametrize("args,code", [
    ((None, P, P, P, H, Y, None, 4096, 14336, None), rz.RZ_EINVAL),
    ((P, P, P, None, H, Y, None, 4096, 14336, None), rz.RZ_EINVAL),
    ((P, P, P, P, None, Y, None, 4096, 14336, None), rz.RZ_EINVAL),
    ((P, P, P, H + 64, H, Y, None, 4096, 14336, None), rz.RZ_EINVAL),    # x overlaps h
    ((P, P, P, P, H, H + 64, None, 4096, 14336, None), rz.RZ_EINVAL),    # y overlaps h
    ((P, P, P, P, H, Y, H + 64, 4096, 14336, None), rz.RZ_EINVAL),       # gu overlaps h
    ((P, P, P, P, H, Y, None, 4000, 14336, None), rz.RZ_EDIM),
    ((P, P, P, P, H, Y, None, 4096, 14000, None), rz.RZ_EDIM),
    ((P + 8, P, P, P, H, Y, None, 4096, 14336, None), rz.RZ_EALIGN),
    ((P, P, P, P_ODD, H, Y, None, 4096, 14336, None), rz.RZ_EALIGN),
    ((P, P, P, P, H, Y, P_ODD, 4096, 14336, None), rz.RZ_EALIGN),
])
def test_swiglu_ffn_f32_rejects(lib, args, code):
    assert _rc("rz_swiglu_ffn_q4k_f32", *args) == code
    assert _rc.last.startswith("rz_swiglu_ffn_q4k_f32")


def test_swiglu_ffn_f32_accepts_y_on_x(lib):
    (rc, _), = run_isolated([("rz_swiglu_ffn_q4k_f32", [P, P, P, Y, H, Y, None, 4096, 14336,
                                                        None])])
    assert rc == rz.RZ_ELAUNCH


def test_lm_head_workspace_bytes(lib):
    # 151936 x 1024: 16 pairs a row -> 16 lanes a row, 4 rows side by side, 4 unrolled,
    # 9496 row groups of 16 rows, one a wave, four waves a workgroup: 2374 workgroups
    assert rz.rz_lm_head_q4_0_workspace_bytes(151936, 1024, 0) == 2374 * 8
    assert rz.rz_lm_head_q4_0_workspace_bytes(151936, 1024, 1) == 2374 * 8
    assert rz.rz_lm_head_q4_0_workspace_bytes(1, 64, 0) == 8
    for bad in ((0, 1024, 0), (151936, 1000, 0), (151936, 1024, 2), (151936, 0, 1)):
        assert rz.rz_lm_head_q4_0_workspace_bytes(*bad) == 0


WS = P + (3 << 30)
IDX = P + (4 << 30)
@pytest.mark.parametrize("args,code", [
    ((None, P, 0, None, Y, 151936, 1024, None, None, None, 0, None), rz.RZ_EINVAL),
    ((P, None, 0, None, Y, 151936, 1024, None, None, None, 0, None), rz.RZ_EINVAL),
    ((P, P, 0, None, None, 151936, 1024, None, None, None, 0, None), rz.RZ_EINVAL),
    ((P, P, 2, None, Y, 151936, 1024, None, None, None, 0, None), rz.RZ_EINVAL),
    ((P, P, 0, None, Y, 151936, 1000, None, None, None, 0, None), rz.RZ_EDIM),
    ((P, P, 0, None, Y, 0, 1024, None, None, None, 0, None), rz.RZ_EDIM),
    ((P, P, 0, None, Y, 151936, 1024, IDX, None, None, 0, None), rz.RZ_EINVAL),     # no workspace
    ((P, P, 0, None, Y, 151936, 1024, IDX, None, WS, 18991, None), rz.RZ_EINVAL),    # short
    ((P, P, 1, None, Y, 151936, 1024, None, IDX, WS, 18991, None), rz.RZ_EINVAL),    # short (Q8_1)
    ((P, P, 0, Y + 4, Y, 151936, 1024, None, None, None, 0, None), rz.RZ_EINVAL),   # bias overlaps
    ((P, P, 0, None, Y, 151936, 1024, IDX, None, Y + 64, 18992, None), rz.RZ_EINVAL),  # ws on logits
    ((P, P, 0, None, Y, 151936, 1024, WS + 8, None, WS, 18992, None), rz.RZ_EINVAL),   # idx in ws
    ((P, P, 0, None, Y, 151936, 1024, IDX, None, WS + 2, 18992, None), rz.RZ_EALIGN),
    ((P, P + 8, 0, None, Y, 151936, 1024, None, None, None, 0, None), rz.RZ_EALIGN),
    ((P, P, 0, P_ODD, Y, 151936, 1024, None, None, None, 0, None), rz.RZ_EALIGN),
    ((P, P, 0, None, Y, 151936, 1024, IDX + 2, None, WS, 18992, None), rz.RZ_EALIGN),
])
def test_lm_head_rejects(lib, args, code):
    assert _rc("rz_lm_head_q4_0", *args) == code
    assert _rc.last.startswith("rz_lm_head_q4_0")


def test_lm_head_accepts_bias_in_place_and_exact_workspace(lib):
    res = run_isolated([("rz_lm_head_q4_0", [P, P, 0, Y, Y, 151936, 1024, None, None, None, 0,
                                             None]),
                        ("rz_lm_head_q4_0", [P, P, 0, None, Y, 151936, 1024, IDX, IDX + 4, WS,
                                             2374 * 8, None])])
    assert [rc for rc, _ in res] == [rz.RZ_ELAUNCH, rz.RZ_ELAUNCH]


W_FAR = P + (8 << 30)   # a weight matrix of over a gigabyte, clear of Y, IDX and WS


@pytest.mark.parametrize("args,code", [
    ((None, P, 0, None, Y, 151936, 1024, None, None, None), rz.RZ_EINVAL),
    ((P, P, 2, None, Y, 151936, 1024, None, None, None), rz.RZ_EINVAL),
    ((P, P, 0, None, Y, 151936, 1000, None, None, None), rz.RZ_EDIM),
    ((P, P + 8, 0, None, Y, 151936, 1024, None, None, None), rz.RZ_EALIGN),
    ((P, P, 0, Y + 4, Y, 151936, 1024, None, None, None), rz.RZ_EINVAL),        # bias overlaps
    ((P, P, 0, None, Y, 151936, 1024, Y + 8, None, None), rz.RZ_EINVAL),        # idx in logits
    # 600000 x 4096 with an argmax needs 37500 pairs: beyond the fixed array
    ((W_FAR, P, 0, None, Y, 600000, 4096, IDX, None, None), rz.RZ_EINVAL),
    ((W_FAR, P, 1, None, Y, 600000, 4096, None, IDX, None), rz.RZ_EINVAL),
])
def test_lm_head_noalloc_rejects(lib, args, code):
    """The checks of rz_lm_head_q4_0, and a shape whose argmax needs more pairs
    than the fixed array holds."""
    assert _rc("rz_lm_head_q4_0_noalloc", *args) == code
    assert _rc.last.startswith("rz_lm_head_q4_0_noalloc")


def test_lm_head_noalloc_size_limit_message_and_accepts(lib):
    """Beyond the fixed array the call says how many pairs it needs and what the
    array holds; the largest shape within it, and any shape without an argmax,
    pass validation (and then fail at launch for want of a device)."""
    res = run_isolated([("rz_lm_head_q4_0_noalloc", [W_FAR, P, 0, None, Y, 600000, 4096, IDX,
                                                     None, None]),
                        # 524288 x 4096: 32768 pairs, exactly the array
                        ("rz_lm_head_q4_0_noalloc", [W_FAR, P, 0, None, Y, 524288, 4096, IDX,
                                                     None, None]),
                        ("rz_lm_head_q4_0_noalloc", [W_FAR, P, 0, None, Y, 600000, 4096, None,
                                                     None, None])])
    assert res[0][0] == rz.RZ_EINVAL and "37500" in res[0][1] and "32768" in res[0][1]
    assert res[1][0] == rz.RZ_ELAUNCH and res[2][0] == rz.RZ_ELAUNCH
    assert rz.rz_lm_head_q4_0_workspace_bytes(524288, 4096, 0) == 32768 * 8
    assert rz.NOALLOC_ARGMAX_PAIRS == 32768


@pytest.mark.parametrize("args,code", [
    ((None, P, P, None, None, H, Y, 2560, 10240, None), rz.RZ_EINVAL),
    ((P, P, None, None, None, H, Y, 2560, 10240, None), rz.RZ_EINVAL),
    ((P, P, P, None, None, None, Y, 2560, 10240, None), rz.RZ_EINVAL),
    ((P, P, P, None, None, H, None, 2560, 10240, None), rz.RZ_EINVAL),
    ((P, P, H + 64, None, None, H, Y, 2560, 10240, None), rz.RZ_EINVAL),       # x overlaps h
    ((P, P, P, None, None, H, H + 64, 2560, 10240, None), rz.RZ_EINVAL),       # y overlaps h
    ((P, P, P, H + 4, None, H, Y, 2560, 10240, None), rz.RZ_EINVAL),          # up_bias shifted on h
    ((P, P, P, None, Y + 4, H, Y, 2560, 10240, None), rz.RZ_EINVAL),          # down_bias shifted on y
    ((P, P, P, None, None, H, Y, 2500, 10240, None), rz.RZ_EDIM),
    ((P, P, P, None, None, H, Y, 2560, 10000, None), rz.RZ_EDIM),
    ((P + 2, P, P, None, None, H, Y, 2560, 10240, None), rz.RZ_EALIGN),
    ((P, P, P + 8, None, None, H, Y, 2560, 10240, None), rz.RZ_EALIGN),         # x needs 16
    ((P, P, P, None, None, H + 8, Y, 2560, 10240, None), rz.RZ_EALIGN),         # h needs 16
    ((P, P, P, P_ODD, None, H, Y, 2560, 10240, None), rz.RZ_EALIGN),
])
def test_gelu_ffn_rejects(lib, args, code):
    assert _rc("rz_gelu_ffn_q4_0", *args) == code
    assert _rc.last.startswith("rz_gelu_ffn_q4_0")


def test_error_message_is_per_call(lib):
    (rc1, m1), (rc2, m2) = run_isolated([("rz_q4k_q8_gemv", [P, P, P, 10, 100, 1, None]),
                                         ("rz_q4_0_gemv", [P, P, 7, P, 10, 64, None])])
    assert rc1 == rz.RZ_EDIM and "in_dim=100" in m1
    assert rc2 == rz.RZ_EINVAL and "x_format=7" in m2


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        rz.rz_q8_1_quantize(torch.zeros(32), 32, 32, 1, torch.zeros(40, dtype=torch.uint8), stream=0)


_READ_CHILD = r"""
import ctypes, json, sys
lib = ctypes.CDLL(sys.argv[1])
f = lib.rz_stream_read
f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
f.restype = ctypes.c_int
print(json.dumps([f(*a) for a in json.loads(sys.stdin.read())]))
"""


def test_stream_read_helper_rejects_bad_arguments():
    """The benchmark's streaming-read helper (librz_stream_read.so, not part of
    librz.so) exports rz_stream_read and refuses null, unaligned or ragged
    buffers and grids out of range before any launch."""
    path = os.path.join(ROOT, "q4_q8_integer_quantize_amd", "librz_stream_read.so")
    if not os.path.exists(path):
        pytest.skip("librz_stream_read.so not built")
    calls = [[None, 1024, P, 256, None], [P, 1024, None, 256, None], [P + 8, 1024, P, 256, None],
             [P, 1000, P, 256, None], [P, 0, P, 256, None], [P, 1024, P, 0, None],
             [P, 1024, P, 65537, None]]
    env = dict(os.environ, ROCR_VISIBLE_DEVICES="-1", HIP_VISIBLE_DEVICES="-1")
    res = subprocess.run([sys.executable, "-c", _READ_CHILD, path], input=json.dumps(calls),
                         capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stderr
    assert json.loads(res.stdout) == [-1] * len(calls)


# Buffers 4 GiB apart never overlap; an output placed on an input does.
def _b(k):
    return P + (k << 32)


_OVERLAP_CASES = [
    # (entry, args with separate buffers, index of an output, index of an input it is moved onto)
    ("rz_q8_1_quantize", [_b(0), 896, 1024, 2, _b(1), None], 4, 0),
    ("rz_rmsnorm_q8_1", [_b(0), _b(1), 1e-5, 4096, 4096, 1, _b(2), _b(3), None], 6, 0),
    ("rz_rmsnorm_q8_1", [_b(0), _b(1), 1e-5, 4096, 4096, 1, _b(2), _b(3), None], 7, 1),
    ("rz_q4k_q8_gemv", [_b(0), _b(1), _b(2), 4096, 4096, 1, None], 2, 1),
    ("rz_q4k_q8_gemv", [_b(0), _b(1), _b(2), 4096, 4096, 1, None], 2, 0),
    ("rz_q4k_q8_gemv_add", [_b(0), _b(1), _b(3), _b(2), 4096, 4096, 1, None], 3, 1),
    ("rz_q4k_q8_gemv_f32", [_b(0), _b(1), 4096, _b(2), _b(3), 4096, 4096, None], 3, 1),
    ("rz_q4k_q8_gemv_f32", [_b(0), _b(1), 4096, _b(2), _b(3), 4096, 4096, None], 4, 3),
    ("rz_q4k_q8_gemv_f32", [_b(0), _b(1), 4096, _b(2), _b(3), 4096, 4096, None], 4, 0),
    ("rz_q4k_gemv", [_b(0), _b(1), 4096, _b(2), 4096, 4096, None], 3, 0),
    ("rz_q4k_q8_gemv_f32_add", [_b(0), _b(1), 4096, _b(2), _b(3), _b(4), 4096, 4096, None], 5, 1),
    ("rz_q4k_q8_gemv_f32_add", [_b(0), _b(1), 4096, _b(2), _b(3), _b(4), 4096, 4096, None], 5, 0),
    ("rz_q4k_q8_gemv_f32_add", [_b(0), _b(1), 4096, _b(2), _b(3), _b(4), 4096, 4096, None], 3, 4),
    ("rz_q4k_q8_gemv_f32_add", [_b(0), _b(1), 4096, _b(2), _b(3), _b(4), 4096, 4096, None], 5, 3),
    ("rz_q4_0_gemv", [_b(0), _b(1), 0, _b(2), 4096, 1024, None], 3, 1),
    ("rz_q4_0_gemv", [_b(0), _b(1), 1, _b(2), 4096, 1024, None], 3, 0),
    ("rz_swiglu_ffn_q4k", [_b(0), _b(1), _b(2), _b(3), _b(4), _b(5), _b(6), None, 4096, 14336, None], 4, 3),
    ("rz_swiglu_ffn_q4k", [_b(0), _b(1), _b(2), _b(3), _b(4), _b(5), _b(6), None, 4096, 14336, None], 6, 5),
    ("rz_swiglu_ffn_q4k", [_b(0), _b(1), _b(2), _b(3), _b(4), _b(5), _b(6), None, 4096, 14336, None], 5, 1),
    ("rz_swiglu_ffn_q4k", [_b(0), _b(1), _b(2), _b(3), _b(4), _b(5), _b(6), _b(7), 4096, 14336, None], 6, 4),
    ("rz_swiglu_ffn_q4k", [_b(0), _b(1), _b(2), _b(3), _b(4), _b(5), _b(6), _b(7), 4096, 14336, None], 6, 7),
    ("rz_swiglu_ffn_q4k_f32", [_b(0), _b(1), _b(2), _b(3), _b(4), _b(5), None, 4096, 14336, None], 5, 2),
    ("rz_swiglu_ffn_q4k_f32", [_b(0), _b(1), _b(2), _b(3), _b(4), _b(5), _b(6), 4096, 14336, None], 5, 6),
    ("rz_gelu_ffn_q4_0", [_b(0), _b(1), _b(2), None, None, _b(3), _b(4), 2560, 10240, None], 5, 0),
    ("rz_gelu_ffn_q4_0", [_b(0), _b(1), _b(2), None, None, _b(3), _b(4), 2560, 10240, None], 6, 1),
]


@pytest.mark.parametrize("fn,args,out_i,in_i", _OVERLAP_CASES)
def test_outputs_must_not_overlap_inputs(lib, fn, args, out_i, in_i):
    """With every buffer apart the call passes validation (and, with no device
    visible, fails at the launch); with the output moved onto one of the
    call's inputs it is rejected before any HIP call."""
    bad = list(args)
    bad[out_i] = args[in_i]
    (rc_ok, _), (rc_bad, msg) = run_isolated([(fn, args), (fn, bad)])
    assert rc_ok == rz.RZ_ELAUNCH
    assert rc_bad == rz.RZ_EINVAL and "overlap" in msg, msg


def test_lm_head_outputs_must_not_overlap_inputs(lib):
    need = 2374 * 8     # fp32 x, 151936 x 1024
    base = [_b(0), _b(1), 0, None, _b(2), 151936, 1024, _b(3), _b(4), _b(5), need, None]
    cases = [list(base)]
    for out_i, in_i in [(4, 0), (4, 1), (7, 1), (9, 0), (8, 7)]:
        c = list(base)
        c[out_i] = base[in_i]
        cases.append(c)
    res = run_isolated([("rz_lm_head_q4_0", c) for c in cases])
    assert res[0][0] == rz.RZ_ELAUNCH
    for rc, msg in res[1:]:
        assert rc == rz.RZ_EINVAL and "overlap" in msg, msg



def test_topk_workspace_bytes():
    # One candidate (32-bit key + int32 index) per slice of 2048 values and
    # selected entry: 151936 values are 75 slices.
    assert rz.rz_topk_f32_workspace_bytes(151936, 40) == 75 * 40 * 8
    assert rz.rz_topk_f32_workspace_bytes(1, 1) == 8
    assert rz.rz_topk_f32_workspace_bytes(100, 100) == 100 * 8
    assert rz.rz_topk_f32_workspace_bytes(262144, 128) == 16384 * 8
    assert rz.rz_topk_f32_workspace_bytes(524288, 64) == 16384 * 8
    assert rz.rz_topk_f32_workspace_bytes(1 << 24, 2) == 16384 * 8
    for bad in ((0, 1), (7, 8), (10, 0), (1000, 129), (262145, 128), (524289, 64),
                ((1 << 24) + 1, 1), ((1 << 24), 3)):
        assert rz.rz_topk_f32_workspace_bytes(*bad) == 0, bad


TK = 75 * 40 * 8    # workspace for 151936 values, k = 40
@pytest.mark.parametrize("args,code", [
    ((None, 151936, 40, IDX, None, WS, TK, None), rz.RZ_EINVAL),           # null values
    ((Y, 151936, 40, IDX, None, None, TK, None), rz.RZ_EINVAL),            # null workspace
    ((Y, 151936, 40, None, None, WS, TK, None), rz.RZ_EINVAL),             # no output
    ((Y, 151936, 0, IDX, None, WS, TK, None), rz.RZ_EINVAL),               # k 0
    ((Y, 151936, 129, IDX, None, WS, 1 << 20, None), rz.RZ_EINVAL),        # k above 128
    ((Y, 7, 8, IDX, None, WS, 64, None), rz.RZ_EINVAL),                    # k above n
    ((Y, 300000, 128, IDX, None, WS, 1 << 20, None), rz.RZ_EINVAL),        # 18816 candidates
    ((Y, 0, 1, IDX, None, WS, 8, None), rz.RZ_EDIM),
    ((Y, (1 << 24) + 1, 1, IDX, None, WS, 1 << 20, None), rz.RZ_EDIM),
    ((Y, 151936, 40, IDX, None, WS, TK - 1, None), rz.RZ_EINVAL),          # short workspace
    ((Y + 2, 151936, 40, IDX, None, WS, TK, None), rz.RZ_EALIGN),
    ((Y, 151936, 40, IDX + 2, None, WS, TK, None), rz.RZ_EALIGN),
    ((Y, 151936, 40, None, IDX + 2, WS, TK, None), rz.RZ_EALIGN),
    ((Y, 151936, 40, IDX, None, WS + 2, TK, None), rz.RZ_EALIGN),
    ((Y, 151936, 40, IDX, None, Y + 64, TK, None), rz.RZ_EINVAL),          # workspace on values
    ((Y, 151936, 40, Y + 4, None, WS, TK, None), rz.RZ_EINVAL),            # idx on values
    ((Y, 151936, 40, WS + 8, None, WS, TK, None), rz.RZ_EINVAL),           # idx in workspace
    ((Y, 151936, 40, IDX, IDX + 64, WS, TK, None), rz.RZ_EINVAL),          # val on idx
    ((Y, 151936, 40, None, Y + 4, WS, TK, None), rz.RZ_EINVAL),            # val on values
])
def test_topk_rejects(lib, args, code):
    assert _rc("rz_topk_f32", *args) == code
    assert _rc.last.startswith("rz_topk_f32"), _rc.last


def test_topk_accepts_limits_and_exact_workspace(lib):
    res = run_isolated([("rz_topk_f32", [Y, 151936, 40, IDX, IDX + 160, WS, TK, None]),
                        ("rz_topk_f32", [Y, 1, 1, IDX, None, WS, 8, None]),
                        ("rz_topk_f32", [Y, 128, 128, None, IDX, WS, 1024, None]),
                        ("rz_topk_f32", [Y, 262144, 128, IDX, None, WS, 131072, None]),
                        ("rz_topk_f32", [Y, 524288, 64, IDX, None, WS, 131072, None]),
                        ("rz_topk_f32", [Y, 1 << 24, 2, IDX, None, WS, 131072, None])])
    assert [rc for rc, _ in res] == [rz.RZ_ELAUNCH] * 6, res


LM_TK = [P, H, 0, None, Y, 151936, 1024, 40, IDX, IDX + 160, WS, TK, None]
@pytest.mark.parametrize("change,code", [
    ({0: None}, rz.RZ_EINVAL),                        # null weights
    ({6: 1000}, rz.RZ_EDIM),                          # in_dim not a multiple of 32
    ({2: 2}, rz.RZ_EINVAL),                           # x_format
    ({7: 0}, rz.RZ_EINVAL),                           # k 0
    ({7: 129}, rz.RZ_EINVAL),                         # k above 128
    ({8: None, 9: None}, rz.RZ_EINVAL),               # no top-k output
    ({10: None}, rz.RZ_EINVAL),                       # no workspace
    ({11: TK - 1}, rz.RZ_EINVAL),                     # short workspace
    ({5: 600000, 7: 128}, rz.RZ_EINVAL),              # too many candidates
    ({10: P + 64}, rz.RZ_EINVAL),                     # workspace on the weights
    ({10: Y + 64}, rz.RZ_EINVAL),                     # workspace on the logits
    ({8: H + 8}, rz.RZ_EINVAL),                       # idx on x
    ({3: W_FAR, 9: W_FAR + 64}, rz.RZ_EINVAL),        # val on the bias
    ({8: Y + 8}, rz.RZ_EINVAL),                       # idx on the logits
    ({8: IDX + 2}, rz.RZ_EALIGN),
    ({10: WS + 2}, rz.RZ_EALIGN),
])
def test_lm_head_topk_rejects(lib, change, code):
    args = list(LM_TK)
    for i, v in change.items():
        args[i] = v
    assert _rc("rz_lm_head_q4_0_topk", *args) == code
    assert _rc.last.startswith("rz_lm_head_q4_0_topk"), _rc.last


def test_lm_head_topk_accepts(lib):
    q8 = list(LM_TK)
    q8[2] = 1
    bias = list(LM_TK)
    bias[3] = W_FAR
    res = run_isolated([("rz_lm_head_q4_0_topk", LM_TK), ("rz_lm_head_q4_0_topk", q8),
                        ("rz_lm_head_q4_0_topk", bias)])
    assert [rc for rc, _ in res] == [rz.RZ_ELAUNCH] * 3, res


@pytest.mark.parametrize("args,code", [
    ((0,) + _m([P], [Y], [4096])[:3] + (P + 16, H, 1e-5, 4096, None, 4096, None), rz.RZ_EINVAL),   # n_mats 0
    ((1,) + _m([P], [Y], [4096])[:3] + (None, H, 1e-5, 4096, None, 4096, None), rz.RZ_EINVAL),     # null x
    ((1,) + _m([P], [Y], [4096])[:3] + (H, None, 1e-5, 4096, None, 4096, None), rz.RZ_EINVAL),     # null gamma
    ((1,) + _m([P], [Y], [4096])[:3] + (H, H + 65536, 0.0, 4096, None, 4096, None), rz.RZ_EINVAL),  # eps 0
    ((1,) + _m([P], [Y], [4096])[:3] + (H, H + 65536, 1e-5, 4096, None, 20480, None), rz.RZ_EDIM),  # above 16384
    ((1,) + _m([P], [Y], [4096])[:3] + (H, H + 65536, 1e-5, 4097, None, 4096, None), rz.RZ_EDIM),   # n > in_dim
    ((1,) + _m([P], [Y], [4096])[:3] + (H, H + 65536, 1e-5, 4096, None, 4000, None), rz.RZ_EDIM),
    ((1,) + _m([P], [Y], [4096])[:3] + (H + 2, H + 65536, 1e-5, 4096, None, 4096, None), rz.RZ_EALIGN),
    ((1,) + _m([P], [Y], [4096])[:3] + (H, H + 65536, 1e-5, 4096, WS + 8, 4096, None), rz.RZ_EALIGN),
    ((1,) + _m([P + 8], [Y], [4096])[:3] + (H, H + 65536, 1e-5, 4096, None, 4096, None), rz.RZ_EALIGN),
    ((1,) + _m([P], [H], [4096])[:3] + (H, H + 65536, 1e-5, 4096, None, 4096, None), rz.RZ_EINVAL),  # y on x
    ((1,) + _m([P], [Y], [4096])[:3] + (H, H + 65536, 1e-5, 4096, Y, 4096, None), rz.RZ_EINVAL),    # x_q8 on y
])
def test_rmsnorm_q4k_q8_gemv_multi_rejects(lib, args, code):
    assert _rc("rz_rmsnorm_q4k_q8_gemv_multi", *args) == code
    assert _rc.last.startswith("rz_rmsnorm_q4k_q8_gemv_multi")


def test_rmsnorm_q4k_q8_gemv_multi_accepts(lib):
    (rc, msg), = run_isolated([("rz_rmsnorm_q4k_q8_gemv_multi",
                                [2] + list(_m([P, P + (1 << 24)], [Y, Y + 65536], [4096, 1024])) +
                                [H, H + 65536, 1e-5, 4000, WS, 4096, None])])
    assert rc == rz.RZ_ELAUNCH, msg


# rz_rmsnorm_swiglu_ffn_q4k_add(w_gate, w_up, w_down, x, gamma, eps, h, h_q8, y, gu, hidden, inter, stream)
_NSW = [_b(0), _b(1), _b(2), _b(3), _b(4), 1e-5, _b(5), _b(6), _b(7), _b(8), 4096, 14336, None]


def _nsw(**kw):
    names = ["wg", "wu", "wd", "x", "gamma", "eps", "h", "hq", "y", "gu", "hidden", "inter", "s"]
    a = list(_NSW)
    for k, v in kw.items():
        a[names.index(k)] = v
    return a


@pytest.mark.parametrize("args,code", [
    (_nsw(wg=None), rz.RZ_EINVAL),
    (_nsw(x=None), rz.RZ_EINVAL),
    (_nsw(gamma=None), rz.RZ_EINVAL),
    (_nsw(h=None), rz.RZ_EINVAL),
    (_nsw(hq=None), rz.RZ_EINVAL),
    (_nsw(y=None), rz.RZ_EINVAL),
    (_nsw(eps=0.0), rz.RZ_EINVAL),
    (_nsw(eps=float("nan")), rz.RZ_EINVAL),
    (_nsw(eps=float("inf")), rz.RZ_EINVAL),
    (_nsw(hidden=4000), rz.RZ_EDIM),
    (_nsw(inter=14000), rz.RZ_EDIM),
    (_nsw(hidden=0), rz.RZ_EDIM),
    (_nsw(hidden=32768), rz.RZ_EDIM),                  # above the fused gate/up limit
    (_nsw(wd=_b(2) + 8), rz.RZ_EALIGN),
    (_nsw(hq=_b(6) + 4), rz.RZ_EALIGN),                # Q8_1 staging is 16-byte
    (_nsw(x=_b(3) + 2), rz.RZ_EALIGN),
    (_nsw(gamma=_b(4) + 1), rz.RZ_EALIGN),
    (_nsw(gu=_b(8) + 2), rz.RZ_EALIGN),
    (_nsw(y=_b(3) + 4), rz.RZ_EINVAL),                 # y overlaps x without being x
    (_nsw(y=_b(4)), rz.RZ_EINVAL),                     # y on gamma
    (_nsw(y=_b(6) + 64), rz.RZ_EINVAL),                # y inside h_q8
    (_nsw(h=_b(3)), rz.RZ_EINVAL),                     # h on x
    (_nsw(h=_b(1) + 4096), rz.RZ_EINVAL),              # h inside w_up
    (_nsw(hq=_b(4) + 16), rz.RZ_EINVAL),               # h_q8 on gamma
    (_nsw(gu=_b(5) + 4 * 14336 - 4), rz.RZ_EINVAL),    # gu meets h
    (_nsw(y=_b(5) + 64), rz.RZ_EINVAL),                # y inside h
    (_nsw(y=_b(8) + 4 * 14336), rz.RZ_EINVAL),         # y inside gu's up half
])
def test_rmsnorm_swiglu_ffn_add_rejects(lib, args, code):
    assert _rc("rz_rmsnorm_swiglu_ffn_q4k_add", *args) == code
    assert _rc.last.startswith("rz_rmsnorm_swiglu_ffn_q4k_add")


def test_rmsnorm_swiglu_ffn_add_accepts(lib):
    # separate buffers, y written over x in place, and no gu: all pass
    # validation, and with no device visible the launch fails
    res = run_isolated([("rz_rmsnorm_swiglu_ffn_q4k_add", _nsw()),
                        ("rz_rmsnorm_swiglu_ffn_q4k_add", _nsw(y=_b(3))),
                        ("rz_rmsnorm_swiglu_ffn_q4k_add", _nsw(gu=None)),
                        ("rz_rmsnorm_swiglu_ffn_q4k_add", _nsw(hidden=16384, inter=256))])
    assert [rc for rc, _ in res] == [rz.RZ_ELAUNCH] * 4, res


# rz_q4k_q8_gemv_f32_add(w, x, n, x_q8, r, y, out_dim, in_dim, stream)
_FA = [_b(0), _b(1), 4096, None, _b(3), _b(4), 14336, 4096, None]


def _fa(**kw):
    names = ["w", "x", "n", "xq", "r", "y", "out", "ind", "s"]
    a = list(_FA)
    for k, v in kw.items():
        a[names.index(k)] = v
    return a


@pytest.mark.parametrize("args,code", [
    (_fa(w=None), rz.RZ_EINVAL),
    (_fa(x=None), rz.RZ_EINVAL),
    (_fa(r=None), rz.RZ_EINVAL),
    (_fa(y=None), rz.RZ_EINVAL),
    (_fa(n=0), rz.RZ_EDIM),
    (_fa(n=4097), rz.RZ_EDIM),
    (_fa(ind=4000), rz.RZ_EDIM),
    (_fa(ind=20480, n=20480), rz.RZ_EDIM),            # above the fused limit
    (_fa(out=0), rz.RZ_EDIM),
    (_fa(w=_b(0) + 8), rz.RZ_EALIGN),
    (_fa(x=_b(1) + 2), rz.RZ_EALIGN),
    (_fa(r=_b(3) + 2), rz.RZ_EALIGN),
    (_fa(y=_b(4) + 2), rz.RZ_EALIGN),
    (_fa(xq=_b(2) + 8), rz.RZ_EALIGN),
    (_fa(y=_b(4), r=_b(4) + 4), rz.RZ_EINVAL),        # r overlaps y without being y
    (_fa(y=_b(1) + 64), rz.RZ_EINVAL),                # y inside x
    (_fa(xq=_b(3) + 16), rz.RZ_EINVAL),               # x_q8 on r
])
def test_q4k_q8_gemv_f32_add_rejects(lib, args, code):
    assert _rc("rz_q4k_q8_gemv_f32_add", *args) == code
    assert _rc.last.startswith("rz_q4k_q8_gemv_f32_add")


def test_q4k_q8_gemv_f32_add_accepts_in_place(lib):
    res = run_isolated([("rz_q4k_q8_gemv_f32_add", _fa()),
                        ("rz_q4k_q8_gemv_f32_add", _fa(r=_b(4))),                   # r is y
                        ("rz_q4k_q8_gemv_f32_add", _fa(xq=_b(2), n=4000))])
    assert [rc for rc, _ in res] == [rz.RZ_ELAUNCH] * 3, res


def test_c_consumer_host_paths(tmp_path):
    """The plain C consumer of include/rz.h compiles with -Werror against the
    header, links librz.so and the HIP runtime without Python, and its
    host-side checks (version, the error codes and message of rejected
    arguments, no HIP call) pass here."""
    from q4_q8_integer_quantize_amd import build as rzbuild
    exe = rzbuild.build_consumer(str(tmp_path / "abi_consumer"))
    res = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0 and "passed: 0 failure(s)" in res.stdout, res.stdout + res.stderr
