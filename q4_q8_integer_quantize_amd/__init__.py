"""Python binding of librz.so -- Q4_K / Q4_0 x Q8_1 integer GEMV for MI355X.

The functions carry the names of the C entry points (include/rz.h) and do
argument marshalling only: tensors become device pointers, the stream defaults
to PyTorch's current stream, and a negative return code becomes a
``RuntimeError`` carrying ``rz_last_error()``.  Every step of the computation
runs in the HIP kernels of librz.so; there is no fallback.  If the library has
not been built (``python -m q4_q8_integer_quantize_amd.build``) every call
raises.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "RZ_OK", "RZ_EINVAL", "RZ_EDIM", "RZ_EALIGN", "RZ_ELAUNCH",
    "Q8_1_BLOCK_BYTES", "Q4K_BLOCK_BYTES", "Q4_0_BLOCK_BYTES", "MAX_TOKENS",
    "library_path", "load_library", "rz_last_error", "rz_abi_version",
    "rz_q8_1_quantize", "rz_rmsnorm_q8_1", "rz_q4k_q8_gemv", "rz_q4k_q8_gemv_add",
    "rz_q4k_q8_gemv_multi", "rz_rmsnorm_q4k_q8_gemv_multi", "rz_rmsnorm_swiglu_ffn_q4k_add",
    "rz_q4k_q8_gemv_f32", "rz_q4k_q8_gemv_f32_add",
    "rz_q4_0_gemv", "rz_swiglu_ffn_q4k", "rz_swiglu_ffn_q4k_add", "rz_q4k_gemv",
    "rz_swiglu_ffn_q4k_f32",
    "rz_lm_head_q4_0", "rz_lm_head_q4_0_workspace_bytes", "rz_lm_head_q4_0_noalloc",
    "rz_gelu_ffn_q4_0", "rz_topk_f32", "rz_topk_f32_workspace_bytes", "rz_lm_head_q4_0_topk",
    "TOPK_MAX", "q8_1_nbytes", "RzError", "NOALLOC_ARGMAX_PAIRS",
]

RZ_OK, RZ_EINVAL, RZ_EDIM, RZ_EALIGN, RZ_ELAUNCH = 0, -1, -2, -3, -4
Q8_1_BLOCK_BYTES = 40
Q4K_BLOCK_BYTES = 144
Q4_0_BLOCK_BYTES = 18
MAX_TOKENS = 8
NOALLOC_ARGMAX_PAIRS = 32768
TOPK_MAX = 128

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class RzError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (rz code %d)" % (msg, code))
        self.code = code


def library_path() -> str:
    return os.path.join(_HERE, "librz.so")


def load_library(preload_torch: bool = True) -> ctypes.CDLL:
    """Load librz.so (built in-tree).  Raises if it is missing.  preload_torch
    False skips importing torch first; only for processes that never run a
    kernel (host-side argument checks), where a second HIP runtime is
    harmless."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError("librz.so is not built (%s); run "
                           "`python -m q4_q8_integer_quantize_amd.build`" % path)
    # One HIP runtime per process: torch ships its own libamdhip64 and asks
    # for it by its unversioned name, so if librz.so (which asks for
    # libamdhip64.so.7) came first, torch would load a second copy and the two
    # would not share devices or memory.  With torch loaded first, librz.so
    # binds to torch's copy.
    if preload_torch:
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.rz_q8_1_quantize.argtypes = [vp, i, i, i, vp, vp]
    lib.rz_rmsnorm_q8_1.argtypes = [vp, vp, ctypes.c_float, i, i, i, vp, vp, vp]
    lib.rz_q4k_q8_gemv.argtypes = [vp, vp, vp, i, i, i, vp]
    lib.rz_q4k_q8_gemv_add.argtypes = [vp, vp, vp, vp, i, i, i, vp]
    lib.rz_q4k_q8_gemv_f32.argtypes = [vp, vp, i, vp, vp, i, i, vp]
    lib.rz_q4k_q8_gemv_multi.argtypes = [i, vp, vp, vp, vp, i, i, vp]
    lib.rz_rmsnorm_q4k_q8_gemv_multi.argtypes = [i, vp, vp, vp, vp, vp, ctypes.c_float, i, vp, i, vp]
    lib.rz_rmsnorm_swiglu_ffn_q4k_add.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, i, i, vp]
    lib.rz_q4k_q8_gemv_f32_add.argtypes = [vp, vp, i, vp, vp, vp, i, i, vp]
    lib.rz_q4_0_gemv.argtypes = [vp, vp, i, vp, i, i, vp]
    lib.rz_swiglu_ffn_q4k.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, vp]
    lib.rz_swiglu_ffn_q4k_add.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, vp]
    lib.rz_q4k_gemv.argtypes = [vp, vp, i, vp, i, i, vp]
    lib.rz_swiglu_ffn_q4k_f32.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, vp]
    lib.rz_lm_head_q4_0.argtypes = [vp, vp, i, vp, vp, i, i, vp, vp, vp, ctypes.c_size_t, vp]
    lib.rz_lm_head_q4_0_noalloc.argtypes = [vp, vp, i, vp, vp, i, i, vp, vp, vp]
    lib.rz_gelu_ffn_q4_0.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, vp]
    lib.rz_lm_head_q4_0_workspace_bytes.argtypes = [i, i, i]
    lib.rz_lm_head_q4_0_workspace_bytes.restype = ctypes.c_size_t
    lib.rz_topk_f32.argtypes = [vp, i, i, vp, vp, vp, ctypes.c_size_t, vp]
    lib.rz_topk_f32_workspace_bytes.argtypes = [i, i]
    lib.rz_topk_f32_workspace_bytes.restype = ctypes.c_size_t
    lib.rz_lm_head_q4_0_topk.argtypes = [vp, vp, i, vp, vp, i, i, i, vp, vp, vp, ctypes.c_size_t, vp]
    for fn in ("rz_q8_1_quantize", "rz_rmsnorm_q8_1", "rz_q4k_q8_gemv", "rz_q4k_q8_gemv_add",
               "rz_q4k_q8_gemv_f32", "rz_q4k_q8_gemv_multi", "rz_rmsnorm_q4k_q8_gemv_multi",
               "rz_rmsnorm_swiglu_ffn_q4k_add", "rz_q4k_q8_gemv_f32_add",
               "rz_q4_0_gemv", "rz_swiglu_ffn_q4k",
               "rz_swiglu_ffn_q4k_add", "rz_q4k_gemv", "rz_swiglu_ffn_q4k_f32",
               "rz_lm_head_q4_0", "rz_lm_head_q4_0_noalloc", "rz_gelu_ffn_q4_0",
               "rz_topk_f32", "rz_lm_head_q4_0_topk", "rz_abi_version"):
        getattr(lib, fn).restype = i
    lib.rz_last_error.argtypes = []
    lib.rz_last_error.restype = ctypes.c_char_p
    lib.rz_abi_version.argtypes = []
    _LIB = lib
    return lib


def rz_last_error() -> str:
    return load_library().rz_last_error().decode()


def rz_abi_version() -> int:
    return load_library().rz_abi_version()


def q8_1_nbytes(n_padded: int, n_tokens: int = 1) -> int:
    return n_tokens * (n_padded // 32) * Q8_1_BLOCK_BYTES


def _ptr(t):
    """Device pointer of a tensor (or pass an int / None through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("librz takes device tensors (got a %s tensor)" % t.device)
    if not t.is_contiguous():
        raise ValueError("librz takes contiguous tensors")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc != RZ_OK:
        raise RzError(rc, rz_last_error())


def _need(t, nbytes: int, name: str):
    if t is None or isinstance(t, int):
        return
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError("%s holds %d bytes, needs %d" % (name, have, nbytes))


def rz_q8_1_quantize(x, n: int, n_padded: int, n_tokens: int, x_q8, stream=None) -> None:
    """x fp32 [n_tokens, n] -> x_q8 uint8 [n_tokens * n_padded/32 * 40]."""
    _need(x, 4 * n * n_tokens, "x")
    _need(x_q8, q8_1_nbytes(n_padded, n_tokens) if n_padded > 0 else 0, "x_q8")
    _check(load_library().rz_q8_1_quantize(_ptr(x), n, n_padded, n_tokens, _ptr(x_q8),
                                           _stream(stream)))


def rz_rmsnorm_q8_1(x, gamma, eps: float, n: int, n_padded: int, n_tokens: int, normed, x_q8,
                    stream=None) -> None:
    """RMSNorm of x fp32 [n_tokens, n] with weights gamma [n], quantized to
    x_q8 uint8 [n_tokens * n_padded/32 * 40]; normed fp32 [n_tokens, n] is
    written too unless None."""
    _need(x, 4 * n * n_tokens, "x")
    _need(gamma, 4 * n, "gamma")
    _need(normed, 4 * n * n_tokens, "normed")
    _need(x_q8, q8_1_nbytes(n_padded, n_tokens) if n_padded > 0 else 0, "x_q8")
    _check(load_library().rz_rmsnorm_q8_1(_ptr(x), _ptr(gamma), float(eps), n, n_padded,
                                          n_tokens, _ptr(normed), _ptr(x_q8), _stream(stream)))


def rz_q4k_q8_gemv(w_q4k, x_q8, y, out_dim: int, in_dim: int, n_tokens: int = 1,
                   stream=None) -> None:
    """y fp32 [n_tokens, out_dim] = W (Q4_K [out_dim, in_dim/256, 144]) x (Q8_1)."""
    if in_dim > 0 and in_dim % 256 == 0 and out_dim > 0:
        _need(w_q4k, out_dim * (in_dim // 256) * Q4K_BLOCK_BYTES, "w_q4k")
        _need(x_q8, q8_1_nbytes(in_dim, n_tokens), "x_q8")
        _need(y, 4 * out_dim * n_tokens, "y")
    _check(load_library().rz_q4k_q8_gemv(_ptr(w_q4k), _ptr(x_q8), _ptr(y), out_dim, in_dim,
                                         n_tokens, _stream(stream)))


def rz_q4k_q8_gemv_add(w_q4k, x_q8, r, y, out_dim: int, in_dim: int, n_tokens: int = 1,
                       stream=None) -> None:
    """y fp32 [n_tokens, out_dim] = W (Q4_K) x (Q8_1) + r; r may be y itself."""
    if in_dim > 0 and in_dim % 256 == 0 and out_dim > 0:
        _need(w_q4k, out_dim * (in_dim // 256) * Q4K_BLOCK_BYTES, "w_q4k")
        _need(x_q8, q8_1_nbytes(in_dim, n_tokens), "x_q8")
        _need(r, 4 * out_dim * n_tokens, "r")
        _need(y, 4 * out_dim * n_tokens, "y")
    _check(load_library().rz_q4k_q8_gemv_add(_ptr(w_q4k), _ptr(x_q8), _ptr(r), _ptr(y), out_dim,
                                             in_dim, n_tokens, _stream(stream)))


def rz_q4k_q8_gemv_multi(ws, x_q8, ys, out_dims, in_dim: int, n_tokens: int = 1,
                         stream=None) -> None:
    """ys[m] fp32 [n_tokens, out_dims[m]] = ws[m] (Q4_K) x (Q8_1) for every m,
    in one launch (see rz_q4k_q8_gemv_multi in include/rz.h)."""
    n = len(ws)
    if len(ys) != n or len(out_dims) != n:
        raise ValueError("ws, ys and out_dims must have the same length")
    if in_dim > 0 and in_dim % 256 == 0:
        _need(x_q8, q8_1_nbytes(in_dim, n_tokens), "x_q8")
        for w, y, od in zip(ws, ys, out_dims):
            if od > 0:
                _need(w, od * (in_dim // 256) * Q4K_BLOCK_BYTES, "w_q4k")
                _need(y, 4 * od * n_tokens, "y")
    wa = (ctypes.c_void_p * max(n, 1))(*[_ptr(w) for w in ws])
    ya = (ctypes.c_void_p * max(n, 1))(*[_ptr(y) for y in ys])
    da = (ctypes.c_int * max(n, 1))(*[int(d) for d in out_dims])
    _check(load_library().rz_q4k_q8_gemv_multi(n, wa, ya, da, _ptr(x_q8), in_dim, n_tokens,
                                               _stream(stream)))


def rz_rmsnorm_q4k_q8_gemv_multi(ws, x, gamma, eps: float, n: int, x_q8, ys, out_dims,
                                 in_dim: int, stream=None) -> None:
    """ys[m] fp32 [out_dims[m]] = ws[m] (Q4_K) x Q8_1(RMSNorm(x[:n], gamma, eps)) for
    every m, in one launch; x_q8 (or None) receives the Q8_1 blocks."""
    nm = len(ws)
    if len(ys) != nm or len(out_dims) != nm:
        raise ValueError("ws, ys and out_dims must have the same length")
    _need(x, 4 * n, "x")
    _need(gamma, 4 * n, "gamma")
    if in_dim > 0 and in_dim % 256 == 0:
        _need(x_q8, q8_1_nbytes(in_dim), "x_q8")
        for w, y, od in zip(ws, ys, out_dims):
            if od > 0:
                _need(w, od * (in_dim // 256) * Q4K_BLOCK_BYTES, "w_q4k")
                _need(y, 4 * od, "y")
    wa = (ctypes.c_void_p * max(nm, 1))(*[_ptr(w) for w in ws])
    ya = (ctypes.c_void_p * max(nm, 1))(*[_ptr(y) for y in ys])
    da = (ctypes.c_int * max(nm, 1))(*[int(d) for d in out_dims])
    _check(load_library().rz_rmsnorm_q4k_q8_gemv_multi(nm, wa, ya, da, _ptr(x), _ptr(gamma),
                                                       eps, n, _ptr(x_q8), in_dim,
                                                       _stream(stream)))


def rz_rmsnorm_swiglu_ffn_q4k_add(w_gate, w_up, w_down, x, gamma, eps: float, h, h_q8, y, gu,
                                  hidden_dim: int, inter_dim: int, stream=None) -> None:
    """The pre-norm FFN block: y = x + SwiGLU chain of Q8_1(RMSNorm(x, gamma, eps));
    y may be x.  h, h_q8 (and gu unless None) receive the chain's stages."""
    if hidden_dim > 0 and inter_dim > 0 and hidden_dim % 256 == 0 and inter_dim % 256 == 0:
        nw = inter_dim * (hidden_dim // 256) * Q4K_BLOCK_BYTES
        for t_, nm in ((w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down")):
            _need(t_, nw, nm)
        for t_, nb, nm in ((x, 4 * hidden_dim, "x"), (gamma, 4 * hidden_dim, "gamma"),
                           (h, 4 * inter_dim, "h"), (h_q8, q8_1_nbytes(inter_dim), "h_q8"),
                           (y, 4 * hidden_dim, "y"), (gu, 8 * inter_dim, "gu")):
            _need(t_, nb, nm)
    _check(load_library().rz_rmsnorm_swiglu_ffn_q4k_add(
        _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(x), _ptr(gamma), eps, _ptr(h), _ptr(h_q8),
        _ptr(y), _ptr(gu), hidden_dim, inter_dim, _stream(stream)))


def rz_q4k_q8_gemv_f32(w_q4k, x, n: int, x_q8, y, out_dim: int, in_dim: int,
                       stream=None) -> None:
    """Quantize fp32 x [n] to Q8_1 in-kernel (optionally writing the blocks to
    x_q8, or pass None) and compute y fp32 [out_dim] = W (Q4_K) x, one launch."""
    if in_dim > 0 and in_dim % 256 == 0 and out_dim > 0:
        _need(w_q4k, out_dim * (in_dim // 256) * Q4K_BLOCK_BYTES, "w_q4k")
        _need(x, 4 * n, "x")
        _need(x_q8, q8_1_nbytes(in_dim), "x_q8")
        _need(y, 4 * out_dim, "y")
    _check(load_library().rz_q4k_q8_gemv_f32(_ptr(w_q4k), _ptr(x), n, _ptr(x_q8), _ptr(y),
                                             out_dim, in_dim, _stream(stream)))


def rz_q4_0_gemv(w_q4_0, x, x_format: int, y, out_dim: int, in_dim: int, stream=None) -> None:
    """y fp32 [out_dim] = W (Q4_0 [out_dim, in_dim/32, 18]) x; x_format 0 = fp32, 1 = Q8_1."""
    if in_dim > 0 and in_dim % 64 == 0 and out_dim > 0:
        _need(w_q4_0, out_dim * (in_dim // 32) * Q4_0_BLOCK_BYTES, "w_q4_0")
        _need(x, 4 * in_dim if x_format == 0 else q8_1_nbytes(in_dim), "x")
        _need(y, 4 * out_dim, "y")
    _check(load_library().rz_q4_0_gemv(_ptr(w_q4_0), _ptr(x), x_format, _ptr(y), out_dim,
                                       in_dim, _stream(stream)))


def rz_swiglu_ffn_q4k(w_gate, w_up, w_down, x_q8, h, h_q8, y, gu, hidden_dim: int,
                      inter_dim: int, stream=None) -> None:
    """SwiGLU FFN: h = silu(W_gate x) * (W_up x), h_q8 = Q8_1(h), y = W_down h_q8."""
    if hidden_dim > 0 and inter_dim > 0 and hidden_dim % 256 == 0 and inter_dim % 256 == 0:
        nw = inter_dim * (hidden_dim // 256) * Q4K_BLOCK_BYTES
        _need(w_gate, nw, "w_gate")
        _need(w_up, nw, "w_up")
        _need(w_down, nw, "w_down")
        _need(x_q8, q8_1_nbytes(hidden_dim), "x_q8")
        _need(h, 4 * inter_dim, "h")
        _need(h_q8, q8_1_nbytes(inter_dim), "h_q8")
        _need(y, 4 * hidden_dim, "y")
        _need(gu, 8 * inter_dim, "gu")
    _check(load_library().rz_swiglu_ffn_q4k(_ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(x_q8),
                                            _ptr(h), _ptr(h_q8), _ptr(y), _ptr(gu), hidden_dim,
                                            inter_dim, _stream(stream)))


def rz_swiglu_ffn_q4k_add(w_gate, w_up, w_down, x_q8, h, h_q8, r, y, gu, hidden_dim: int,
                          inter_dim: int, stream=None) -> None:
    """rz_swiglu_ffn_q4k with the residual: y = W_down h_q8 + r (r may be y)."""
    if hidden_dim > 0 and inter_dim > 0 and hidden_dim % 256 == 0 and inter_dim % 256 == 0:
        nw = inter_dim * (hidden_dim // 256) * Q4K_BLOCK_BYTES
        _need(w_gate, nw, "w_gate")
        _need(w_up, nw, "w_up")
        _need(w_down, nw, "w_down")
        _need(x_q8, q8_1_nbytes(hidden_dim), "x_q8")
        _need(h, 4 * inter_dim, "h")
        _need(h_q8, q8_1_nbytes(inter_dim), "h_q8")
        _need(r, 4 * hidden_dim, "r")
        _need(y, 4 * hidden_dim, "y")
        _need(gu, 8 * inter_dim, "gu")
    _check(load_library().rz_swiglu_ffn_q4k_add(_ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                                _ptr(x_q8), _ptr(h), _ptr(h_q8), _ptr(r), _ptr(y),
                                                _ptr(gu), hidden_dim, inter_dim, _stream(stream)))


def rz_q4k_q8_gemv_f32_add(w_q4k, x, n: int, x_q8, r, y, out_dim: int, in_dim: int,
                           stream=None) -> None:
    """y fp32 [out_dim] = W (Q4_K) x Q8_1(x[:n]) + r in one launch; r may be y;
    x_q8 (or None) receives the Q8_1 blocks."""
    if out_dim > 0 and in_dim > 0 and in_dim % 256 == 0:
        _need(w_q4k, out_dim * (in_dim // 256) * Q4K_BLOCK_BYTES, "w_q4k")
        _need(x, 4 * n, "x")
        _need(x_q8, q8_1_nbytes(in_dim), "x_q8")
        _need(r, 4 * out_dim, "r")
        _need(y, 4 * out_dim, "y")
    _check(load_library().rz_q4k_q8_gemv_f32_add(_ptr(w_q4k), _ptr(x), n, _ptr(x_q8), _ptr(r),
                                                 _ptr(y), out_dim, in_dim, _stream(stream)))


def rz_q4k_gemv(w_q4k, x, n: int, y, out_dim: int, in_dim: int, stream=None) -> None:
    """y fp32 [out_dim] = W (Q4_K) x with x fp32 [n] (zero past n), no Q8_1."""
    if in_dim > 0 and in_dim % 256 == 0 and out_dim > 0:
        _need(w_q4k, out_dim * (in_dim // 256) * Q4K_BLOCK_BYTES, "w_q4k")
        _need(x, 4 * n, "x")
        _need(y, 4 * out_dim, "y")
    _check(load_library().rz_q4k_gemv(_ptr(w_q4k), _ptr(x), n, _ptr(y), out_dim, in_dim,
                                      _stream(stream)))


def rz_swiglu_ffn_q4k_f32(w_gate, w_up, w_down, x, h, y, gu, hidden_dim: int, inter_dim: int,
                          stream=None) -> None:
    """SwiGLU FFN on fp32 activations: h = silu(W_gate x) * (W_up x), y = W_down h."""
    if hidden_dim > 0 and inter_dim > 0 and hidden_dim % 256 == 0 and inter_dim % 256 == 0:
        nw = inter_dim * (hidden_dim // 256) * Q4K_BLOCK_BYTES
        _need(w_gate, nw, "w_gate")
        _need(w_up, nw, "w_up")
        _need(w_down, nw, "w_down")
        _need(x, 4 * hidden_dim, "x")
        _need(h, 4 * inter_dim, "h")
        _need(y, 4 * hidden_dim, "y")
        _need(gu, 8 * inter_dim, "gu")
    _check(load_library().rz_swiglu_ffn_q4k_f32(_ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(x),
                                                _ptr(h), _ptr(y), _ptr(gu), hidden_dim,
                                                inter_dim, _stream(stream)))


def rz_lm_head_q4_0_workspace_bytes(out_dim: int, in_dim: int, x_format: int) -> int:
    """Workspace bytes rz_lm_head_q4_0 needs for its argmax (0 for bad arguments)."""
    return int(load_library().rz_lm_head_q4_0_workspace_bytes(out_dim, in_dim, x_format))


def rz_lm_head_q4_0(w_q4_0, x, x_format: int, bias, logits, out_dim: int, in_dim: int,
                    argmax_idx=None, argmax_val=None, workspace=None, stream=None) -> None:
    """logits fp32 [out_dim] = W (Q4_0) x + bias (bias may be None); with
    argmax_idx (int32 [1]) and/or argmax_val (fp32 [1]) also the index and value
    of the largest logit (smallest index on ties), using `workspace` (device
    bytes, rz_lm_head_q4_0_workspace_bytes of them)."""
    if in_dim > 0 and in_dim % 64 == 0 and out_dim > 0 and x_format in (0, 1):
        _need(w_q4_0, out_dim * (in_dim // 32) * Q4_0_BLOCK_BYTES, "w_q4_0")
        _need(x, 4 * in_dim if x_format == 0 else q8_1_nbytes(in_dim), "x")
        _need(bias, 4 * out_dim, "bias")
        _need(logits, 4 * out_dim, "logits")
        _need(argmax_idx, 4, "argmax_idx")
        _need(argmax_val, 4, "argmax_val")
    ws_bytes = 0
    if workspace is not None and not isinstance(workspace, int):
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().rz_lm_head_q4_0(_ptr(w_q4_0), _ptr(x), x_format, _ptr(bias),
                                          _ptr(logits), out_dim, in_dim, _ptr(argmax_idx),
                                          _ptr(argmax_val), _ptr(workspace), ws_bytes,
                                          _stream(stream)))


def rz_lm_head_q4_0_noalloc(w_q4_0, x, x_format: int, bias, logits, out_dim: int, in_dim: int,
                            argmax_idx=None, argmax_val=None, stream=None) -> None:
    """rz_lm_head_q4_0 without a workspace: the argmax pairs live in the
    library's fixed per-GPU array (at most NOALLOC_ARGMAX_PAIRS of them).
    Calls on one GPU that may overlap race on that array."""
    if in_dim > 0 and in_dim % 64 == 0 and out_dim > 0 and x_format in (0, 1):
        _need(w_q4_0, out_dim * (in_dim // 32) * Q4_0_BLOCK_BYTES, "w_q4_0")
        _need(x, 4 * in_dim if x_format == 0 else q8_1_nbytes(in_dim), "x")
        _need(bias, 4 * out_dim, "bias")
        _need(logits, 4 * out_dim, "logits")
        _need(argmax_idx, 4, "argmax_idx")
        _need(argmax_val, 4, "argmax_val")
    _check(load_library().rz_lm_head_q4_0_noalloc(_ptr(w_q4_0), _ptr(x), x_format, _ptr(bias),
                                                  _ptr(logits), out_dim, in_dim, _ptr(argmax_idx),
                                                  _ptr(argmax_val), _stream(stream)))


def _nbytes(t) -> int:
    return 0 if t is None or isinstance(t, int) else t.numel() * t.element_size()


def rz_topk_f32_workspace_bytes(n: int, k: int) -> int:
    """Workspace bytes rz_topk_f32 needs (0 for arguments it would reject)."""
    return int(load_library().rz_topk_f32_workspace_bytes(n, k))


def rz_topk_f32(values, n: int, k: int, topk_idx=None, topk_val=None, workspace=None,
                stream=None) -> None:
    """The k largest of values fp32 [n], largest first, equal values by index:
    their indices into topk_idx (int32 [k]) and/or the values into topk_val
    (fp32 [k]), using `workspace` (rz_topk_f32_workspace_bytes of them)."""
    if n > 0 and 0 < k <= n:
        _need(values, 4 * n, "values")
        _need(topk_idx, 4 * k, "topk_idx")
        _need(topk_val, 4 * k, "topk_val")
    _check(load_library().rz_topk_f32(_ptr(values), n, k, _ptr(topk_idx), _ptr(topk_val),
                                      _ptr(workspace), _nbytes(workspace), _stream(stream)))


def rz_lm_head_q4_0_topk(w_q4_0, x, x_format: int, bias, logits, out_dim: int, in_dim: int,
                         k: int, topk_idx=None, topk_val=None, workspace=None,
                         stream=None) -> None:
    """rz_lm_head_q4_0's logits (bias may be None), then the top k of them as
    rz_topk_f32 selects them, in one call."""
    if in_dim > 0 and in_dim % 64 == 0 and out_dim > 0 and x_format in (0, 1):
        _need(w_q4_0, out_dim * (in_dim // 32) * Q4_0_BLOCK_BYTES, "w_q4_0")
        _need(x, 4 * in_dim if x_format == 0 else q8_1_nbytes(in_dim), "x")
        _need(bias, 4 * out_dim, "bias")
        _need(logits, 4 * out_dim, "logits")
        if 0 < k <= out_dim:
            _need(topk_idx, 4 * k, "topk_idx")
            _need(topk_val, 4 * k, "topk_val")
    _check(load_library().rz_lm_head_q4_0_topk(_ptr(w_q4_0), _ptr(x), x_format, _ptr(bias),
                                               _ptr(logits), out_dim, in_dim, k, _ptr(topk_idx),
                                               _ptr(topk_val), _ptr(workspace),
                                               _nbytes(workspace), _stream(stream)))


def rz_gelu_ffn_q4_0(w_up, w_down, x, up_bias, down_bias, h, y, hidden_dim: int, inter_dim: int,
                     stream=None) -> None:
    """GELU FFN on Q4_0 weights: h = gelu(W_up x + up_bias), y = W_down h + down_bias
    (either bias may be None)."""
    if hidden_dim > 0 and inter_dim > 0 and hidden_dim % 64 == 0 and inter_dim % 64 == 0:
        nw = inter_dim * (hidden_dim // 32) * Q4_0_BLOCK_BYTES
        _need(w_up, nw, "w_up")
        _need(w_down, nw, "w_down")
        _need(x, 4 * hidden_dim, "x")
        _need(up_bias, 4 * inter_dim, "up_bias")
        _need(down_bias, 4 * hidden_dim, "down_bias")
        _need(h, 4 * inter_dim, "h")
        _need(y, 4 * hidden_dim, "y")
    _check(load_library().rz_gelu_ffn_q4_0(_ptr(w_up), _ptr(w_down), _ptr(x), _ptr(up_bias),
                                           _ptr(down_bias), _ptr(h), _ptr(y), hidden_dim,
                                           inter_dim, _stream(stream)))
