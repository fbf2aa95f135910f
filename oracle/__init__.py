"""CPU oracle for the Q4_K / Q4_0 x Q8_1 GEMV path -- TEST INFRASTRUCTURE ONLY.

A plain, slow statement of what the path computes, written from the realizar
source pages (docs.rs, realizar 0.8.4/0.8.5):

* ``src/cuda/executor/cached.rs``, ``transformer_layer_gpu_true_dp4a``: the
  normed activation is quantized to Q8_1 once (step 2) and shared by the Q, K and
  V projections, which are Q4_K x Q8_1 integer dot products (step 3); the
  attention output is requantized before the O projection (steps 5-6); the FFN
  is the SwiGLU chain on the same integer path (step 9).
* ``src/gpu/adapters/using.rs``, ``GpuModelQ4::forward`` step 5: the LM head is a
  Q4_0 GEMV over the fp32 normed hidden state; ``ffn_swiglu_gpu``: gate and up
  GEMVs, ``silu(gate) * up``, down GEMV.
* ``src/gguf/cuda/clone_layer_weights.rs``, ``cuda_swiglu_ffn``: SiLU applied to
  the gate output, then multiplied elementwise by the up output.
* ``src/cuda/executor/layers/forward_utils.rs``, ``pad_and_upload_input``: the
  activation is zero-padded to a multiple of the 256-value super-block.
* ``cached.rs``, ``transformer_layer_gpu_cached`` steps 2, 4 and 7: the same
  projections and FFN with the fp32 normed activation, not quantized
  (``q4k_gemv_cached_async``, ``fused_ffn_swiglu_gpu``).
* ``src/gpu/adapters/using.rs``, ``rms_norm_inplace``, and ``cached.rs`` steps 1, 7,
  8 and 10: the RMSNorm before the quantize and the residual adds after the O
  projection and the FFN.

* ``cached.rs``, ``preload_lm_head_bias`` and ``dispatch_lm_head_and_download``:
  the LM head's output bias and the logits it produces (the greedy token is the
  index of the largest logit).

* using.rs ``ffn_standard_gpu`` and clone_layer_weights.rs ``cuda_gelu_ffn``: the
  GELU FFN (up projection, optional bias, GELU, down projection, optional bias).

The block formats are not printed on the pages; the GGML layouts the pages name
(Q4_K super-blocks of 256 values, type id 12; Q4_0; Q8_1) are read as written in
each module's docstring.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path never calls it.

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests against
hand-worked blocks (``tests/golden/``), closed forms, exact-integer cases and the
dequantize-then-dot identity.
"""
from .q8_1 import (QK8_1, Q8_1_BLOCK_BYTES, quantize_q8_1, q8_1_to_bytes,
                   q8_1_from_bytes, dequantize_q8_1, Q8Blocks)
from .q4k import (q4k_fields, q4k_unpack_scales, dequantize_q4k,
                  gemv_q4k_q8_def, gemv_q4k_q8_int, gemv_q4k_f32)
from .q4_0 import (q4_0_fields, dequantize_q4_0, gemv_q4_0_f32,
                   gemv_q4_0_q8_int)
from .swiglu import (silu, silu_grad, silu_curv, swiglu, ffn_swiglu_q4k, ffn_swiglu_q4k_f32,
                     h_tolerance)
from .tolerance import gemv_tolerance, GEMV_REL, GEMV_ABS
from .norm import rmsnorm, rmsnorm_tolerance, residual_add
from .lm_head import lm_head_q4_0, argmax_first, topk_first
from .gelu import gelu, gelu_grad, gelu_h_tolerance, ffn_gelu_q4_0

__all__ = [
    "QK8_1", "Q8_1_BLOCK_BYTES", "quantize_q8_1", "q8_1_to_bytes", "q8_1_from_bytes",
    "dequantize_q8_1", "Q8Blocks",
    "q4k_fields", "q4k_unpack_scales", "dequantize_q4k", "gemv_q4k_q8_def",
    "gemv_q4k_q8_int", "gemv_q4k_f32",
    "q4_0_fields", "dequantize_q4_0", "gemv_q4_0_f32", "gemv_q4_0_q8_int",
    "silu", "silu_grad", "silu_curv", "swiglu", "ffn_swiglu_q4k", "ffn_swiglu_q4k_f32", "h_tolerance",
    "gemv_tolerance", "GEMV_REL", "GEMV_ABS",
    "rmsnorm", "rmsnorm_tolerance", "residual_add",
    "lm_head_q4_0", "argmax_first", "topk_first",
    "gelu", "gelu_grad", "gelu_h_tolerance", "ffn_gelu_q4_0",
]
