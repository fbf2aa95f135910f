/*
 * rz.h -- C ABI of librz.so: integer-quantized GEMV for MI355X (gfx950).
 *
 * The operations are the quantized decode-time matrix-vector products of the
 * realizar source pages (docs.rs, realizar 0.8.4 / 0.8.5):
 *
 *   - src/cuda/executor/cached.rs, transformer_layer_gpu_true_dp4a: the fp32
 *     activation is quantized to Q8_1 once (step 2) and multiplied by Q4_K
 *     weight matrices with integer dot products (steps 3 and 6); the FFN runs
 *     on the same integer path (step 9);
 *   - src/gpu/adapters/using.rs, GpuModelQ4::forward step 5: the LM head is a
 *     Q4_0 GEMV over the fp32 normed hidden state;
 *   - src/cuda/executor/layers/forward_utils.rs, pad_and_upload_input: the
 *     activation is zero-padded to a multiple of the 256-value super-block.
 *
 * Formats (GGML layouts; little endian):
 *   Q8_1 block, 40 bytes : float d; float s; int8 q[32];   x ~= d * q, s = d * sum(q)
 *   Q4_K super-block, 144: fp16 d; fp16 dmin; u8 scales[12]; u8 qs[128]  (256 values)
 *   Q4_0 block, 18 bytes : fp16 d; u8 qs[16]                            (32 values)
 * Weight matrices are row-major: row r is out_dim-major, its blocks follow
 * each other along in_dim.  Arguments are ordered (out_dim, in_dim) as in the
 * pages' q4k_q8_gemv_async / q4_0_gemv_into calls.
 *
 * Conventions shared by every entry point:
 *   - every pointer argument except `stream` is a DEVICE pointer owned by the
 *     caller; the library allocates, frees and synchronises nothing and keeps
 *     no state but a thread-local error message;
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream); the
 *     work is enqueued asynchronously on it;
 *   - arguments are validated on the host before any HIP call; the return
 *     value is RZ_OK or a negative RZ_E* code, and rz_last_error() then holds a
 *     message.  A device-side fault surfaces at the caller's next sync.
 *   - in_dim is always the PADDED length (the caller zero-pads activations;
 *     rz_q8_1_quantize does it while quantizing);
 *   - empty work is an error, not a no-op: a zero dimension gives RZ_EDIM and
 *     zero tokens or matrices RZ_EINVAL, before anything is enqueued;
 *   - an output must not overlap the call's weights, its activations or its
 *     other outputs, except where an entry point allows it (a residual may be
 *     the output it is added to, a bias may be its output, a chain's final
 *     output may be its input); an overlap gives RZ_EINVAL.
 */
#ifndef RZ_H
#define RZ_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RZ_OK 0
#define RZ_EINVAL (-1)  /* null pointer, bad n_tokens or format flag          */
#define RZ_EDIM (-2)    /* dimension not a positive multiple of the block size */
#define RZ_EALIGN (-3)  /* pointer alignment below the stated requirement      */
#define RZ_ELAUNCH (-4) /* the HIP runtime rejected a kernel launch            */

#define RZ_Q8_1_BLOCK_BYTES 40
#define RZ_Q4K_BLOCK_BYTES 144
#define RZ_Q4_0_BLOCK_BYTES 18
#define RZ_MAX_TOKENS 8
#define RZ_MAX_MATS 8
#define RZ_MAX_DIM (1 << 24)
#define RZ_TOPK_MAX 128

/* rz_q8_1_quantize -- fp32 activations to Q8_1 blocks.
 * Passage: realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_true_dp4a, steps 2 and 5 (quantize once, share).
 * Per block of 32: amax = max|x|, d = amax / 127 (IEEE fp32 division),
 * q = round-half-even(x / d) (fp32 division), s = d * sum(q); amax == 0 gives
 * an all-zero block.
 *   x        fp32 [n_tokens][n] (token rows of n values, contiguous), 4-byte aligned
 *   n        logical length, 1 <= n <= n_padded
 *   n_padded multiple of 32; values n..n_padded-1 are taken as +0.0
 *   n_tokens 1 <= n_tokens <= RZ_MAX_TOKENS
 *   x_q8     out: [n_tokens][n_padded/32] blocks, 16-byte aligned
 * Errors: RZ_EINVAL (null pointer, n_tokens out of range), RZ_EDIM,
 * RZ_EALIGN, RZ_ELAUNCH.  The output is bit-exact (a unique result). */
int rz_q8_1_quantize(const float* x, int n, int n_padded, int n_tokens,
                     void* x_q8, void* stream);

/* rz_rmsnorm_q8_1 -- RMSNorm of fp32 activations, quantized to Q8_1, in one
 * launch.
 * Passages: realizar 0.8.4 src/gpu/adapters/using.rs, rms_norm_inplace (the
 * root of mean(x^2) + eps is the RMS; each value is multiplied by 1/RMS and
 * by its weight); realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_true_dp4a, steps 1-2 and 8 (the normed activation
 * is quantized once for the projections that follow).
 * Per token: ss = sum(x^2) in fp32, scale = 1 / sqrt(ss / n + eps) (IEEE
 * division and square root), v = (x * scale) * gamma; the Q8_1 blocks of v
 * then follow the rule of rz_q8_1_quantize and equal
 * rz_q8_1_quantize(v) byte for byte.  ss is summed in a fixed order (per
 * thread over 4 of every 1024 values, then an 8-level tree; rows longer than
 * 16384 values: 4 of every 4096, then 10 levels), so v differs from the exact
 * value by rounding only, the same on every run.
 *   x        fp32 [n_tokens][n], 4-byte aligned
 *   gamma    fp32 [n] weights, 4-byte aligned
 *   eps      > 0 and finite
 *   n        1 <= n <= n_padded; n_padded multiple of 32 (values n..n_padded-1
 *            are +0.0, as for rz_q8_1_quantize)
 *   n_tokens 1..RZ_MAX_TOKENS
 *   normed   optional out (NULL to skip): fp32 [n_tokens][n], the values v
 *   x_q8     out: [n_tokens][n_padded/32] blocks, 16-byte aligned
 * Inputs whose sum of squares overflows fp32 are outside the contract.
 * Errors: RZ_EINVAL (null pointer, n_tokens or eps), RZ_EDIM, RZ_EALIGN,
 * RZ_ELAUNCH. */
int rz_rmsnorm_q8_1(const float* x, const float* gamma, float eps, int n, int n_padded,
                    int n_tokens, float* normed, void* x_q8, void* stream);

/* rz_q4k_q8_gemv -- y = W x with W Q4_K and x Q8_1, for 1..8 tokens.
 * Passage: realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_true_dp4a, steps 3 and 6 (Q4K x Q8 integer dot
 * product; weights streamed once per call, whatever the token count).
 * Per 32-value sub-block j of super-block b: isum = sum(q4 * q8) in int32,
 * y += d * sc_j * d_x * isum - dmin * m_j * s_x.
 *   w_q4k    [out_dim][in_dim/256] super-blocks, 16-byte aligned
 *   x_q8     [n_tokens][in_dim/32] Q8_1 blocks, 16-byte aligned
 *   y        out: fp32 [n_tokens][out_dim] (token-major), 4-byte aligned
 *   out_dim  >= 1; in_dim multiple of 256 (padded); both <= RZ_MAX_DIM;
 *            the matrix (out_dim * in_dim/256 * 144 bytes) < 2 GiB
 *   n_tokens 1..RZ_MAX_TOKENS
 * Errors: RZ_EINVAL, RZ_EDIM, RZ_EALIGN, RZ_ELAUNCH. */
int rz_q4k_q8_gemv(const void* w_q4k, const void* x_q8, float* y,
                   int out_dim, int in_dim, int n_tokens, void* stream);

/* rz_q4k_q8_gemv_add -- y = W x + r: the GEMV with the residual add in its
 * store.
 * Passage: realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_true_dp4a, steps 6-7 and 10 (the output projection
 * and the FFN output are each added to the layer's running hidden state).
 * Same operation as rz_q4k_q8_gemv, plus r.  When one pass covers the row
 * (in_dim <= 16384 for 1-2 tokens, <= 4096 for 3-8 tokens) y is
 * fl32(rz_q4k_q8_gemv result + r) bit for bit; longer rows run in column
 * passes, and r is added to the first pass's partial sum.
 *   r        fp32 [n_tokens][out_dim] (token-major, like y), 4-byte aligned;
 *            may be y itself (in place) but must not overlap it otherwise
 *   w_q4k, x_q8, y, out_dim, in_dim, n_tokens: as for rz_q4k_q8_gemv
 * Errors: RZ_EINVAL (also a partial overlap of r and y), RZ_EDIM, RZ_EALIGN,
 * RZ_ELAUNCH. */
int rz_q4k_q8_gemv_add(const void* w_q4k, const void* x_q8, const float* r, float* y,
                       int out_dim, int in_dim, int n_tokens, void* stream);

/* rz_q4k_q8_gemv_multi -- several Q4_K matrices times one Q8_1 activation.
 * Passage: realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_true_dp4a, steps 2-3 (the activation is quantized
 * once and the Q, K and V projections all read it).
 * One launch covers the row groups of every matrix (small matrices such as a
 * GQA layer's K and V would otherwise pay a launch each); each y[m] equals
 * rz_q4k_q8_gemv(w_q4k[m], x_q8, y[m], out_dims[m], in_dim, n_tokens) bit for
 * bit.  With more than 2 tokens or in_dim above 16384 the matrices are
 * processed by one rz_q4k_q8_gemv call each.
 *   n_mats    1..RZ_MAX_MATS
 *   w_q4k     HOST array of n_mats device pointers; matrix m is
 *             [out_dims[m]][in_dim/256] super-blocks, 16-byte aligned, < 2 GiB
 *   y         HOST array of n_mats device pointers, out: fp32
 *             [n_tokens][out_dims[m]], 4-byte aligned, not overlapping
 *   out_dims  HOST array of n_mats row counts, each >= 1 and <= RZ_MAX_DIM
 *   x_q8, in_dim, n_tokens: as for rz_q4k_q8_gemv
 * The three host arrays are read during the call only.
 * Errors: RZ_EINVAL (null pointer or array entry, n_mats or n_tokens out of
 * range), RZ_EDIM, RZ_EALIGN, RZ_ELAUNCH. */
int rz_q4k_q8_gemv_multi(int n_mats, const void* const* w_q4k, float* const* y,
                         const int* out_dims, const void* x_q8, int in_dim, int n_tokens,
                         void* stream);

/* rz_rmsnorm_q4k_q8_gemv_multi -- RMSNorm, Q8_1 quantize and several Q4_K
 * GEMVs in one launch (one token).
 * Passages: realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_true_dp4a, steps 1-3 (RMSNorm of the hidden state,
 * one Q8_1 quantize, the Q, K and V projections); realizar 0.8.4
 * src/gpu/adapters/using.rs, rms_norm_inplace.
 * Bit for bit the result of rz_rmsnorm_q8_1(x, gamma, eps, n, in_dim, 1, NULL,
 * x_q8) followed by rz_q4k_q8_gemv_multi(n_mats, w_q4k, y, out_dims, x_q8,
 * in_dim, 1): every workgroup normalizes and quantizes the row into its LDS,
 * summing the squares in the same order as rz_rmsnorm_q8_1.
 *   n_mats, w_q4k, y, out_dims: as for rz_q4k_q8_gemv_multi (one token)
 *   x        fp32 [n], the hidden state, 4-byte aligned; values n..in_dim-1
 *            are taken as 0
 *   gamma    fp32 [n] RMSNorm weights, 4-byte aligned
 *   eps      > 0 and finite
 *   n        1 <= n <= in_dim
 *   x_q8     optional out (NULL to skip): the [in_dim/32] Q8_1 blocks of the
 *            normed row, 16-byte aligned
 *   in_dim   multiple of 256, <= 16384
 * Errors: RZ_EINVAL (null pointer or array entry, n_mats, eps, overlaps),
 * RZ_EDIM, RZ_EALIGN, RZ_ELAUNCH. */
int rz_rmsnorm_q4k_q8_gemv_multi(int n_mats, const void* const* w_q4k, float* const* y,
                                 const int* out_dims, const float* x, const float* gamma,
                                 float eps, int n, void* x_q8, int in_dim, void* stream);

/* rz_q4k_q8_gemv_f32 -- Q8_1 quantize and Q4_K x Q8_1 GEMV in one launch.
 * Passage: realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_true_dp4a, steps 2-3 (quantize the normed
 * activation to Q8_1, then the Q4K x Q8 integer dot product).
 * Bit for bit the result of rz_q8_1_quantize(x, n, in_dim, 1, x_q8) followed
 * by rz_q4k_q8_gemv(w_q4k, x_q8, y, out_dim, in_dim, 1): each workgroup
 * quantizes the activation into its LDS while its first weight tiles load.
 *   w_q4k    [out_dim][in_dim/256] super-blocks, 16-byte aligned, < 2 GiB
 *   x        fp32 [n], 4-byte aligned; values n..in_dim-1 are taken as 0
 *   n        1 <= n <= in_dim
 *   x_q8     optional out (NULL to skip): the [in_dim/32] Q8_1 blocks, for
 *            further projections of the same activation; 16-byte aligned
 *   y        out: fp32 [out_dim], 4-byte aligned
 *   in_dim   multiple of 256, <= 16384; one token
 * Errors: RZ_EINVAL, RZ_EDIM, RZ_EALIGN, RZ_ELAUNCH. */
int rz_q4k_q8_gemv_f32(const void* w_q4k, const float* x, int n, void* x_q8, float* y,
                       int out_dim, int in_dim, void* stream);

/* rz_q4k_q8_gemv_f32_add -- Q8_1 quantize, Q4_K x Q8_1 GEMV and a residual
 * add in one launch: y = W Q8_1(x) + r.
 * Passage: realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_true_dp4a, steps 5-7 (the attention output quantized
 * to Q8_1 for the O projection, whose output is added to the hidden state).
 * Bit for bit the result of rz_q8_1_quantize(x, n, in_dim, 1, x_q8) followed
 * by rz_q4k_q8_gemv_add(w_q4k, x_q8, r, y, out_dim, in_dim, 1).
 *   w_q4k, x, n, x_q8, out_dim, in_dim: as for rz_q4k_q8_gemv_f32
 *   r        fp32 [out_dim] residual, 4-byte aligned; may be y itself (the
 *            hidden state updated in place), otherwise must not overlap it
 *   y        out: fp32 [out_dim], 4-byte aligned
 * y and x_q8 must not overlap w_q4k, x or each other, nor x_q8 overlap r.
 * Errors: RZ_EINVAL (also overlaps), RZ_EDIM, RZ_EALIGN, RZ_ELAUNCH. */
int rz_q4k_q8_gemv_f32_add(const void* w_q4k, const float* x, int n, void* x_q8, const float* r,
                           float* y, int out_dim, int in_dim, void* stream);

/* rz_q4k_gemv -- y = W x with W Q4_K and x fp32, no Q8_1 (one token).
 * Passage: realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_cached, steps 2 and 4 (q4k_gemv_cached_async and
 * tiled_q4k_gemv_cached_async over the fp32 normed activation).
 * Per 32-value sub-block j of super-block b, in fp32:
 * y += d * (sc_j * sum(q * x)) - dmin * (m_j * sum(x)).
 *   w_q4k    [out_dim][in_dim/256] super-blocks, 16-byte aligned, < 2 GiB
 *   x        fp32 [n], 4-byte aligned; values n..in_dim-1 are taken as 0;
 *            must not overlap y
 *   n        1 <= n <= in_dim
 *   y        out: fp32 [out_dim], 4-byte aligned
 *   out_dim  >= 1; in_dim multiple of 256; both <= RZ_MAX_DIM (any in_dim:
 *            rows longer than 4096 values are walked in column chunks inside
 *            the one launch)
 * Errors: RZ_EINVAL (also overlap), RZ_EDIM, RZ_EALIGN, RZ_ELAUNCH. */
int rz_q4k_gemv(const void* w_q4k, const float* x, int n, float* y, int out_dim, int in_dim,
                void* stream);

/* rz_swiglu_ffn_q4k_f32 -- the SwiGLU FFN on fp32 activations, no Q8_1.
 * Passages: realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_cached step 7 (fused_ffn_swiglu_gpu); realizar 0.8.4
 * src/gpu/adapters/using.rs, ffn_swiglu_gpu (gate and up GEMVs, the fused
 * SwiGLU, the down GEMV of its output).
 *   g = W_gate x, u = W_up x            (rz_q4k_gemv arithmetic)
 *   h = silu(g) * u = g / (1 + exp(-g)) * u      (fp32)
 *   y = W_down h                        (rz_q4k_gemv arithmetic, in_dim inter)
 *   w_gate, w_up  [inter_dim][hidden_dim/256] super-blocks, 16-byte aligned
 *   w_down        [hidden_dim][inter_dim/256] super-blocks, 16-byte aligned
 *   x             fp32 [hidden_dim]
 *   h             out: fp32 [inter_dim]
 *   y             out: fp32 [hidden_dim] (may be x itself)
 *   gu            optional out (NULL to skip): fp32 [2][inter_dim], g then u
 *   hidden_dim, inter_dim  multiples of 256; each matrix < 2 GiB
 * Two kernels run in order on `stream`.  x, h and gu must not overlap each
 * other, nor y h or gu (y may overlap x).  Errors: RZ_EINVAL, RZ_EDIM,
 * RZ_EALIGN, RZ_ELAUNCH. */
int rz_swiglu_ffn_q4k_f32(const void* w_gate, const void* w_up, const void* w_down,
                          const float* x, float* h, float* y, float* gu, int hidden_dim,
                          int inter_dim, void* stream);

/* rz_q4_0_gemv -- y = W x with W Q4_0 and x fp32 or Q8_1 (the LM head).
 * Passage: realizar 0.8.4 src/gpu/adapters/using.rs, GpuModelQ4::forward
 * step 5 (q4_0_gemv_into(lm_head, normed, logits, vocab, hidden)).
 * Weight value = (q - 8) * d.
 *   w_q4_0   [out_dim][in_dim/32] blocks of 18 bytes, 4-byte aligned
 *   x        x_format 0: fp32 [in_dim], 16-byte aligned;
 *            x_format 1: Q8_1 [in_dim/32] blocks, 16-byte aligned
 *   y        out: fp32 [out_dim], 4-byte aligned
 *   in_dim   multiple of 64 (pairs of blocks keep every load 4-byte aligned)
 * Errors: RZ_EINVAL (also unknown x_format), RZ_EDIM, RZ_EALIGN, RZ_ELAUNCH. */
int rz_q4_0_gemv(const void* w_q4_0, const void* x, int x_format, float* y,
                 int out_dim, int in_dim, void* stream);

/* rz_lm_head_q4_0 -- the LM head: Q4_0 GEMV, output bias, greedy token.
 * Passages: realizar 0.8.4 src/gpu/adapters/using.rs, GpuModelQ4::forward
 * step 5 (the Q4_0 LM-head GEMV); realizar 0.8.5 src/cuda/executor/cached.rs,
 * preload_lm_head_bias (an output bias of vocab values added to the logits
 * after the GEMV) and dispatch_lm_head_and_download (the logits go to the
 * host, where the next token is chosen).
 *   logits = W x + bias, W x as rz_q4_0_gemv computes it (bit for bit when
 *   bias is NULL).  A row that one pass covers (in_dim <= 14336 for fp32 x,
 *   <= 16384 for Q8_1 x) gets fl32(W x + bias); a longer row is summed in
 *   column passes and the bias enters the first pass's partial sum, so a
 *   bias that is logits itself is read before it is overwritten, at every
 *   size.  With argmax_idx and/or argmax_val, the index of the
 *   largest logit (the smallest index among equal largest values) and that
 *   logit: each workgroup reduces its rows in the GEMV's epilogue and one
 *   small kernel merges the pairs, so a greedy step reads back 4 bytes
 *   instead of 4 * out_dim.
 *   w_q4_0, x, x_format, out_dim, in_dim: as for rz_q4_0_gemv
 *   bias        optional [out_dim] fp32 (NULL: none), 4-byte aligned; may be
 *               logits itself, must not overlap it otherwise
 *   logits      out: fp32 [out_dim], 4-byte aligned
 *   argmax_idx  optional out: int32 [1]; argmax_val optional out: fp32 [1]
 *   workspace   with an argmax output: device memory of at least
 *               rz_lm_head_q4_0_workspace_bytes(out_dim, in_dim, x_format)
 *               bytes, 4-byte aligned, not overlapping logits, bias or the
 *               argmax outputs; its contents on entry do not matter
 * Finite logits are assumed (a NaN never ranks as the largest).
 * Errors: RZ_EINVAL (also a short workspace or overlaps), RZ_EDIM,
 * RZ_EALIGN, RZ_ELAUNCH. */
int rz_lm_head_q4_0(const void* w_q4_0, const void* x, int x_format, const float* bias,
                    float* logits, int out_dim, int in_dim, int* argmax_idx, float* argmax_val,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace rz_lm_head_q4_0 needs for its argmax (0 for arguments it
 * would reject). */
size_t rz_lm_head_q4_0_workspace_bytes(int out_dim, int in_dim, int x_format);

/* rz_lm_head_q4_0_noalloc -- rz_lm_head_q4_0 without the workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 *   The arguments, checks, outputs and errors are those of rz_lm_head_q4_0
 *   (logits and the greedy token bit for bit), except that the argmax's
 *   per-workgroup (value, row) pairs live in a fixed array of the library:
 *   RZ_NOALLOC_ARGMAX_PAIRS pairs (256 KiB) on every GPU the library runs on,
 *   held until the process ends.  Nothing is allocated, freed or
 *   synchronised.  A shape whose argmax needs more pairs than that
 *   (rz_lm_head_q4_0_workspace_bytes / 8 > RZ_NOALLOC_ARGMAX_PAIRS; 151936 x
 *   1024 needs 2374, 262144 x 4096 needs 16384) gives RZ_EINVAL.  Without
 *   argmax_idx and argmax_val the array is not used.
 *   `stream` must belong to the current device (else RZ_EINVAL); the array of
 *   the current device is used.  Every call on a GPU shares that GPU's array
 *   and its last contents; the kernels write every pair a call reads before
 *   reading it, so nothing needs clearing.  Calls on one GPU whose kernels
 *   may overlap (different streams without ordering) race on the array and
 *   may return a wrong greedy token; calls in one stream, or ordered by
 *   events, do not.
 * Errors: those of rz_lm_head_q4_0, plus RZ_EINVAL for a shape beyond the
 * array or a stream of another device. */
#define RZ_NOALLOC_ARGMAX_PAIRS 32768
int rz_lm_head_q4_0_noalloc(const void* w_q4_0, const void* x, int x_format, const float* bias,
                            float* logits, int out_dim, int in_dim, int* argmax_idx,
                            float* argmax_val, void* stream);

/* rz_topk_f32 -- the k largest of n fp32 values, on the device: the
 * candidates a top-k sampler draws the next token from.
 * Passage: realizar 0.8.5 src/cuda/executor/cached.rs,
 * dispatch_lm_head_and_download (the logits go to the host, where the next
 * token is chosen); selecting the k candidates here reads back 8 k bytes
 * instead of 4 n.  The pages print no sampler: the k largest values in
 * descending order, equal values in index order (-0 and +0 equal), which makes
 * the selection unique; k = 1 is the greedy token of rz_lm_head_q4_0.
 *   values    fp32 [n], 4-byte aligned; finite values assumed
 *   n         1 .. RZ_MAX_DIM, at least k
 *   k         1 .. RZ_TOPK_MAX; n and k must also satisfy
 *             rz_topk_f32_workspace_bytes(n, k) > 0 (the candidates, n/2048
 *             rounded up times k, must not exceed 16384: n <= 262144 at k = 128,
 *             n <= 524288 at k <= 64, any n at k <= 2)
 *   topk_idx  optional out: int32 [k], the values' indices, largest first
 *   topk_val  optional out: fp32 [k], those values (at least one of the two)
 *   workspace device memory of rz_topk_f32_workspace_bytes(n, k) bytes,
 *             4-byte aligned; its contents on entry do not matter
 * Two kernels run in order on `stream`.  The outputs and the workspace must
 * not overlap the values or each other.
 * Errors: RZ_EINVAL (also k out of range, too many candidates, a short
 * workspace, overlaps), RZ_EDIM (n), RZ_EALIGN, RZ_ELAUNCH. */
int rz_topk_f32(const float* values, int n, int k, int* topk_idx, float* topk_val, void* workspace,
                size_t workspace_bytes, void* stream);

/* Bytes of workspace rz_topk_f32 needs (0 for arguments it would reject). */
size_t rz_topk_f32_workspace_bytes(int n, int k);

/* rz_lm_head_q4_0_topk -- the LM head with its top-k: rz_lm_head_q4_0's
 * logits (with the bias, without the greedy token), then rz_topk_f32 over
 * them, in one call (three kernels in order on `stream`).
 * Passages: those of rz_lm_head_q4_0 and rz_topk_f32.
 *   w_q4_0, x, x_format, bias, logits, out_dim, in_dim: as for rz_lm_head_q4_0
 *   k, topk_idx, topk_val: as for rz_topk_f32 with n = out_dim
 *   workspace rz_topk_f32_workspace_bytes(out_dim, k) bytes, 4-byte aligned
 * The top-k outputs and the workspace must not overlap the weights, x, the
 * bias, the logits or each other.
 * Errors: those of rz_lm_head_q4_0 and rz_topk_f32. */
int rz_lm_head_q4_0_topk(const void* w_q4_0, const void* x, int x_format, const float* bias,
                         float* logits, int out_dim, int in_dim, int k, int* topk_idx,
                         float* topk_val, void* workspace, size_t workspace_bytes, void* stream);

/* rz_gelu_ffn_q4_0 -- the GELU FFN on Q4_0 weights and fp32 activations.
 * Passages: realizar 0.8.4 src/gpu/adapters/using.rs, ffn_standard_gpu (up
 * projection, GELU in place, down projection, all Q4_0 GEMVs on fp32
 * activations); realizar 0.8.4 src/gguf/cuda/clone_layer_weights.rs,
 * cuda_gelu_ffn (the phi-2-style path, with optional biases).
 *   h = gelu(W_up x + up_bias)        gelu(u) = 0.5 u (1 + tanh(sqrt(2/pi)
 *                                      (u + 0.044715 u^3))), evaluated as
 *                                      u / (1 + exp(-2 sqrt(2/pi) (u + 0.044715 u^3)))
 *   y = W_down h + down_bias          (fp32 h, rz_q4_0_gemv arithmetic)
 *   w_up      [inter_dim][hidden_dim/32] Q4_0 blocks; w_down [hidden_dim][inter_dim/32];
 *             4-byte aligned
 *   x         fp32 [hidden_dim], 16-byte aligned
 *   up_bias   optional fp32 [inter_dim]; down_bias optional fp32 [hidden_dim]
 *   h         out: fp32 [inter_dim], 16-byte aligned (the down projection's input)
 *   y         out: fp32 [hidden_dim], 4-byte aligned
 *   hidden_dim, inter_dim  multiples of 64
 * Two GEMV launches run in order on `stream`.  Each adds its bias as
 * rz_lm_head_q4_0 does (in the first column pass; GELU after the last).  x
 * and h, h and y must not overlap; a bias may be its output itself (at any
 * size) but must not overlap it otherwise.
 * Errors: RZ_EINVAL, RZ_EDIM, RZ_EALIGN, RZ_ELAUNCH. */
int rz_gelu_ffn_q4_0(const void* w_up, const void* w_down, const float* x, const float* up_bias,
                     const float* down_bias, float* h, float* y, int hidden_dim, int inter_dim,
                     void* stream);

/* rz_swiglu_ffn_q4k -- the SwiGLU FFN on the integer path.
 * Passages: realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_true_dp4a step 9 (fused_ffn_swiglu_gpu_true_dp4a);
 * realizar 0.8.4 src/gguf/cuda/clone_layer_weights.rs, cuda_swiglu_ffn
 * (silu on gate, times up, then down).
 *   g = W_gate x, u = W_up x            (Q4_K x Q8_1, inter_dim rows)
 *   h = silu(g) * u = g / (1 + exp(-g)) * u      (fp32)
 *   h_q8 = Q8_1(h)                      (same rule as rz_q8_1_quantize)
 *   y = W_down h_q8                     (Q4_K x Q8_1, hidden_dim rows)
 *   w_gate, w_up  [inter_dim][hidden_dim/256] super-blocks, 16-byte aligned
 *   w_down        [hidden_dim][inter_dim/256] super-blocks, 16-byte aligned
 *   x_q8          [hidden_dim/32] Q8_1 blocks, 16-byte aligned
 *   h             out: fp32 [inter_dim]
 *   h_q8          out: [inter_dim/32] Q8_1 blocks, 16-byte aligned
 *   y             out: fp32 [hidden_dim]
 *   gu            optional out (NULL to skip): fp32 [2][inter_dim], g then u
 *   hidden_dim, inter_dim  multiples of 256; hidden_dim <= 16384 (the fused
 *                 gate/up kernel keeps a row's activation in registers);
 *                 each matrix < 2 GiB
 * Two kernels run in order on `stream`; h and h_q8 are written by the first
 * and read by the second.  h, h_q8, gu and y must not overlap x_q8, the
 * weights or each other (y may overlap x_q8).  Errors: RZ_EINVAL (also
 * overlaps), RZ_EDIM, RZ_EALIGN, RZ_ELAUNCH. */
int rz_swiglu_ffn_q4k(const void* w_gate, const void* w_up, const void* w_down,
                      const void* x_q8, float* h, void* h_q8, float* y,
                      float* gu, int hidden_dim, int inter_dim, void* stream);

/* rz_rmsnorm_swiglu_ffn_q4k_add -- the pre-norm FFN block of one token:
 * y = x + W_down Q8_1(silu(g) * u), with g, u = W_gate, W_up times
 * Q8_1(RMSNorm(x, gamma, eps)).
 * Passages: realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_true_dp4a, steps 8-10 (RMSNorm of the hidden state,
 * the FFN on its Q8_1 form, the residual add); realizar 0.8.4
 * src/gpu/adapters/using.rs, rms_norm_inplace and ffn_swiglu_gpu.
 * Bit for bit the result of rz_rmsnorm_q8_1(x, gamma, eps, hidden_dim,
 * hidden_dim, 1, NULL, x_q8) followed by rz_swiglu_ffn_q4k_add(w_gate, w_up,
 * w_down, x_q8, h, h_q8, x, y, gu, hidden_dim, inter_dim): every gate/up
 * workgroup normalizes and quantizes x into its LDS, summing the squares in
 * the same order as rz_rmsnorm_q8_1.  Two kernels run in order on `stream`.
 *   w_gate, w_up, w_down, h, h_q8, gu, hidden_dim, inter_dim: as for
 *                 rz_swiglu_ffn_q4k (hidden_dim <= 16384)
 *   x             fp32 [hidden_dim], the hidden state (also the residual),
 *                 4-byte aligned
 *   gamma         fp32 [hidden_dim] RMSNorm weights, 4-byte aligned
 *   eps           > 0 and finite
 *   y             out: fp32 [hidden_dim], 4-byte aligned; may be x itself
 * h, h_q8, gu and y must not overlap x, gamma, the weights or each other
 * (y may be x).  Errors: RZ_EINVAL (also overlaps), RZ_EDIM, RZ_EALIGN,
 * RZ_ELAUNCH. */
int rz_rmsnorm_swiglu_ffn_q4k_add(const void* w_gate, const void* w_up, const void* w_down,
                                  const float* x, const float* gamma, float eps, float* h,
                                  void* h_q8, float* y, float* gu, int hidden_dim, int inter_dim,
                                  void* stream);

/* rz_swiglu_ffn_q4k_add -- the SwiGLU FFN with the residual add:
 * y = W_down h_q8 + r.
 * Passage: realizar 0.8.5 src/cuda/executor/cached.rs,
 * transformer_layer_gpu_true_dp4a, steps 9-10 (the FFN output is added to
 * the hidden state).  Everything as rz_swiglu_ffn_q4k; the down projection
 * stores fl32(W_down h_q8 + r) as rz_q4k_q8_gemv_add does for one token.
 *   r        fp32 [hidden_dim], 4-byte aligned; may be y itself but must not
 *            overlap it otherwise, nor h, h_q8 or gu
 * Errors: RZ_EINVAL (also overlaps), RZ_EDIM, RZ_EALIGN, RZ_ELAUNCH. */
int rz_swiglu_ffn_q4k_add(const void* w_gate, const void* w_up, const void* w_down,
                          const void* x_q8, float* h, void* h_q8, const float* r, float* y,
                          float* gu, int hidden_dim, int inter_dim, void* stream);

/* Message for the most recent non-zero return on the calling thread. */
const char* rz_last_error(void);

/* ABI version (major * 100 + minor). */
int rz_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RZ_H */
