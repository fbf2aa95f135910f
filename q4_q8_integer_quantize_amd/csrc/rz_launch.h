// rz_launch.h -- host-side launchers of the librz kernels (internal).
// Arguments are validated by the C ABI (rz_abi.cpp) before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rz {

hipError_t launch_q8_1_quantize(const float* x, int n, int n_padded, int n_tokens,
                                uint8_t* out, hipStream_t stream);

// RMSNorm of [n_tokens][n] fp32 values with weights gamma[n], quantized to
// Q8_1 ([n_tokens][n_padded/32] blocks); normed ([n_tokens][n]) is optional.
hipError_t launch_rmsnorm_q8_1(const float* x, const float* gamma, float eps, int n,
                               int n_padded, int n_tokens, float* normed, uint8_t* x_q8,
                               hipStream_t stream);

// Q4_K x Q8_1 GEMV for 1..8 tokens (token-major y).  With r (token-major,
// like y; may be y) the result is W x + r.
hipError_t launch_q4k_q8_gemv(const uint8_t* w, const uint8_t* xq, float* y, int out_dim,
                              int in_dim, int n_tokens, hipStream_t stream,
                              const float* r = nullptr);

// The same for a batch of tokens on the matrix cores (used by
// launch_q4k_q8_gemv from kMfmaMinTokens tokens on).
hipError_t launch_q4k_q8_gemm_mfma(const uint8_t* w, const uint8_t* xq, float* y, int out_dim,
                                   int in_dim, int n_tokens, hipStream_t stream,
                                   const float* r = nullptr);
constexpr int kMfmaMinTokens = 3;

// Several Q4_K matrices (at most kMaxMats) times one Q8_1 activation; one
// launch for 1..2 tokens and in_dim <= kMultiMaxInDim, else one call per matrix.
constexpr int kMaxMats = 8;
constexpr int kMultiMaxInDim = 16384;
hipError_t launch_q4k_q8_gemv_multi(int n_mats, const uint8_t* const* w, float* const* y,
                                    const int* out_dims, const uint8_t* xq, int in_dim,
                                    int n_tokens, hipStream_t stream);

// The same for one fp32 token row x[n] (zero-padded to in_dim <= kMultiMaxInDim):
// every workgroup RMSNorms it with gamma[n] and quantizes it into LDS
// (bit-identical to launch_rmsnorm_q8_1 followed by launch_q4k_q8_gemv_multi);
// workgroup 0 writes the Q8_1 blocks to xq_out when it is not null.
hipError_t launch_rmsnorm_q4k_q8_gemv_multi(int n_mats, const uint8_t* const* w, float* const* y,
                                            const int* out_dims, const float* x,
                                            const float* gamma, float eps, int n,
                                            uint8_t* xq_out, int in_dim, hipStream_t stream);

// The k largest of v[n] (largest first, equal values by index) into out_i /
// out_v (either may be null), through cand_key / cand_idx of topk_slices(n) * k
// entries each, at most kTopkMerge; 1 <= k <= min(n, kTopkMaxK).
constexpr int kTopkSlice = 2048;    // values one slice workgroup selects from
constexpr int kTopkMerge = 16384;   // candidates the merge workgroup selects from
constexpr int kTopkMaxK = 128;
long topk_slices(int n);
hipError_t launch_topk_f32(const float* v, int n, int k, int* out_i, float* out_v,
                           unsigned* cand_key, int* cand_idx, hipStream_t stream);

// Q8_1 quantize of an fp32 activation fused into the Q4_K GEMV (1 token); with
// r, y = W Q8_1(x) + r (r may be y).
hipError_t launch_q4k_q8_gemv_f32(const uint8_t* w, const float* x, int n, uint8_t* xq_out,
                                  float* y, int out_dim, int in_dim, hipStream_t stream,
                                  const float* r = nullptr);

// Q4_K times an fp32 activation without Q8_1 (1 token), and the SwiGLU FFN on
// that path (gate/up with silu*up into h, then the down GEMV over fp32 h).
hipError_t launch_q4k_gemv_xf32(const uint8_t* w, const float* x, int n, float* y, int out_dim,
                                int in_dim, hipStream_t stream);
hipError_t launch_swiglu_ffn_q4k_xf32(const uint8_t* w_gate, const uint8_t* w_up,
                                      const uint8_t* w_down, const float* x, float* h, float* y,
                                      float* gu, int hidden_dim, int inter_dim,
                                      hipStream_t stream);

hipError_t launch_q4_0_gemv(const uint8_t* w, const void* x, int x_format, float* y,
                            int out_dim, int in_dim, hipStream_t stream);

// The LM head: Q4_0 GEMV with the output bias added in the store and,
// when argmax_idx or argmax_val is given, the greedy token (per-workgroup
// pairs in part_val/part_idx, q4_0_lm_head_partials of each, then one merge).
long q4_0_lm_head_partials(int out_dim, int in_dim, int x_format);

// GELU FFN on Q4_0 weights and fp32 activations, optional biases.
hipError_t launch_gelu_ffn_q4_0(const uint8_t* w_up, const uint8_t* w_down, const float* x,
                                const float* up_bias, const float* down_bias, float* h, float* y,
                                int hidden_dim, int inter_dim, hipStream_t stream);
hipError_t launch_q4_0_lm_head(const uint8_t* w, const void* x, int x_format, const float* bias,
                               float* logits, int out_dim, int in_dim, int* argmax_idx,
                               float* argmax_val, float* part_val, int* part_idx,
                               hipStream_t stream);

// SwiGLU FFN chain; with r the down projection's output is y = W_down h + r.
hipError_t launch_swiglu_ffn_q4k(const uint8_t* w_gate, const uint8_t* w_up,
                                 const uint8_t* w_down, const uint8_t* xq, float* h,
                                 uint8_t* h_q8, float* y, float* gu, int hidden_dim,
                                 int inter_dim, hipStream_t stream, const float* r = nullptr);

// The pre-norm FFN block on one token: y = x + SwiGLU chain of
// Q8_1(RMSNorm(x, gamma, eps)), the RMSNorm and quantize in every gate/up
// workgroup (bit-identical to launch_rmsnorm_q8_1 followed by
// launch_swiglu_ffn_q4k with r = x); y may be x.
hipError_t launch_rmsnorm_swiglu_ffn_q4k(const uint8_t* w_gate, const uint8_t* w_up,
                                         const uint8_t* w_down, const float* x,
                                         const float* gamma, float eps, float* h,
                                         uint8_t* h_q8, float* y, float* gu, int hidden_dim,
                                         int inter_dim, hipStream_t stream);

}  // namespace rz
