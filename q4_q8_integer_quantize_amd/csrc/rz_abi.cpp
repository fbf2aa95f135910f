// rz_abi.cpp -- the extern "C" boundary of librz.so (declared in include/rz.h).
//
// Every entry point validates its arguments on the host first and returns a
// negative code with a message before touching the HIP runtime, so the checks
// run on machines without a GPU.  Kernels are only enqueued on the caller's
// stream; nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <mutex>

#include "rz.h"
#include "rz_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

// Weight matrices are addressed with 32-bit offsets (raw buffer loads).
constexpr long long kMaxMatrixBytes = (1LL << 31) - 1;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return RZ_OK;
  return fail(RZ_ELAUNCH, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
}

// Byte ranges [a, a + na) and [b, b + nb) do not overlap.
bool disjoint(const void* a, long long na, const void* b, long long nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa + static_cast<uintptr_t>(na) <= pb || pb + static_cast<uintptr_t>(nb) <= pa;
}

// Two fp32 arrays of `count` values either coincide or do not overlap.
bool same_or_disjoint(const float* a, const float* b, long long count) {
  return a == b || disjoint(a, count * 4, b, count * 4);
}

// A buffer and its byte length, for the overlap checks below.
struct Span {
  const void* p;
  long long n;
};

// An output span overlaps none of `others` (null pointers are skipped).
bool clear_of(Span out, std::initializer_list<Span> others) {
  if (!out.p) return true;
  for (const Span& o : others)
    if (o.p && !disjoint(out.p, out.n, o.p, o.n)) return false;
  return true;
}

long long q4k_bytes(int out_dim, int in_dim) { return (long long)out_dim * (in_dim / 256) * RZ_Q4K_BLOCK_BYTES; }
long long q4_0_bytes(int out_dim, int in_dim) { return (long long)out_dim * (in_dim / 32) * RZ_Q4_0_BLOCK_BYTES; }
long long q8_bytes(int n_tokens, int n_padded) { return (long long)n_tokens * (n_padded / 32) * RZ_Q8_1_BLOCK_BYTES; }

int check_dim(const char* what, const char* name, int v, int multiple) {
  if (v <= 0 || v > RZ_MAX_DIM || v % multiple != 0)
    return fail(RZ_EDIM, "%s: %s=%d must be a positive multiple of %d and <= %d", what, name, v,
                multiple, RZ_MAX_DIM);
  return RZ_OK;
}

}  // namespace

extern "C" {

const char* rz_last_error(void) { return g_err; }

int rz_abi_version(void) { return 100; }

int rz_q8_1_quantize(const float* x, int n, int n_padded, int n_tokens, void* x_q8,
                     void* stream) {
  const char* what = "rz_q8_1_quantize";
  if (!x || !x_q8) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (n_tokens < 1 || n_tokens > RZ_MAX_TOKENS)
    return fail(RZ_EINVAL, "%s: n_tokens=%d outside 1..%d", what, n_tokens, RZ_MAX_TOKENS);
  if (int rc = check_dim(what, "n_padded", n_padded, 32)) return rc;
  if (n <= 0 || n > n_padded)
    return fail(RZ_EDIM, "%s: n=%d must satisfy 1 <= n <= n_padded=%d", what, n, n_padded);
  if (!aligned(x, 4)) return fail(RZ_EALIGN, "%s: x must be 4-byte aligned", what);
  if (!aligned(x_q8, 16)) return fail(RZ_EALIGN, "%s: x_q8 must be 16-byte aligned", what);
  if (!clear_of({x_q8, q8_bytes(n_tokens, n_padded)}, {{x, 4LL * n_tokens * n}}))
    return fail(RZ_EINVAL, "%s: x_q8 must not overlap x", what);
  return launch_status(rz::launch_q8_1_quantize(x, n, n_padded, n_tokens,
                                                static_cast<uint8_t*>(x_q8),
                                                static_cast<hipStream_t>(stream)),
                       what);
}

int rz_rmsnorm_q8_1(const float* x, const float* gamma, float eps, int n, int n_padded,
                    int n_tokens, float* normed, void* x_q8, void* stream) {
  const char* what = "rz_rmsnorm_q8_1";
  if (!x || !gamma || !x_q8) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (n_tokens < 1 || n_tokens > RZ_MAX_TOKENS)
    return fail(RZ_EINVAL, "%s: n_tokens=%d outside 1..%d", what, n_tokens, RZ_MAX_TOKENS);
  if (!(eps > 0.0f) || !(eps <= 3.0e38f))
    return fail(RZ_EINVAL, "%s: eps=%g must be positive and finite", what, (double)eps);
  if (int rc = check_dim(what, "n_padded", n_padded, 32)) return rc;
  if (n <= 0 || n > n_padded)
    return fail(RZ_EDIM, "%s: n=%d must satisfy 1 <= n <= n_padded=%d", what, n, n_padded);
  if (!aligned(x, 4) || !aligned(gamma, 4) || (normed && !aligned(normed, 4)))
    return fail(RZ_EALIGN, "%s: fp32 buffers must be 4-byte aligned", what);
  if (!aligned(x_q8, 16)) return fail(RZ_EALIGN, "%s: x_q8 must be 16-byte aligned", what);
  // every workgroup reads the whole row while others write their slices
  const Span xs{x, 4LL * n_tokens * n}, gs{gamma, 4LL * n}, qs{x_q8, q8_bytes(n_tokens, n_padded)};
  if (!clear_of(qs, {xs, gs}) || !clear_of({normed, 4LL * n_tokens * n}, {xs, gs, qs}))
    return fail(RZ_EINVAL, "%s: normed and x_q8 must not overlap x, gamma or each other", what);
  return launch_status(rz::launch_rmsnorm_q8_1(x, gamma, eps, n, n_padded, n_tokens, normed,
                                               static_cast<uint8_t*>(x_q8),
                                               static_cast<hipStream_t>(stream)),
                       what);
}

int rz_q4k_q8_gemv(const void* w_q4k, const void* x_q8, float* y, int out_dim, int in_dim,
                   int n_tokens, void* stream) {
  const char* what = "rz_q4k_q8_gemv";
  if (!w_q4k || !x_q8 || !y) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (n_tokens < 1 || n_tokens > RZ_MAX_TOKENS)
    return fail(RZ_EINVAL, "%s: n_tokens=%d outside 1..%d", what, n_tokens, RZ_MAX_TOKENS);
  if (int rc = check_dim(what, "out_dim", out_dim, 1)) return rc;
  if (int rc = check_dim(what, "in_dim", in_dim, 256)) return rc;
  if ((long long)out_dim * (in_dim / 256) * RZ_Q4K_BLOCK_BYTES > kMaxMatrixBytes)
    return fail(RZ_EDIM, "%s: weight matrix larger than %lld bytes", what, kMaxMatrixBytes);
  if (!aligned(w_q4k, 16)) return fail(RZ_EALIGN, "%s: w_q4k must be 16-byte aligned", what);
  if (!aligned(x_q8, 16)) return fail(RZ_EALIGN, "%s: x_q8 must be 16-byte aligned", what);
  if (!aligned(y, 4)) return fail(RZ_EALIGN, "%s: y must be 4-byte aligned", what);
  if (!clear_of({y, 4LL * n_tokens * out_dim},
                {{w_q4k, q4k_bytes(out_dim, in_dim)}, {x_q8, q8_bytes(n_tokens, in_dim)}}))
    return fail(RZ_EINVAL, "%s: y must not overlap w_q4k or x_q8", what);
  return launch_status(rz::launch_q4k_q8_gemv(static_cast<const uint8_t*>(w_q4k),
                                               static_cast<const uint8_t*>(x_q8), y, out_dim,
                                               in_dim, n_tokens,
                                               static_cast<hipStream_t>(stream)),
                       what);
}

int rz_q4k_q8_gemv_add(const void* w_q4k, const void* x_q8, const float* r, float* y,
                       int out_dim, int in_dim, int n_tokens, void* stream) {
  const char* what = "rz_q4k_q8_gemv_add";
  if (!w_q4k || !x_q8 || !r || !y) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (n_tokens < 1 || n_tokens > RZ_MAX_TOKENS)
    return fail(RZ_EINVAL, "%s: n_tokens=%d outside 1..%d", what, n_tokens, RZ_MAX_TOKENS);
  if (int rc = check_dim(what, "out_dim", out_dim, 1)) return rc;
  if (int rc = check_dim(what, "in_dim", in_dim, 256)) return rc;
  if ((long long)out_dim * (in_dim / 256) * RZ_Q4K_BLOCK_BYTES > kMaxMatrixBytes)
    return fail(RZ_EDIM, "%s: weight matrix larger than %lld bytes", what, kMaxMatrixBytes);
  if (!aligned(w_q4k, 16)) return fail(RZ_EALIGN, "%s: w_q4k must be 16-byte aligned", what);
  if (!aligned(x_q8, 16)) return fail(RZ_EALIGN, "%s: x_q8 must be 16-byte aligned", what);
  if (!aligned(r, 4) || !aligned(y, 4))
    return fail(RZ_EALIGN, "%s: r and y must be 4-byte aligned", what);
  if (!same_or_disjoint(r, y, (long long)n_tokens * out_dim))
    return fail(RZ_EINVAL, "%s: r must be y itself or not overlap it", what);
  if (!clear_of({y, 4LL * n_tokens * out_dim},
                {{w_q4k, q4k_bytes(out_dim, in_dim)}, {x_q8, q8_bytes(n_tokens, in_dim)}}))
    return fail(RZ_EINVAL, "%s: y must not overlap w_q4k or x_q8", what);
  return launch_status(rz::launch_q4k_q8_gemv(static_cast<const uint8_t*>(w_q4k),
                                               static_cast<const uint8_t*>(x_q8), y, out_dim,
                                               in_dim, n_tokens,
                                               static_cast<hipStream_t>(stream), r),
                       what);
}

int rz_q4k_q8_gemv_multi(int n_mats, const void* const* w_q4k, float* const* y,
                         const int* out_dims, const void* x_q8, int in_dim, int n_tokens,
                         void* stream) {
  const char* what = "rz_q4k_q8_gemv_multi";
  if (!w_q4k || !y || !out_dims || !x_q8) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (n_mats < 1 || n_mats > RZ_MAX_MATS)
    return fail(RZ_EINVAL, "%s: n_mats=%d outside 1..%d", what, n_mats, RZ_MAX_MATS);
  if (n_tokens < 1 || n_tokens > RZ_MAX_TOKENS)
    return fail(RZ_EINVAL, "%s: n_tokens=%d outside 1..%d", what, n_tokens, RZ_MAX_TOKENS);
  if (int rc = check_dim(what, "in_dim", in_dim, 256)) return rc;
  if (!aligned(x_q8, 16)) return fail(RZ_EALIGN, "%s: x_q8 must be 16-byte aligned", what);
  const uint8_t* w[RZ_MAX_MATS];
  float* yy[RZ_MAX_MATS];
  int od[RZ_MAX_MATS];
  for (int m = 0; m < n_mats; ++m) {
    if (!w_q4k[m] || !y[m]) return fail(RZ_EINVAL, "%s: null pointer in matrix %d", what, m);
    if (int rc = check_dim(what, "out_dims[m]", out_dims[m], 1)) return rc;
    if ((long long)out_dims[m] * (in_dim / 256) * RZ_Q4K_BLOCK_BYTES > kMaxMatrixBytes)
      return fail(RZ_EDIM, "%s: matrix %d larger than %lld bytes", what, m, kMaxMatrixBytes);
    if (!aligned(w_q4k[m], 16))
      return fail(RZ_EALIGN, "%s: w_q4k[%d] must be 16-byte aligned", what, m);
    if (!aligned(y[m], 4)) return fail(RZ_EALIGN, "%s: y[%d] must be 4-byte aligned", what, m);
    w[m] = static_cast<const uint8_t*>(w_q4k[m]);
    yy[m] = y[m];
    od[m] = out_dims[m];
  }
  // each output clear of the activation, every weight blob and the other outputs
  for (int m = 0; m < n_mats; ++m) {
    const Span ym{yy[m], 4LL * n_tokens * od[m]};
    if (!clear_of(ym, {{x_q8, q8_bytes(n_tokens, in_dim)}}))
      return fail(RZ_EINVAL, "%s: y[%d] must not overlap x_q8", what, m);
    for (int k = 0; k < n_mats; ++k) {
      if (!clear_of(ym, {{w[k], q4k_bytes(od[k], in_dim)}}) ||
          (k != m && !clear_of(ym, {{yy[k], 4LL * n_tokens * od[k]}})))
        return fail(RZ_EINVAL, "%s: y[%d] overlaps a weight blob or another output", what, m);
    }
  }
  return launch_status(rz::launch_q4k_q8_gemv_multi(n_mats, w, yy, od,
                                                     static_cast<const uint8_t*>(x_q8), in_dim,
                                                     n_tokens, static_cast<hipStream_t>(stream)),
                       what);
}

int rz_rmsnorm_q4k_q8_gemv_multi(int n_mats, const void* const* w_q4k, float* const* y,
                                 const int* out_dims, const float* x, const float* gamma,
                                 float eps, int n, void* x_q8, int in_dim, void* stream) {
  const char* what = "rz_rmsnorm_q4k_q8_gemv_multi";
  if (!w_q4k || !y || !out_dims || !x || !gamma) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (n_mats < 1 || n_mats > RZ_MAX_MATS)
    return fail(RZ_EINVAL, "%s: n_mats=%d outside 1..%d", what, n_mats, RZ_MAX_MATS);
  if (!(eps > 0.0f) || !(eps <= 3.0e38f))
    return fail(RZ_EINVAL, "%s: eps=%g must be positive and finite", what, (double)eps);
  if (int rc = check_dim(what, "in_dim", in_dim, 256)) return rc;
  if (in_dim > 16384)
    return fail(RZ_EDIM, "%s: in_dim=%d above the fused limit 16384", what, in_dim);
  if (n <= 0 || n > in_dim)
    return fail(RZ_EDIM, "%s: n=%d must satisfy 1 <= n <= in_dim=%d", what, n, in_dim);
  if (!aligned(x, 4) || !aligned(gamma, 4))
    return fail(RZ_EALIGN, "%s: x and gamma must be 4-byte aligned", what);
  if (x_q8 && !aligned(x_q8, 16)) return fail(RZ_EALIGN, "%s: x_q8 must be 16-byte aligned", what);
  const uint8_t* w[RZ_MAX_MATS];
  float* yy[RZ_MAX_MATS];
  int od[RZ_MAX_MATS];
  for (int m = 0; m < n_mats; ++m) {
    if (!w_q4k[m] || !y[m]) return fail(RZ_EINVAL, "%s: null pointer in matrix %d", what, m);
    if (int rc = check_dim(what, "out_dims[m]", out_dims[m], 1)) return rc;
    if (q4k_bytes(out_dims[m], in_dim) > kMaxMatrixBytes)
      return fail(RZ_EDIM, "%s: matrix %d larger than %lld bytes", what, m, kMaxMatrixBytes);
    if (!aligned(w_q4k[m], 16))
      return fail(RZ_EALIGN, "%s: w_q4k[%d] must be 16-byte aligned", what, m);
    if (!aligned(y[m], 4)) return fail(RZ_EALIGN, "%s: y[%d] must be 4-byte aligned", what, m);
    w[m] = static_cast<const uint8_t*>(w_q4k[m]);
    yy[m] = y[m];
    od[m] = out_dims[m];
  }
  const Span xs{x, 4LL * n}, gs{gamma, 4LL * n}, qs{x_q8, q8_bytes(1, in_dim)};
  for (int m = 0; m < n_mats; ++m) {
    const Span ym{yy[m], 4LL * od[m]};
    if (!clear_of(ym, {xs, gs, qs}))
      return fail(RZ_EINVAL, "%s: y[%d] must not overlap x, gamma or x_q8", what, m);
    for (int k = 0; k < n_mats; ++k)
      if (!clear_of(ym, {{w[k], q4k_bytes(od[k], in_dim)}}) ||
          (k != m && !clear_of(ym, {{yy[k], 4LL * od[k]}})))
        return fail(RZ_EINVAL, "%s: y[%d] overlaps a weight blob or another output", what, m);
  }
  if (!clear_of(qs, {xs, gs}))
    return fail(RZ_EINVAL, "%s: x_q8 must not overlap x or gamma", what);
  for (int k = 0; k < n_mats; ++k)
    if (!clear_of(qs, {{w[k], q4k_bytes(od[k], in_dim)}}))
      return fail(RZ_EINVAL, "%s: x_q8 must not overlap a weight blob", what);
  return launch_status(rz::launch_rmsnorm_q4k_q8_gemv_multi(n_mats, w, yy, od, x, gamma, eps, n,
                                                             static_cast<uint8_t*>(x_q8), in_dim,
                                                             static_cast<hipStream_t>(stream)),
                       what);
}

int rz_q4k_q8_gemv_f32(const void* w_q4k, const float* x, int n, void* x_q8, float* y,
                       int out_dim, int in_dim, void* stream) {
  const char* what = "rz_q4k_q8_gemv_f32";
  if (!w_q4k || !x || !y) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (int rc = check_dim(what, "out_dim", out_dim, 1)) return rc;
  if (int rc = check_dim(what, "in_dim", in_dim, 256)) return rc;
  if (in_dim > 16384)
    return fail(RZ_EDIM, "%s: in_dim=%d above the fused limit 16384", what, in_dim);
  if (n <= 0 || n > in_dim)
    return fail(RZ_EDIM, "%s: n=%d must satisfy 1 <= n <= in_dim=%d", what, n, in_dim);
  if ((long long)out_dim * (in_dim / 256) * RZ_Q4K_BLOCK_BYTES > kMaxMatrixBytes)
    return fail(RZ_EDIM, "%s: weight matrix larger than %lld bytes", what, kMaxMatrixBytes);
  if (!aligned(w_q4k, 16)) return fail(RZ_EALIGN, "%s: w_q4k must be 16-byte aligned", what);
  if (!aligned(x, 4) || !aligned(y, 4))
    return fail(RZ_EALIGN, "%s: x and y must be 4-byte aligned", what);
  if (x_q8 && !aligned(x_q8, 16)) return fail(RZ_EALIGN, "%s: x_q8 must be 16-byte aligned", what);
  {
    const Span ws{w_q4k, q4k_bytes(out_dim, in_dim)}, xs{x, 4LL * n}, qs{x_q8, q8_bytes(1, in_dim)};
    if (!clear_of({y, 4LL * out_dim}, {ws, xs, qs}) || !clear_of(qs, {ws, xs}))
      return fail(RZ_EINVAL, "%s: y and x_q8 must not overlap w_q4k, x or each other", what);
  }
  return launch_status(rz::launch_q4k_q8_gemv_f32(static_cast<const uint8_t*>(w_q4k), x, n,
                                                   static_cast<uint8_t*>(x_q8), y, out_dim,
                                                   in_dim, static_cast<hipStream_t>(stream)),
                       what);
}

int rz_q4k_q8_gemv_f32_add(const void* w_q4k, const float* x, int n, void* x_q8, const float* r,
                           float* y, int out_dim, int in_dim, void* stream) {
  const char* what = "rz_q4k_q8_gemv_f32_add";
  if (!w_q4k || !x || !r || !y) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (int rc = check_dim(what, "out_dim", out_dim, 1)) return rc;
  if (int rc = check_dim(what, "in_dim", in_dim, 256)) return rc;
  if (in_dim > 16384)
    return fail(RZ_EDIM, "%s: in_dim=%d above the fused limit 16384", what, in_dim);
  if (n <= 0 || n > in_dim)
    return fail(RZ_EDIM, "%s: n=%d must satisfy 1 <= n <= in_dim=%d", what, n, in_dim);
  if ((long long)out_dim * (in_dim / 256) * RZ_Q4K_BLOCK_BYTES > kMaxMatrixBytes)
    return fail(RZ_EDIM, "%s: weight matrix larger than %lld bytes", what, kMaxMatrixBytes);
  if (!aligned(w_q4k, 16)) return fail(RZ_EALIGN, "%s: w_q4k must be 16-byte aligned", what);
  if (!aligned(x, 4) || !aligned(r, 4) || !aligned(y, 4))
    return fail(RZ_EALIGN, "%s: x, r and y must be 4-byte aligned", what);
  if (x_q8 && !aligned(x_q8, 16)) return fail(RZ_EALIGN, "%s: x_q8 must be 16-byte aligned", what);
  {
    // every workgroup reads all of x while others store y; r is read by the
    // wave that stores the same rows, so r may be y itself
    const Span ws{w_q4k, q4k_bytes(out_dim, in_dim)}, xs{x, 4LL * n}, qs{x_q8, q8_bytes(1, in_dim)},
        rs{r, 4LL * out_dim}, ys{y, 4LL * out_dim};
    if (!clear_of(ys, {ws, xs, qs}) || !clear_of(qs, {ws, xs, rs}) ||
        !same_or_disjoint(y, r, out_dim))
      return fail(RZ_EINVAL, "%s: y and x_q8 must not overlap w_q4k, x or each other, x_q8 must "
                  "not overlap r, and r must be y itself or not overlap it", what);
  }
  return launch_status(rz::launch_q4k_q8_gemv_f32(static_cast<const uint8_t*>(w_q4k), x, n,
                                                   static_cast<uint8_t*>(x_q8), y, out_dim,
                                                   in_dim, static_cast<hipStream_t>(stream), r),
                       what);
}

int rz_q4k_gemv(const void* w_q4k, const float* x, int n, float* y, int out_dim, int in_dim,
                void* stream) {
  const char* what = "rz_q4k_gemv";
  if (!w_q4k || !x || !y) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (int rc = check_dim(what, "out_dim", out_dim, 1)) return rc;
  if (int rc = check_dim(what, "in_dim", in_dim, 256)) return rc;
  if (n <= 0 || n > in_dim)
    return fail(RZ_EDIM, "%s: n=%d must satisfy 1 <= n <= in_dim=%d", what, n, in_dim);
  if ((long long)out_dim * (in_dim / 256) * RZ_Q4K_BLOCK_BYTES > kMaxMatrixBytes)
    return fail(RZ_EDIM, "%s: weight matrix larger than %lld bytes", what, kMaxMatrixBytes);
  if (!aligned(w_q4k, 16)) return fail(RZ_EALIGN, "%s: w_q4k must be 16-byte aligned", what);
  if (!aligned(x, 4) || !aligned(y, 4))
    return fail(RZ_EALIGN, "%s: x and y must be 4-byte aligned", what);
  if (!clear_of({y, 4LL * out_dim}, {{x, 4LL * n}, {w_q4k, q4k_bytes(out_dim, in_dim)}}))
    return fail(RZ_EINVAL, "%s: y must not overlap x or w_q4k", what);
  return launch_status(rz::launch_q4k_gemv_xf32(static_cast<const uint8_t*>(w_q4k), x, n, y,
                                                out_dim, in_dim, static_cast<hipStream_t>(stream)),
                       what);
}

int rz_swiglu_ffn_q4k_f32(const void* w_gate, const void* w_up, const void* w_down,
                          const float* x, float* h, float* y, float* gu, int hidden_dim,
                          int inter_dim, void* stream) {
  const char* what = "rz_swiglu_ffn_q4k_f32";
  if (!w_gate || !w_up || !w_down || !x || !h || !y)
    return fail(RZ_EINVAL, "%s: null pointer", what);
  if (int rc = check_dim(what, "hidden_dim", hidden_dim, 256)) return rc;
  if (int rc = check_dim(what, "inter_dim", inter_dim, 256)) return rc;
  if ((long long)inter_dim * (hidden_dim / 256) * RZ_Q4K_BLOCK_BYTES > kMaxMatrixBytes)
    return fail(RZ_EDIM, "%s: weight matrix larger than %lld bytes", what, kMaxMatrixBytes);
  if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16))
    return fail(RZ_EALIGN, "%s: weight blobs must be 16-byte aligned", what);
  if (!aligned(x, 4) || !aligned(h, 4) || !aligned(y, 4) || (gu && !aligned(gu, 4)))
    return fail(RZ_EALIGN, "%s: fp32 buffers must be 4-byte aligned", what);
  // x is read by the first kernel while it writes h and gu; h by the second while it writes y
  if (!disjoint(x, 4LL * hidden_dim, h, 4LL * inter_dim) ||
      (gu && (!disjoint(x, 4LL * hidden_dim, gu, 8LL * inter_dim) ||
              !disjoint(h, 4LL * inter_dim, gu, 8LL * inter_dim) ||
              !disjoint(y, 4LL * hidden_dim, gu, 8LL * inter_dim))) ||
      !disjoint(h, 4LL * inter_dim, y, 4LL * hidden_dim))
    return fail(RZ_EINVAL, "%s: x, h, gu and y must not overlap (x and y may)", what);
  {
    const long long wb = q4k_bytes(inter_dim, hidden_dim), db = q4k_bytes(hidden_dim, inter_dim);
    for (Span o : {Span{h, 4LL * inter_dim}, Span{y, 4LL * hidden_dim}, Span{gu, 8LL * inter_dim}})
      if (!clear_of(o, {{w_gate, wb}, {w_up, wb}, {w_down, db}}))
        return fail(RZ_EINVAL, "%s: h, y and gu must not overlap the weight blobs", what);
  }
  return launch_status(
      rz::launch_swiglu_ffn_q4k_xf32(static_cast<const uint8_t*>(w_gate),
                                     static_cast<const uint8_t*>(w_up),
                                     static_cast<const uint8_t*>(w_down), x, h, y, gu, hidden_dim,
                                     inter_dim, static_cast<hipStream_t>(stream)),
      what);
}

int rz_q4_0_gemv(const void* w_q4_0, const void* x, int x_format, float* y, int out_dim,
                 int in_dim, void* stream) {
  const char* what = "rz_q4_0_gemv";
  if (!w_q4_0 || !x || !y) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (x_format != 0 && x_format != 1)
    return fail(RZ_EINVAL, "%s: x_format=%d (0 = fp32, 1 = Q8_1)", what, x_format);
  if (int rc = check_dim(what, "out_dim", out_dim, 1)) return rc;
  if (int rc = check_dim(what, "in_dim", in_dim, 64)) return rc;
  if (!aligned(w_q4_0, 4)) return fail(RZ_EALIGN, "%s: w_q4_0 must be 4-byte aligned", what);
  if (!aligned(x, 16)) return fail(RZ_EALIGN, "%s: x must be 16-byte aligned", what);
  if (!aligned(y, 4)) return fail(RZ_EALIGN, "%s: y must be 4-byte aligned", what);
  if (!clear_of({y, 4LL * out_dim}, {{w_q4_0, q4_0_bytes(out_dim, in_dim)},
                                     {x, x_format == 0 ? 4LL * in_dim : q8_bytes(1, in_dim)}}))
    return fail(RZ_EINVAL, "%s: y must not overlap w_q4_0 or x", what);
  return launch_status(rz::launch_q4_0_gemv(static_cast<const uint8_t*>(w_q4_0), x, x_format, y,
                                            out_dim, in_dim, static_cast<hipStream_t>(stream)),
                       what);
}

}  // extern "C"

namespace {

int swiglu_ffn(const char* what, const void* w_gate, const void* w_up, const void* w_down,
               const void* x_q8, float* h, void* h_q8, const float* r, float* y, float* gu,
               int hidden_dim, int inter_dim, void* stream) {
  if (!w_gate || !w_up || !w_down || !x_q8 || !h || !h_q8 || !y)
    return fail(RZ_EINVAL, "%s: null pointer", what);
  if (int rc = check_dim(what, "hidden_dim", hidden_dim, 256)) return rc;
  if (int rc = check_dim(what, "inter_dim", inter_dim, 256)) return rc;
  if ((long long)inter_dim * (hidden_dim / 256) * RZ_Q4K_BLOCK_BYTES > kMaxMatrixBytes)
    return fail(RZ_EDIM, "%s: weight matrix larger than %lld bytes", what, kMaxMatrixBytes);
  if (hidden_dim > 16384)
    return fail(RZ_EDIM, "%s: hidden_dim=%d above the fused gate/up limit 16384", what,
                hidden_dim);
  if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16))
    return fail(RZ_EALIGN, "%s: weight blobs must be 16-byte aligned", what);
  if (!aligned(x_q8, 16) || !aligned(h_q8, 16))
    return fail(RZ_EALIGN, "%s: Q8_1 buffers must be 16-byte aligned", what);
  if (!aligned(h, 4) || !aligned(y, 4) || (gu && !aligned(gu, 4)) || (r && !aligned(r, 4)))
    return fail(RZ_EALIGN, "%s: fp32 buffers must be 4-byte aligned", what);
  if (r && !same_or_disjoint(r, y, hidden_dim))
    return fail(RZ_EINVAL, "%s: r must be y itself or not overlap it", what);
  {
    // the first kernel reads x_q8 and the gate/up weights while it writes h,
    // h_q8 and gu; the second reads h_q8 and the down weights while it writes y
    const long long wb = q4k_bytes(inter_dim, hidden_dim), db = q4k_bytes(hidden_dim, inter_dim);
    const Span xs{x_q8, q8_bytes(1, hidden_dim)}, hs{h, 4LL * inter_dim},
        hq{h_q8, q8_bytes(1, inter_dim)}, gs{gu, 8LL * inter_dim}, ys{y, 4LL * hidden_dim},
        wg{w_gate, wb}, wu{w_up, wb}, wd{w_down, db};
    if (!clear_of(hs, {xs, hq, gs, ys, wg, wu, wd}) || !clear_of(hq, {xs, gs, ys, wg, wu, wd}) ||
        !clear_of(gs, {xs, ys, wg, wu, wd}) || !clear_of(ys, {wd, wg, wu}))
      return fail(RZ_EINVAL, "%s: h, h_q8, gu and y must not overlap x_q8, the weights or each "
                  "other (y may overlap x_q8)", what);
  }
  // the first kernel writes h, h_q8 and gu before the second reads r
  if (r && (!disjoint(r, 4LL * hidden_dim, h, 4LL * inter_dim) ||
            !disjoint(r, 4LL * hidden_dim, h_q8, (long long)inter_dim / 32 * RZ_Q8_1_BLOCK_BYTES) ||
            (gu && !disjoint(r, 4LL * hidden_dim, gu, 8LL * inter_dim))))
    return fail(RZ_EINVAL, "%s: r must not overlap h, h_q8 or gu", what);
  return launch_status(
      rz::launch_swiglu_ffn_q4k(static_cast<const uint8_t*>(w_gate),
                                static_cast<const uint8_t*>(w_up),
                                static_cast<const uint8_t*>(w_down),
                                static_cast<const uint8_t*>(x_q8), h,
                                static_cast<uint8_t*>(h_q8), y, gu, hidden_dim, inter_dim,
                                static_cast<hipStream_t>(stream), r),
      what);
}

// Argument checks shared by the two LM-head entry points (everything but the
// argmax workspace).
int lm_head_check(const char* what, const void* w_q4_0, const void* x, int x_format,
                  const float* bias, const float* logits, int out_dim, int in_dim,
                  const int* argmax_idx, const float* argmax_val) {
  if (!w_q4_0 || !x || !logits) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (x_format != 0 && x_format != 1)
    return fail(RZ_EINVAL, "%s: x_format=%d (0 = fp32, 1 = Q8_1)", what, x_format);
  if (int rc = check_dim(what, "out_dim", out_dim, 1)) return rc;
  if (int rc = check_dim(what, "in_dim", in_dim, 64)) return rc;
  if (!aligned(w_q4_0, 4)) return fail(RZ_EALIGN, "%s: w_q4_0 must be 4-byte aligned", what);
  if (!aligned(x, 16)) return fail(RZ_EALIGN, "%s: x must be 16-byte aligned", what);
  if (!aligned(logits, 4) || (bias && !aligned(bias, 4)) || (argmax_idx && !aligned(argmax_idx, 4)) ||
      (argmax_val && !aligned(argmax_val, 4)))
    return fail(RZ_EALIGN, "%s: logits, bias and the argmax outputs must be 4-byte aligned", what);
  if (bias && !same_or_disjoint(bias, logits, out_dim))
    return fail(RZ_EINVAL, "%s: bias must be logits itself or not overlap it", what);
  const Span wspan{w_q4_0, q4_0_bytes(out_dim, in_dim)},
      xspan{x, x_format == 0 ? 4LL * in_dim : q8_bytes(1, in_dim)};
  if (!clear_of({logits, 4LL * out_dim}, {wspan, xspan}))
    return fail(RZ_EINVAL, "%s: logits must not overlap w_q4_0 or x", what);
  if (!clear_of({argmax_idx, 4}, {wspan, xspan, {logits, 4LL * out_dim}, {argmax_val, 4}}) ||
      !clear_of({argmax_val, 4}, {wspan, xspan, {logits, 4LL * out_dim}}))
    return fail(RZ_EINVAL, "%s: the argmax outputs must not overlap w_q4_0, x, logits or "
                "each other", what);
  return RZ_OK;
}

}  // namespace

// ----------------------------------------------------------------- no-alloc LM head
// The argmax pairs of rz_lm_head_q4_0_noalloc: (value, row) for at most
// kNoAllocPairs workgroups, values first, rows after them (256 KiB).  Every
// GPU the library runs on holds its own copy for the life of the process.  In
// host code the array's name is a host-side stand-in, not a device address:
// kernels only ever get the address hipGetSymbolAddress returns for the
// current device (kept in g_scratch_ptr).
constexpr size_t kNoAllocPairs = RZ_NOALLOC_ARGMAX_PAIRS;
static __device__ __align__(256) unsigned char scratch[kNoAllocPairs * 8];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device, taken once with that device current

// The current device's copy of `scratch` (looked up on the first call on the
// device), after checking that `stream` belongs to that device.
int scratch_for_current_device(const char* what, hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(RZ_ELAUNCH, "%s: hipGetDevice failed: %s", what, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RZ_EINVAL, "%s: device %d, this library tracks devices 0..%d", what, dev,
                kMaxDevices - 1);
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess)
      return fail(RZ_ELAUNCH, "%s: hipStreamGetDevice failed: %s", what, hipGetErrorString(e));
    if (sdev != dev)
      return fail(RZ_EINVAL, "%s: the stream belongs to device %d, the current device is %d", what,
                  sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(RZ_ELAUNCH, "%s: hipGetSymbolAddress of the scratch array failed: %s", what,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RZ_OK;
}

}  // namespace

extern "C" {

size_t rz_lm_head_q4_0_workspace_bytes(int out_dim, int in_dim, int x_format) {
  if (out_dim <= 0 || out_dim > RZ_MAX_DIM || in_dim <= 0 || in_dim > RZ_MAX_DIM ||
      in_dim % 64 != 0 || (x_format != 0 && x_format != 1))
    return 0;
  return (size_t)rz::q4_0_lm_head_partials(out_dim, in_dim, x_format) * 8u;
}

int rz_lm_head_q4_0(const void* w_q4_0, const void* x, int x_format, const float* bias,
                    float* logits, int out_dim, int in_dim, int* argmax_idx, float* argmax_val,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const char* what = "rz_lm_head_q4_0";
  if (int rc = lm_head_check(what, w_q4_0, x, x_format, bias, logits, out_dim, in_dim, argmax_idx,
                             argmax_val))
    return rc;
  const Span wspan{w_q4_0, q4_0_bytes(out_dim, in_dim)},
      xspan{x, x_format == 0 ? 4LL * in_dim : q8_bytes(1, in_dim)};
  const bool argmax = argmax_idx || argmax_val;
  float* part_val = nullptr;
  int* part_idx = nullptr;
  if (argmax) {
    const size_t need = rz_lm_head_q4_0_workspace_bytes(out_dim, in_dim, x_format);
    if (!workspace) return fail(RZ_EINVAL, "%s: the argmax needs a workspace", what);
    if (!aligned(workspace, 4)) return fail(RZ_EALIGN, "%s: workspace must be 4-byte aligned", what);
    if (workspace_bytes < need)
      return fail(RZ_EINVAL, "%s: workspace of %zu bytes, %zu needed", what, workspace_bytes, need);
    if (!clear_of({workspace, (long long)need}, {{logits, 4LL * out_dim}, {bias, 4LL * out_dim},
                                                  wspan, xspan}))
      return fail(RZ_EINVAL, "%s: workspace must not overlap logits, bias, w_q4_0 or x", what);
    if ((argmax_idx && !disjoint(argmax_idx, 4, workspace, (long long)need)) ||
        (argmax_val && !disjoint(argmax_val, 4, workspace, (long long)need)))
      return fail(RZ_EINVAL, "%s: the argmax outputs must not overlap the workspace", what);
    part_val = static_cast<float*>(workspace);
    part_idx = reinterpret_cast<int*>(static_cast<char*>(workspace) + need / 2);
  }
  return launch_status(rz::launch_q4_0_lm_head(static_cast<const uint8_t*>(w_q4_0), x, x_format,
                                               bias, logits, out_dim, in_dim, argmax_idx,
                                               argmax_val, part_val, part_idx,
                                               static_cast<hipStream_t>(stream)),
                       what);
}

int rz_lm_head_q4_0_noalloc(const void* w_q4_0, const void* x, int x_format, const float* bias,
                            float* logits, int out_dim, int in_dim, int* argmax_idx,
                            float* argmax_val, void* stream) {
  const char* what = "rz_lm_head_q4_0_noalloc";
  if (int rc = lm_head_check(what, w_q4_0, x, x_format, bias, logits, out_dim, in_dim, argmax_idx,
                             argmax_val))
    return rc;
  float* part_val = nullptr;
  int* part_idx = nullptr;
  if (argmax_idx || argmax_val) {
    const long pairs = rz::q4_0_lm_head_partials(out_dim, in_dim, x_format);
    if (pairs > (long)kNoAllocPairs)
      return fail(RZ_EINVAL,
                  "%s: the argmax needs %ld (value, row) pairs, the fixed scratch holds %zu "
                  "(%zu bytes); use rz_lm_head_q4_0 with a workspace",
                  what, pairs, kNoAllocPairs, kNoAllocPairs * 8);
    void* sp = nullptr;
    if (int rc = scratch_for_current_device(what, static_cast<hipStream_t>(stream), &sp)) return rc;
    part_val = static_cast<float*>(sp);
    part_idx = reinterpret_cast<int*>(static_cast<char*>(sp) + kNoAllocPairs * 4);
  }
  return launch_status(rz::launch_q4_0_lm_head(static_cast<const uint8_t*>(w_q4_0), x, x_format,
                                               bias, logits, out_dim, in_dim, argmax_idx,
                                               argmax_val, part_val, part_idx,
                                               static_cast<hipStream_t>(stream)),
                       what);
}

// ----------------------------------------------------------------- top-k
namespace {

static_assert(rz::kTopkMaxK == RZ_TOPK_MAX, "top-k limit");

// Candidates the top-k of n values keeps (slices x k), or -1 for arguments
// rz_topk_f32 rejects.
long topk_candidates(int n, int k) {
  if (n <= 0 || n > RZ_MAX_DIM || k < 1 || k > RZ_TOPK_MAX || k > n) return -1;
  const long m = rz::topk_slices(n) * k;
  return m <= rz::kTopkMerge ? m : -1;
}

// The checks shared by rz_topk_f32 and rz_lm_head_q4_0_topk for the selection
// over values[n] (`others` are the call's other buffers, which the top-k
// outputs and the workspace must not overlap).
int topk_check(const char* what, const float* values, int n, int k, const int* topk_idx,
               const float* topk_val, const void* workspace, size_t workspace_bytes,
               std::initializer_list<Span> others) {
  if (!values || !workspace) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (!topk_idx && !topk_val)
    return fail(RZ_EINVAL, "%s: neither topk_idx nor topk_val is given", what);
  if (k < 1 || k > RZ_TOPK_MAX)
    return fail(RZ_EINVAL, "%s: k=%d must be in 1..%d", what, k, RZ_TOPK_MAX);
  if (k > n) return fail(RZ_EINVAL, "%s: k=%d is more than the %d values", what, k, n);
  const long m = topk_candidates(n, k);
  if (m < 0)
    return fail(RZ_EINVAL, "%s: %d values in %ld slices of %d keep %ld candidates for k=%d, more "
                "than the %d one workgroup merges",
                what, n, rz::topk_slices(n), rz::kTopkSlice, rz::topk_slices(n) * k, k,
                rz::kTopkMerge);
  if (!aligned(values, 4) || !aligned(workspace, 4) || (topk_idx && !aligned(topk_idx, 4)) ||
      (topk_val && !aligned(topk_val, 4)))
    return fail(RZ_EALIGN, "%s: values, workspace and the top-k outputs must be 4-byte aligned",
                what);
  const size_t need = (size_t)m * 8u;
  if (workspace_bytes < need)
    return fail(RZ_EINVAL, "%s: workspace of %zu bytes, %zu needed", what, workspace_bytes, need);
  const Span vspan{values, 4LL * n}, wsp{workspace, (long long)need}, ispan{topk_idx, 4LL * k},
      fspan{topk_val, 4LL * k};
  if (!clear_of(wsp, {vspan}) || !clear_of(wsp, others))
    return fail(RZ_EINVAL, "%s: workspace must not overlap the values or the call's other buffers",
                what);
  if (!clear_of(ispan, {vspan, wsp, fspan}) || !clear_of(fspan, {vspan, wsp}) ||
      !clear_of(ispan, others) || !clear_of(fspan, others))
    return fail(RZ_EINVAL, "%s: the top-k outputs must not overlap the values, the workspace, "
                "each other or the call's other buffers", what);
  return RZ_OK;
}

}  // namespace

size_t rz_topk_f32_workspace_bytes(int n, int k) {
  const long m = topk_candidates(n, k);
  return m < 0 ? 0 : (size_t)m * 8u;
}

int rz_topk_f32(const float* values, int n, int k, int* topk_idx, float* topk_val, void* workspace,
                size_t workspace_bytes, void* stream) {
  const char* what = "rz_topk_f32";
  if (int rc = check_dim(what, "n", n, 1)) return rc;
  if (int rc = topk_check(what, values, n, k, topk_idx, topk_val, workspace, workspace_bytes, {}))
    return rc;
  const long m = topk_candidates(n, k);
  unsigned* cand_key = static_cast<unsigned*>(workspace);
  int* cand_idx = reinterpret_cast<int*>(static_cast<char*>(workspace) + (size_t)m * 4u);
  return launch_status(rz::launch_topk_f32(values, n, k, topk_idx, topk_val, cand_key, cand_idx,
                                           static_cast<hipStream_t>(stream)),
                       what);
}

int rz_lm_head_q4_0_topk(const void* w_q4_0, const void* x, int x_format, const float* bias,
                         float* logits, int out_dim, int in_dim, int k, int* topk_idx,
                         float* topk_val, void* workspace, size_t workspace_bytes, void* stream) {
  const char* what = "rz_lm_head_q4_0_topk";
  if (int rc = lm_head_check(what, w_q4_0, x, x_format, bias, logits, out_dim, in_dim, nullptr,
                             nullptr))
    return rc;
  const Span wspan{w_q4_0, q4_0_bytes(out_dim, in_dim)},
      xspan{x, x_format == 0 ? 4LL * in_dim : q8_bytes(1, in_dim)}, bspan{bias, 4LL * out_dim};
  if (int rc = topk_check(what, logits, out_dim, k, topk_idx, topk_val, workspace, workspace_bytes,
                          {wspan, xspan, bspan}))
    return rc;
  const long m = topk_candidates(out_dim, k);
  unsigned* cand_key = static_cast<unsigned*>(workspace);
  int* cand_idx = reinterpret_cast<int*>(static_cast<char*>(workspace) + (size_t)m * 4u);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = rz::launch_q4_0_lm_head(static_cast<const uint8_t*>(w_q4_0), x, x_format,
                                               bias, logits, out_dim, in_dim, nullptr, nullptr,
                                               nullptr, nullptr, st);
  if (e != hipSuccess) return launch_status(e, what);
  return launch_status(rz::launch_topk_f32(logits, out_dim, k, topk_idx, topk_val, cand_key,
                                           cand_idx, st),
                       what);
}

int rz_gelu_ffn_q4_0(const void* w_up, const void* w_down, const float* x, const float* up_bias,
                     const float* down_bias, float* h, float* y, int hidden_dim, int inter_dim,
                     void* stream) {
  const char* what = "rz_gelu_ffn_q4_0";
  if (!w_up || !w_down || !x || !h || !y) return fail(RZ_EINVAL, "%s: null pointer", what);
  if (int rc = check_dim(what, "hidden_dim", hidden_dim, 64)) return rc;
  if (int rc = check_dim(what, "inter_dim", inter_dim, 64)) return rc;
  if (!aligned(w_up, 4) || !aligned(w_down, 4))
    return fail(RZ_EALIGN, "%s: weight blobs must be 4-byte aligned", what);
  if (!aligned(x, 16) || !aligned(h, 16))
    return fail(RZ_EALIGN, "%s: x and h must be 16-byte aligned", what);
  if (!aligned(y, 4) || (up_bias && !aligned(up_bias, 4)) || (down_bias && !aligned(down_bias, 4)))
    return fail(RZ_EALIGN, "%s: y and the biases must be 4-byte aligned", what);
  // the up projection reads x and up_bias while it writes h; the down
  // projection reads h and down_bias while it writes y
  if (!disjoint(x, 4LL * hidden_dim, h, 4LL * inter_dim) ||
      (up_bias && !same_or_disjoint(up_bias, h, inter_dim)) ||
      !disjoint(h, 4LL * inter_dim, y, 4LL * hidden_dim) ||
      (down_bias && !same_or_disjoint(down_bias, y, hidden_dim)))
    return fail(RZ_EINVAL, "%s: overlapping buffers (x, h; h, y; a bias and its output)", what);
  {
    const long long ub = q4_0_bytes(inter_dim, hidden_dim), db = q4_0_bytes(hidden_dim, inter_dim);
    if (!clear_of({h, 4LL * inter_dim}, {{w_up, ub}, {w_down, db}}) ||
        !clear_of({y, 4LL * hidden_dim}, {{w_up, ub}, {w_down, db}}))
      return fail(RZ_EINVAL, "%s: h and y must not overlap the weight blobs", what);
  }
  return launch_status(rz::launch_gelu_ffn_q4_0(static_cast<const uint8_t*>(w_up),
                                                static_cast<const uint8_t*>(w_down), x, up_bias,
                                                down_bias, h, y, hidden_dim, inter_dim,
                                                static_cast<hipStream_t>(stream)),
                       what);
}

int rz_rmsnorm_swiglu_ffn_q4k_add(const void* w_gate, const void* w_up, const void* w_down,
                                  const float* x, const float* gamma, float eps, float* h,
                                  void* h_q8, float* y, float* gu, int hidden_dim, int inter_dim,
                                  void* stream) {
  const char* what = "rz_rmsnorm_swiglu_ffn_q4k_add";
  if (!w_gate || !w_up || !w_down || !x || !gamma || !h || !h_q8 || !y)
    return fail(RZ_EINVAL, "%s: null pointer", what);
  if (!(eps > 0.0f) || !(eps <= 3.0e38f))
    return fail(RZ_EINVAL, "%s: eps=%g must be positive and finite", what, (double)eps);
  if (int rc = check_dim(what, "hidden_dim", hidden_dim, 256)) return rc;
  if (int rc = check_dim(what, "inter_dim", inter_dim, 256)) return rc;
  if (hidden_dim > 16384)
    return fail(RZ_EDIM, "%s: hidden_dim=%d above the fused gate/up limit 16384", what,
                hidden_dim);
  const long long wb = q4k_bytes(inter_dim, hidden_dim), db = q4k_bytes(hidden_dim, inter_dim);
  if (wb > kMaxMatrixBytes)
    return fail(RZ_EDIM, "%s: weight matrix larger than %lld bytes", what, kMaxMatrixBytes);
  if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16))
    return fail(RZ_EALIGN, "%s: weight blobs must be 16-byte aligned", what);
  if (!aligned(h_q8, 16)) return fail(RZ_EALIGN, "%s: h_q8 must be 16-byte aligned", what);
  if (!aligned(x, 4) || !aligned(gamma, 4) || !aligned(h, 4) || !aligned(y, 4) ||
      (gu && !aligned(gu, 4)))
    return fail(RZ_EALIGN, "%s: fp32 buffers must be 4-byte aligned", what);
  // the first kernel reads x, gamma and the gate/up weights while it writes h,
  // h_q8 and gu; the second reads h_q8, x (the residual) and the down weights
  // while it writes y, which may be x itself
  const Span xs{x, 4LL * hidden_dim}, gs{gamma, 4LL * hidden_dim}, hs{h, 4LL * inter_dim},
      hq{h_q8, q8_bytes(1, inter_dim)}, us{gu, 8LL * inter_dim}, ys{y, 4LL * hidden_dim},
      wg{w_gate, wb}, wu{w_up, wb}, wd{w_down, db};
  if (!clear_of(hs, {xs, gs, hq, us, ys, wg, wu, wd}) ||
      !clear_of(hq, {xs, gs, us, ys, wg, wu, wd}) || !clear_of(us, {xs, gs, ys, wg, wu, wd}) ||
      !clear_of(ys, {gs, wg, wu, wd}) ||
      !same_or_disjoint(y, x, hidden_dim))
    return fail(RZ_EINVAL, "%s: h, h_q8, gu and y must not overlap x, gamma, the weights or each "
                "other (y may be x itself)", what);
  return launch_status(
      rz::launch_rmsnorm_swiglu_ffn_q4k(static_cast<const uint8_t*>(w_gate),
                                        static_cast<const uint8_t*>(w_up),
                                        static_cast<const uint8_t*>(w_down), x, gamma, eps, h,
                                        static_cast<uint8_t*>(h_q8), y, gu, hidden_dim, inter_dim,
                                        static_cast<hipStream_t>(stream)),
      what);
}

int rz_swiglu_ffn_q4k(const void* w_gate, const void* w_up, const void* w_down,
                      const void* x_q8, float* h, void* h_q8, float* y, float* gu,
                      int hidden_dim, int inter_dim, void* stream) {
  return swiglu_ffn("rz_swiglu_ffn_q4k", w_gate, w_up, w_down, x_q8, h, h_q8, nullptr, y, gu,
                    hidden_dim, inter_dim, stream);
}

int rz_swiglu_ffn_q4k_add(const void* w_gate, const void* w_up, const void* w_down,
                          const void* x_q8, float* h, void* h_q8, const float* r, float* y,
                          float* gu, int hidden_dim, int inter_dim, void* stream) {
  if (!r) return fail(RZ_EINVAL, "rz_swiglu_ffn_q4k_add: null pointer");
  return swiglu_ffn("rz_swiglu_ffn_q4k_add", w_gate, w_up, w_down, x_q8, h, h_q8, r, y, gu,
                    hidden_dim, inter_dim, stream);
}

}  // extern "C"
