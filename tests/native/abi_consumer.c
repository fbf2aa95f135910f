/* A plain C program that uses librz.so through include/rz.h and the HIP
 * runtime alone: no Python, no torch.  It shows that the boundary stands on
 * its own and checks a few results that are fixed by hand.
 *
 *   abi_consumer host   error paths only (no HIP call at all)
 *   abi_consumer gpu    the error paths, then on device 0:
 *     - Q8_1 quantize of 200 ones padded to 256 (block rule of the realizar
 *       pages, cached.rs transformer_layer_gpu_true_dp4a step 2; padding of
 *       forward_utils.rs pad_and_upload_input): blocks 0-5 hold d = RN(1/127),
 *       q = 127, s = RN(d * 4064); block 6 holds eight 127s and s = RN(d * 1016);
 *       block 7 is all zero;
 *     - Q4_K x Q8_1 GEMV (steps 3 and 6 of that passage) of three rows built
 *       from one hand-worked super-block (d = 1, dmin = 0.5, sixteen distinct
 *       6-bit scales and mins, every qs byte 0xC3) against Q8_1 blocks with
 *       d = 1, q = 1, s = 32: y = 32 * sum_j (d sc_j q_j - dmin m_j), with
 *       sc = 1 2 3 4 17 34 51 63, m = 5 6 7 8 20 40 60 33 and q_j = 3 (even j)
 *       or 12 (odd j), which gives 43600 (d = 1, dmin = 0.5), 90064 (d = 2)
 *       and 46464 (dmin = 0), exact in fp32;
 *     - top 2 of those three values with a caller-allocated workspace:
 *       indices 1, 2.
 * Prints one line per check and exits 0 when every check passes. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "rz.h"

static int failures = 0;

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    printf("FAIL %s: %s\n", what, hipGetErrorString(e));
    ++failures;
    return 0;
  }
  return 1;
}

static uint32_t bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static void host_checks(void) {
  check(rz_abi_version() >= 1, "rz_abi_version");
  /* in_dim 255 is no multiple of the 256-value super-block: rejected before
   * any HIP call, so placeholder addresses are never touched */
  void* w = (void*)(uintptr_t)0x100000;
  void* xq = (void*)(uintptr_t)0x200000;
  float* y = (float*)(uintptr_t)0x300000;
  check(rz_q4k_q8_gemv(w, xq, y, 3, 255, 1, NULL) == RZ_EDIM, "in_dim 255 gives RZ_EDIM");
  check(rz_last_error() != NULL && rz_last_error()[0] != '\0', "RZ_EDIM sets a message");
  check(rz_q4k_q8_gemv(NULL, xq, y, 3, 256, 1, NULL) == RZ_EINVAL, "null weights give RZ_EINVAL");
  check(rz_q4k_q8_gemv(w, xq, y, 3, 256, 0, NULL) == RZ_EINVAL, "zero tokens give RZ_EINVAL");
  check(rz_q4k_q8_gemv(w, xq, y, 3, 256, RZ_MAX_TOKENS + 1, NULL) == RZ_EINVAL,
        "nine tokens give RZ_EINVAL");
}

/* one 144-byte super-block: fp16 d, fp16 dmin, 12 scale bytes, 128 qs bytes */
static void superblock(uint8_t* b, uint16_t d, uint16_t dmin) {
  static const uint8_t scales[12] = {0x41, 0x82, 0xC3, 0xC4, 0x45, 0x86,
                                     0xC7, 0x88, 0x41, 0x82, 0xC3, 0x1F};
  b[0] = (uint8_t)(d & 0xFF);
  b[1] = (uint8_t)(d >> 8);
  b[2] = (uint8_t)(dmin & 0xFF);
  b[3] = (uint8_t)(dmin >> 8);
  memcpy(b + 4, scales, 12);
  memset(b + 16, 0xC3, 128);
}

static void put_f32(uint8_t* p, float f) { memcpy(p, &f, 4); }

static void gpu_checks(void) {
  enum { IN = 256, NB = IN / 32, ROWS = 3 };
  uint8_t w_h[ROWS * RZ_Q4K_BLOCK_BYTES];
  superblock(w_h + 0 * RZ_Q4K_BLOCK_BYTES, 0x3C00, 0x3800); /* d 1, dmin 0.5 */
  superblock(w_h + 1 * RZ_Q4K_BLOCK_BYTES, 0x4000, 0x3800); /* d 2, dmin 0.5 */
  superblock(w_h + 2 * RZ_Q4K_BLOCK_BYTES, 0x3C00, 0x0000); /* d 1, dmin 0   */

  uint8_t xq_h[NB * RZ_Q8_1_BLOCK_BYTES];
  for (int b = 0; b < NB; ++b) {
    uint8_t* p = xq_h + b * RZ_Q8_1_BLOCK_BYTES;
    put_f32(p, 1.0f);
    put_f32(p + 4, 32.0f);
    memset(p + 8, 1, 32);
  }
  float x_h[IN];
  for (int i = 0; i < IN; ++i) x_h[i] = 1.0f;

  void *w = NULL, *xq = NULL, *xq2 = NULL, *ws = NULL;
  float *x = NULL, *y = NULL, *tv = NULL;
  int* ti = NULL;
  const size_t ws_bytes = rz_topk_f32_workspace_bytes(ROWS, 2);
  if (!hip_ok(hipSetDevice(0), "hipSetDevice") ||
      !hip_ok(hipMalloc(&w, sizeof w_h), "hipMalloc w") ||
      !hip_ok(hipMalloc(&xq, sizeof xq_h), "hipMalloc xq") ||
      !hip_ok(hipMalloc(&xq2, sizeof xq_h), "hipMalloc xq2") ||
      !hip_ok(hipMalloc((void**)&x, sizeof x_h), "hipMalloc x") ||
      !hip_ok(hipMalloc((void**)&y, ROWS * sizeof(float)), "hipMalloc y") ||
      !hip_ok(hipMalloc((void**)&ti, 2 * sizeof(int)), "hipMalloc topk idx") ||
      !hip_ok(hipMalloc((void**)&tv, 2 * sizeof(float)), "hipMalloc topk val") ||
      !hip_ok(hipMalloc(&ws, ws_bytes ? ws_bytes : 1), "hipMalloc workspace"))
    goto done;
  if (!hip_ok(hipMemcpy(w, w_h, sizeof w_h, hipMemcpyHostToDevice), "copy w") ||
      !hip_ok(hipMemcpy(xq, xq_h, sizeof xq_h, hipMemcpyHostToDevice), "copy xq") ||
      !hip_ok(hipMemcpy(x, x_h, sizeof x_h, hipMemcpyHostToDevice), "copy x"))
    goto done;

  /* an output that overlaps the weights is rejected before any launch */
  check(rz_q4k_q8_gemv(w, xq, (float*)w, ROWS, IN, 1, NULL) == RZ_EINVAL,
        "output overlapping the weights gives RZ_EINVAL");

  check(rz_q8_1_quantize(x, 200, IN, 1, xq2, NULL) == RZ_OK, "rz_q8_1_quantize returns RZ_OK");
  check(rz_q4k_q8_gemv(w, xq, y, ROWS, IN, 1, NULL) == RZ_OK, "rz_q4k_q8_gemv returns RZ_OK");
  check(rz_topk_f32(y, ROWS, 2, ti, tv, ws, ws_bytes, NULL) == RZ_OK, "rz_topk_f32 returns RZ_OK");
  if (!hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize")) goto done;

  uint8_t q_h[NB * RZ_Q8_1_BLOCK_BYTES];
  float y_h[ROWS], tv_h[2];
  int ti_h[2];
  if (!hip_ok(hipMemcpy(q_h, xq2, sizeof q_h, hipMemcpyDeviceToHost), "copy back Q8_1") ||
      !hip_ok(hipMemcpy(y_h, y, sizeof y_h, hipMemcpyDeviceToHost), "copy back y") ||
      !hip_ok(hipMemcpy(ti_h, ti, sizeof ti_h, hipMemcpyDeviceToHost), "copy back topk idx") ||
      !hip_ok(hipMemcpy(tv_h, tv, sizeof tv_h, hipMemcpyDeviceToHost), "copy back topk val"))
    goto done;

  {
    const volatile float seven = 127.0f; /* keep the division at run time, in fp32 */
    const float d = 1.0f / seven;
    const float s_full = d * 4064.0f, s_part = d * 1016.0f;
    int q_ok = 1;
    for (int b = 0; b < NB; ++b) {
      const uint8_t* p = q_h + b * RZ_Q8_1_BLOCK_BYTES;
      float db, sb;
      memcpy(&db, p, 4);
      memcpy(&sb, p + 4, 4);
      const int live = b < 6 ? 32 : (b == 6 ? 8 : 0);
      const float want_d = live ? d : 0.0f;
      const float want_s = b < 6 ? s_full : (b == 6 ? s_part : 0.0f);
      q_ok &= bits(db) == bits(want_d) && bits(sb) == bits(want_s);
      for (int i = 0; i < 32; ++i) q_ok &= (int8_t)p[8 + i] == (i < live ? 127 : 0);
    }
    check(q_ok, "Q8_1 bytes of 200 ones padded to 256");
  }
  check(y_h[0] == 43600.0f && y_h[1] == 90064.0f && y_h[2] == 46464.0f,
        "GEMV of the hand-worked super-blocks: 43600 90064 46464");
  printf("     y = %.1f %.1f %.1f\n", y_h[0], y_h[1], y_h[2]);
  check(ti_h[0] == 1 && ti_h[1] == 2 && tv_h[0] == 90064.0f && tv_h[1] == 46464.0f,
        "top 2 of the GEMV output: rows 1, 2");

done:
  hipFree(w);
  hipFree(xq);
  hipFree(xq2);
  hipFree(x);
  hipFree(y);
  hipFree(ti);
  hipFree(tv);
  hipFree(ws);
}

int main(int argc, char** argv) {
  const int gpu = argc > 1 && strcmp(argv[1], "gpu") == 0;
  if (argc < 2 || (!gpu && strcmp(argv[1], "host") != 0)) {
    fprintf(stderr, "usage: %s host|gpu\n", argv[0]);
    return 2;
  }
  host_checks();
  if (gpu) gpu_checks();
  printf("%s: %d failure(s)\n", failures ? "FAILED" : "passed", failures);
  fflush(stdout);
  return failures ? 1 : 0;
}
