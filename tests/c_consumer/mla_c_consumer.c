/*
 * A C99 caller of libmla_decode.so that uses include/mla_decode.h alone: no
 * Python, no torch.
 *
 *   host  create a handle, preview a plan on the host, check the error
 *         paths that need no GPU, destroy.
 *   gpu   (built with MLA_C_CONSUMER_GPU) also decode a small batch from a
 *         bf16 cache in HIP device memory and check two closed forms of
 *         attention bit for bit: a sequence with one cached token returns
 *         that token's V row, and a query of zeros (equal logits) returns the
 *         mean of the V rows.  The values are small multiples of 1/4, so every
 *         sum and the mean are exact in fp32 and in bf16.
 *
 * Prints "ok" and returns 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mla_decode.h"

#ifdef MLA_C_CONSUMER_GPU
#include <hip/hip_runtime_api.h>
#endif

#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");             \
      return 1;                          \
    }                                    \
  } while (0)

enum { NH = 16, DQK = 576, DV = 512 };

static int host_checks(void) {
  mla_decode_t h = NULL;
  const int32_t indptr[3] = {0, 1000, 1300};
  int32_t items[5 * 64];
  int n = 0, slots = 0;
  size_t ws = 0;
  CHECK(mla_decode_version() >= 10000, "version %d", mla_decode_version());
  CHECK(strcmp(mla_status_string(MLA_ERR_NOT_PLANNED), "MLA_ERR_NOT_PLANNED") == 0, "status string");
  CHECK(mla_decode_create(&h, 0, 16, 576, 512, 0.0416666679f, MLA_KV_FP8_E4M3, 1) == MLA_OK && h, "create");
  CHECK(mla_decode_create(NULL, 0, 16, 576, 512, 0.04f, MLA_KV_BF16, 1) == MLA_ERR_INVALID_ARG, "null out");
  {
    mla_decode_t h2 = (mla_decode_t)1;
    CHECK(mla_decode_create(&h2, 0, 8, 576, 512, 0.04f, MLA_KV_BF16, 1) == MLA_ERR_UNSUPPORTED && !h2,
          "unsupported head count");
  }
  CHECK(mla_decode_run(h, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL, 0, NULL) == MLA_ERR_NOT_PLANNED,
        "run before plan");
  CHECK(mla_decode_last_error(h)[0] != '\0', "last error set");
  CHECK(mla_decode_plan_preview(2, indptr, NULL, 1, MLA_KV_FP8_E4M3, 0, 256, 1, items, 64, &n, &slots, &ws) ==
            MLA_OK,
        "preview");
  {
    /* every token of both sequences in exactly one item */
    int covered[2] = {0, 0}, i;
    for (i = 0; i < n; ++i) covered[items[5 * i]] += items[5 * i + 2] - items[5 * i + 1];
    CHECK(n >= 2 && covered[0] == 1000 && covered[1] == 300, "preview covers the batch (%d items)", n);
    CHECK(ws == (size_t)slots * NH * (DV + 1) * sizeof(float), "workspace size");
  }
  CHECK(mla_decode_destroy(h) == MLA_OK, "destroy");
  CHECK(mla_decode_destroy(NULL) == MLA_OK, "destroy NULL");
  return 0;
}

#ifdef MLA_C_CONSUMER_GPU
static uint16_t bf16_of(float x) { /* exact for the values used here */
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return (uint16_t)(u >> 16);
}

static int gpu_checks(void) {
  /* sequence 0: one token (row 0); sequence 1: two tokens (rows 1, 2), query 0 */
  enum { ROWS = 3, BATCH = 2 };
  const int32_t indptr[BATCH + 1] = {0, 1, 3};
  uint16_t* kv = (uint16_t*)malloc(sizeof(uint16_t) * ROWS * DQK);
  uint16_t* q = (uint16_t*)calloc((size_t)BATCH * NH * DQK, sizeof(uint16_t));
  uint16_t* out = (uint16_t*)malloc(sizeof(uint16_t) * BATCH * NH * DV);
  void *d_kv = NULL, *d_q = NULL, *d_out = NULL, *d_ip = NULL, *d_ws = NULL;
  mla_decode_t h = NULL;
  size_t ws = 0;
  int r, d, b, hh;
  CHECK(kv && q && out, "host allocation");
  for (r = 0; r < ROWS; ++r)
    for (d = 0; d < DQK; ++d) kv[r * DQK + d] = bf16_of((float)((r * 7 + d) % 13 - 6) / 4.0f);
  for (hh = 0; hh < NH; ++hh)
    for (d = 0; d < DQK; ++d) q[hh * DQK + d] = bf16_of((float)((hh + 3 * d) % 9 - 4) / 8.0f);
  CHECK(hipMalloc(&d_kv, sizeof(uint16_t) * ROWS * DQK) == hipSuccess, "hipMalloc kv");
  CHECK(hipMalloc(&d_q, sizeof(uint16_t) * BATCH * NH * DQK) == hipSuccess, "hipMalloc q");
  CHECK(hipMalloc(&d_out, sizeof(uint16_t) * BATCH * NH * DV) == hipSuccess, "hipMalloc out");
  CHECK(hipMalloc(&d_ip, sizeof indptr) == hipSuccess, "hipMalloc indptr");
  CHECK(hipMemcpy(d_kv, kv, sizeof(uint16_t) * ROWS * DQK, hipMemcpyHostToDevice) == hipSuccess, "copy kv");
  CHECK(hipMemcpy(d_q, q, sizeof(uint16_t) * BATCH * NH * DQK, hipMemcpyHostToDevice) == hipSuccess, "copy q");
  CHECK(hipMemcpy(d_ip, indptr, sizeof indptr, hipMemcpyHostToDevice) == hipSuccess, "copy indptr");

  CHECK(mla_decode_create(&h, 0, NH, DQK, DV, 0.0416666679f, MLA_KV_BF16, 1) == MLA_OK, "create");
  CHECK(mla_decode_plan(h, BATCH, indptr, NULL, 0, &ws) == MLA_OK, "plan: %s", mla_decode_last_error(h));
  if (ws) CHECK(hipMalloc(&d_ws, ws) == hipSuccess, "hipMalloc workspace");
  CHECK(mla_decode_run(h, d_q, d_kv, NULL, 0, (const int32_t*)d_ip, NULL, NULL, d_out, d_ws, ws, NULL) == MLA_OK,
        "run: %s", mla_decode_last_error(h));
  CHECK(hipDeviceSynchronize() == hipSuccess, "synchronize");
  CHECK(hipMemcpy(out, d_out, sizeof(uint16_t) * BATCH * NH * DV, hipMemcpyDeviceToHost) == hipSuccess,
        "copy out");
  for (b = 0; b < BATCH; ++b)
    for (hh = 0; hh < NH; ++hh)
      for (d = 0; d < DV; ++d) {
        const uint16_t want =
            b == 0 ? kv[d]
                   : bf16_of(((float)((7 + d) % 13 - 6) + (float)((14 + d) % 13 - 6)) / 8.0f);
        const uint16_t got = out[(b * NH + hh) * DV + d];
        CHECK(got == want, "sequence %d head %d dim %d: 0x%04x, expected 0x%04x", b, hh, d, got, want);
      }
  CHECK(mla_decode_destroy(h) == MLA_OK, "destroy");
  (void)hipFree(d_kv);
  (void)hipFree(d_q);
  (void)hipFree(d_out);
  (void)hipFree(d_ip);
  if (d_ws) (void)hipFree(d_ws);
  free(kv);
  free(q);
  free(out);
  return 0;
}
#endif

int main(int argc, char** argv) {
  const int gpu = argc > 1 && strcmp(argv[1], "gpu") == 0;
  if (host_checks()) return 1;
#ifdef MLA_C_CONSUMER_GPU
  if (gpu && gpu_checks()) return 1;
#else
  if (gpu) {
    fprintf(stderr, "FAIL: built without MLA_C_CONSUMER_GPU\n");
    return 1;
  }
#endif
  printf("ok\n");
  return 0;
}
