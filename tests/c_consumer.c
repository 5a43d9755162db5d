/*
 * A plain C consumer of libfrattn: no framework types, only the HIP runtime
 * for device memory.  It runs fr_decode_attn (the decomposed decode attention
 * of FlashRT PR #185: softmax(scale * q.K^T + mask).V per query row, rows in
 * t-major order) on a case whose result is known exactly, checks every output
 * bit, then checks that invalid calls return their status.  Exit status 0 on
 * success.
 *
 * The case: query row r = t*n_head + h is one-hot on column r and owns key
 * j(r) = 3r + 1, whose row is 2048 on that column; every other key row is
 * zero.  With scale 1/16 the owned key's logit is 128 and every other 0; e^-128
 * is below the smallest fp32 subnormal, so the softmax is exactly one-hot and
 * out[r] must equal V[j(r)] bit for bit.  70 keys: a ragged last key block.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "fr_decode_attn.h"

enum { NH = 4, NT = 3, NKV = 70, HD = 64, M = NH * NT };

/* binary16 bits of an integer with |x| <= 2048 (exact) */
static uint16_t f16_of_int(int x) {
  if (x == 0) return 0;
  const uint16_t sign = x < 0 ? 0x8000u : 0u;
  const unsigned m = (unsigned)(x < 0 ? -x : x);
  int e = 0;
  while ((m >> (e + 1)) != 0) ++e;                 /* 2^e <= m < 2^(e+1) */
  const unsigned rest = m - (1u << e);
  const unsigned frac = e <= 10 ? rest << (10 - e) : rest >> (e - 10);
  return (uint16_t)(sign | ((unsigned)(e + 15) << 10) | frac);
}

static int v_value(int j, int d) { return (j * 7 + d * 3) % 17 - 8; }

#define CHECK_HIP(call)                                                     \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
      return 1;                                                             \
    }                                                                       \
  } while (0)

int main(void) {
  static float q[M * HD], out[M * HD];
  static uint16_t k[NKV * HD], v[NKV * HD];
  for (int i = 0; i < M * HD; ++i) q[i] = 0.f;
  for (int i = 0; i < NKV * HD; ++i) k[i] = 0;
  for (int j = 0; j < NKV; ++j)
    for (int d = 0; d < HD; ++d) v[j * HD + d] = f16_of_int(v_value(j, d));
  for (int r = 0; r < M; ++r) {
    q[r * HD + r] = 1.f;
    k[(3 * r + 1) * HD + r] = f16_of_int(2048);
  }

  float *dq, *dout;
  uint16_t *dk, *dv;
  CHECK_HIP(hipMalloc((void **)&dq, sizeof q));
  CHECK_HIP(hipMalloc((void **)&dout, sizeof out));
  CHECK_HIP(hipMalloc((void **)&dk, sizeof k));
  CHECK_HIP(hipMalloc((void **)&dv, sizeof v));
  CHECK_HIP(hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dk, k, sizeof k, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, v, sizeof v, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemset(dout, 0xff, sizeof out));   /* NaN everywhere before the call */

  int st = fr_decode_attn(dq, dk, dv, NULL, dout, NH, NT, NKV, HD, 1.0f / 16, NULL);
  if (st != FR_OK) {
    fprintf(stderr, "fr_decode_attn: %s\n", fr_status_str(st));
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));

  int bad = 0;
  for (int r = 0; r < M; ++r)
    for (int d = 0; d < HD; ++d) {
      const float want = (float)v_value(3 * r + 1, d);
      if (out[r * HD + d] != want) {
        if (bad < 5) fprintf(stderr, "out[%d][%d] = %g, want %g\n", r, d, out[r * HD + d], want);
        ++bad;
      }
    }
  if (bad) {
    fprintf(stderr, "%d outputs differ\n", bad);
    return 1;
  }

  /* rejected calls return their status and launch nothing */
  if (fr_decode_attn(NULL, dk, dv, NULL, dout, NH, NT, NKV, HD, 1.0f / 16, NULL) != FR_ERR_INVALID ||
      fr_decode_attn(dq, dk, dv, NULL, dout, NH, NT, NKV, 96, 1.0f / 16, NULL) != FR_ERR_UNSUPPORTED ||
      fr_decode_attn(dq, dk, dv, NULL, dout, 0, NT, NKV, HD, 1.0f / 16, NULL) != FR_ERR_INVALID ||
      fr_decode_attn(dq, dk, dv, NULL, dout, NH, FR_MAX_TOKENS_UNMASKED + 1, NKV, HD, 1.0f / 16,
                     NULL) != FR_ERR_UNSUPPORTED) {
    fprintf(stderr, "an invalid call was not rejected\n");
    return 1;
  }
  CHECK_HIP(hipFree(dq));
  CHECK_HIP(hipFree(dout));
  CHECK_HIP(hipFree(dk));
  CHECK_HIP(hipFree(dv));
  printf("c consumer: %d rows bit-exact, invalid calls rejected\n", M);
  return 0;
}
