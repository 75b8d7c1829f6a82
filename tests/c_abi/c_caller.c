/*
 * A plain C99 caller of the attention library's C ABI (include/attn.h), with
 * no Python and no PyTorch in the path: device buffers from hipMalloc,
 * host <-> device copies, the default stream, status codes.  Built as a
 * small shared library next to this file; the GPU test loads it and calls
 * attn_c_caller_check() in its own process.
 *
 * Every check has a closed form.  With Q = 0 every score is 0, so the
 * softmax weights of a query row are equal over the keys it sees: O is the
 * mean of the visible V rows and LSE = ln(number of visible keys)
 * ("Attention Mechanism: Computation & Memory Patterns", section 1: the
 * softmax of a row of equal scores; "Why Attention Is Difficult to
 * Optimize", "The Attention Computation Flow": the causal mask leaves query
 * i the keys 0 .. i).  V holds small multiples of 1/8, exact in bfloat16.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "attn.h"

#define TOL_O 2e-2
#define TOL_LSE 1e-3

static uint16_t bf16_of(float x) {  /* exact for the values used here */
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}
static float f32_of(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float x;
  memcpy(&x, &u, 4);
  return x;
}
/* V[t][c] of head h: a multiple of 1/8 in [-1, 1] */
static float v_val(int64_t h, int64_t t, int64_t c) {
  return (float)((h * 5 + t * 7 + c * 3) % 17 - 8) / 8.0f;
}

/* Fills a [nh][T][d] bf16 array with V (q = 0: zero). */
static uint16_t* host_v(int64_t nh, int64_t T, int64_t d) {
  uint16_t* v = (uint16_t*)malloc((size_t)(nh * T * d) * 2);
  if (!v) return NULL;
  for (int64_t h = 0; h < nh; ++h)
    for (int64_t t = 0; t < T; ++t)
      for (int64_t c = 0; c < d; ++c) v[(h * T + t) * d + c] = bf16_of(v_val(h, t, c));
  return v;
}

#define HIP_OK(call, what)                                                        \
  do {                                                                            \
    if ((call) != hipSuccess) {                                                   \
      snprintf(msg, len, "%s failed", what);                                      \
      goto done;                                                                  \
    }                                                                             \
  } while (0)

/* Compares O (bf16) and LSE of query rows r = 0 .. nrows - 1 of V head h,
 * row r seeing keys 0 .. first_key_count + r - 1, against the mean of those
 * V rows and ln(first_key_count + r); the column sums grow row by row. */
static int check_rows(const uint16_t* o, const float* lse, int64_t h, int64_t nrows,
                      int64_t d, int64_t first_key_count, char* msg, int len) {
  double sum[128] = {0};
  int64_t have = 0;  /* keys in sum */
  if (d > 128) {
    snprintf(msg, len, "d > 128");
    return 1;
  }
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t vis = first_key_count + r;
    for (; have < vis; ++have)
      for (int64_t c = 0; c < d; ++c) sum[c] += v_val(h, have, c);
    for (int64_t c = 0; c < d; ++c) {
      const double mean = sum[c] / (double)vis;
      const double got = f32_of(o[r * d + c]);
      if (fabs(got - mean) > TOL_O) {
        snprintf(msg, len, "O head %lld row %lld col %lld: %g, want %g", (long long)h,
                 (long long)r, (long long)c, got, mean);
        return 1;
      }
    }
    if (fabs(lse[r] - log((double)vis)) > TOL_LSE) {
      snprintf(msg, len, "LSE head %lld row %lld: %g, want %g", (long long)h, (long long)r,
               lse[r], log((double)vis));
      return 1;
    }
  }
  return 0;
}

/* Forward over B = 1, H heads of T rows, causal, Q = 0. */
static int check_forward(int64_t H, int64_t T, int64_t d, char* msg, int len) {
  int rc = 1;
  const size_t n = (size_t)(H * T * d);
  uint16_t* hv = host_v(H, T, d);
  uint16_t* ho = (uint16_t*)malloc(n * 2);
  float* hl = (float*)malloc((size_t)(H * T) * 4);
  void *q = NULL, *k = NULL, *v = NULL, *o = NULL;
  float* lse = NULL;
  if (!hv || !ho || !hl) {
    snprintf(msg, len, "host allocation failed");
    goto done;
  }
  HIP_OK(hipMalloc(&q, n * 2), "hipMalloc q");
  HIP_OK(hipMalloc(&k, n * 2), "hipMalloc k");
  HIP_OK(hipMalloc(&v, n * 2), "hipMalloc v");
  HIP_OK(hipMalloc(&o, n * 2), "hipMalloc o");
  HIP_OK(hipMalloc((void**)&lse, (size_t)(H * T) * 4), "hipMalloc lse");
  HIP_OK(hipMemset(q, 0, n * 2), "hipMemset q");
  HIP_OK(hipMemset(k, 0x3f, n * 2), "hipMemset k"); /* any finite keys */
  HIP_OK(hipMemcpy(v, hv, n * 2, hipMemcpyHostToDevice), "copy v");
  attn_status st = attn_fwd(q, k, v, o, lse, 1, H, T, d, 1, 0.125f, NULL);
  if (st != ATTN_OK) {
    snprintf(msg, len, "attn_fwd: %s", attn_status_string(st));
    goto done;
  }
  HIP_OK(hipDeviceSynchronize(), "synchronize");
  HIP_OK(hipMemcpy(ho, o, n * 2, hipMemcpyDeviceToHost), "copy o");
  HIP_OK(hipMemcpy(hl, lse, (size_t)(H * T) * 4, hipMemcpyDeviceToHost), "copy lse");
  {
    const int64_t heads[2] = {0, H - 1};
    for (int i = 0; i < 2; ++i)
      if (check_rows(ho + heads[i] * T * d, hl + heads[i] * T, heads[i], T, d, 1, msg, len))
        goto done;
  }
  rc = 0;
done:
  hipFree(q); hipFree(k); hipFree(v); hipFree(o); hipFree(lse);
  free(hv); free(ho); free(hl);
  return rc;
}

/* Decode of Tq = 2 new queries per head over Tk cached keys (several key
 * splits), grouped heads (G = 4), causal, Q = 0; the caller's workspace. */
static int check_decode(int64_t Tk, int64_t d, char* msg, int len) {
  int rc = 1;
  const int64_t H = 8, Hkv = 2, Tq = 2;
  const size_t nq = (size_t)(H * Tq * d), nkv = (size_t)(Hkv * Tk * d);
  uint16_t* hv = host_v(Hkv, Tk, d);
  uint16_t* ho = (uint16_t*)malloc(nq * 2);
  float* hl = (float*)malloc((size_t)(H * Tq) * 4);
  void *q = NULL, *k = NULL, *v = NULL, *o = NULL, *ws = NULL;
  float* lse = NULL;
  const int64_t wsb = attn_decode_workspace_bytes(1, H, Hkv, Tq, Tk, d);
  if (!hv || !ho || !hl || wsb < 0) {
    snprintf(msg, len, "host allocation or workspace size failed");
    goto done;
  }
  HIP_OK(hipMalloc(&q, nq * 2), "hipMalloc q");
  HIP_OK(hipMalloc(&k, nkv * 2), "hipMalloc k");
  HIP_OK(hipMalloc(&v, nkv * 2), "hipMalloc v");
  HIP_OK(hipMalloc(&o, nq * 2), "hipMalloc o");
  HIP_OK(hipMalloc((void**)&lse, (size_t)(H * Tq) * 4), "hipMalloc lse");
  if (wsb > 0) HIP_OK(hipMalloc(&ws, (size_t)wsb), "hipMalloc ws");
  HIP_OK(hipMemset(q, 0, nq * 2), "hipMemset q");
  HIP_OK(hipMemset(k, 0x3f, nkv * 2), "hipMemset k");
  HIP_OK(hipMemcpy(v, hv, nkv * 2, hipMemcpyHostToDevice), "copy v");
  attn_status st = attn_decode(q, k, v, o, lse, ws, wsb, 1, H, Hkv, Tq, Tk, Tk, d, 1, 0.125f,
                               NULL);
  if (st != ATTN_OK) {
    snprintf(msg, len, "attn_decode: %s", attn_status_string(st));
    goto done;
  }
  HIP_OK(hipDeviceSynchronize(), "synchronize");
  HIP_OK(hipMemcpy(ho, o, nq * 2, hipMemcpyDeviceToHost), "copy o");
  HIP_OK(hipMemcpy(hl, lse, (size_t)(H * Tq) * 4, hipMemcpyDeviceToHost), "copy lse");
  /* query head h reads key/value head h / 4; new query i sees Tk - 1 + i
   * keys (rows 0 .. Tk - 2 + i) */
  for (int64_t h = 0; h < H; ++h)
    if (check_rows(ho + h * Tq * d, hl + h * Tq, h / (H / Hkv), Tq, d, Tk - 1, msg, len))
      goto done;
  rc = 0;
done:
  hipFree(q); hipFree(k); hipFree(v); hipFree(o); hipFree(lse); hipFree(ws);
  free(hv); free(ho); free(hl);
  return rc;
}

/* Runs every check; returns 0 when all pass.  msg (len bytes) receives a
 * description of the first failure or of what passed. */
int attn_c_caller_check(char* msg, int len) {
  /* row-chunk forward (small grid), then the 8-wave forward (32 heads) */
  if (check_forward(2, 300, 64, msg, len)) return 1;
  if (check_forward(32, 2048, 128, msg, len)) return 2;
  /* decode with several key splits (their merge) and with one */
  if (attn_decode_splits(1, 8, 2, 2, 20000) < 2) {
    snprintf(msg, len, "expected several key splits");
    return 3;
  }
  if (check_decode(20000, 128, msg, len)) return 4;
  if (check_decode(100, 64, msg, len)) return 5;
  snprintf(msg, len, "forward and decode checks passed");
  return 0;
}
