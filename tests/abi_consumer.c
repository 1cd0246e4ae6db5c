/*
 * abi_consumer.c -- a plain C program that uses librlk_logp.so through
 * include/rlk_logp.h only (HIP runtime for memory and streams, no C++ and no
 * Python).  It checks properties that hold by construction:
 *   - every virtual-shard count S gives the bits of S = 1;
 *   - logp = fp32(x[target]) - LSE exactly, +0.0 on inactive rows;
 *   - each backward row sums to about 0 (g (1 - sum softmax));
 *   - rlk_logp_fwd_bwd gives the bits of rlk_logp_fwd then rlk_logp_bwd, and
 *     rlk_logp_fwd_bwd_ex those of rlk_logp_fwd_ex then rlk_logp_bwd_ex;
 *   - host errors come back as status codes with a reason.
 * Prints one line per check and exits 0 only if all pass.  Built by the
 * package's build step; run by tests/test_gpu_abi_consumer.py.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rlk_logp.h"

#define CHECK_HIP(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 2;                                                             \
    }                                                                       \
  } while (0)
#define CHECK_RLK(x)                                                        \
  do {                                                                      \
    rlk_status s_ = (x);                                                    \
    if (s_ != RLK_OK) {                                                     \
      fprintf(stderr, "%s: %s at line %d\n", rlk_status_string(s_), rlk_last_error_detail(), \
              __LINE__);                                                    \
      return 3;                                                             \
    }                                                                       \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}
static uint16_t f32_to_bf16_trunc(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int main(void) {
  const int64_t n = 96, v_real = 5000, v_pad = 5120, ld = 5120;
  const int32_t tiles = 16;
  uint16_t* x = malloc(sizeof(uint16_t) * n * ld);
  int32_t* tgt = malloc(sizeof(int32_t) * n);
  uint8_t* mask = malloc(n);
  float* g = malloc(sizeof(float) * n);
  for (int64_t i = 0; i < n * ld; ++i) {
    const double u = (double)(next_u64() >> 11) / 9007199254740992.0;
    x[i] = f32_to_bf16_trunc((float)(6.0 * u - 3.0));
  }
  for (int64_t r = 0; r < n; ++r) {
    tgt[r] = (int32_t)(next_u64() % (uint64_t)v_real);
    mask[r] = (r % 5) != 0;
    g[r] = (float)((int)(next_u64() % 200) - 100) / 50.0f;
  }

  void *dx, *dtgt, *dmask, *dg, *dlogp, *dlse, *dlogp2, *dlse2, *dws, *dd;
  CHECK_HIP(hipMalloc(&dx, sizeof(uint16_t) * n * ld));
  CHECK_HIP(hipMalloc(&dtgt, sizeof(int32_t) * n));
  CHECK_HIP(hipMalloc(&dmask, n));
  CHECK_HIP(hipMalloc(&dg, sizeof(float) * n));
  CHECK_HIP(hipMalloc(&dlogp, sizeof(float) * n));
  CHECK_HIP(hipMalloc(&dlse, sizeof(float) * n));
  CHECK_HIP(hipMalloc(&dlogp2, sizeof(float) * n));
  CHECK_HIP(hipMalloc(&dlse2, sizeof(float) * n));
  CHECK_HIP(hipMalloc(&dd, sizeof(float) * n * ld));
  CHECK_HIP(hipMemcpy(dx, x, sizeof(uint16_t) * n * ld, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dtgt, tgt, sizeof(int32_t) * n, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dmask, mask, n, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dg, g, sizeof(float) * n, hipMemcpyHostToDevice));
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  rlk_logp_desc desc = {n, v_real, v_pad, ld, tiles, 1, -100, RLK_FLAG_VALIDATE};
  const size_t ws_bytes = rlk_logp_workspace_bytes(&desc);
  CHECK_HIP(hipMalloc(&dws, ws_bytes));
  CHECK_RLK(rlk_logp_fwd(&desc, dx, dtgt, dmask, dlogp, dlse, dws, ws_bytes, stream));
  float* logp = malloc(sizeof(float) * n);
  float* lse = malloc(sizeof(float) * n);
  float* logp2 = malloc(sizeof(float) * n);
  float* lse2 = malloc(sizeof(float) * n);
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_HIP(hipMemcpy(logp, dlogp, sizeof(float) * n, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(lse, dlse, sizeof(float) * n, hipMemcpyDeviceToHost));

  int failures = 0;
  const int32_t shard_counts[] = {2, 3, 4, 16};
  for (int i = 0; i < 4; ++i) {
    rlk_logp_desc d2 = desc;
    d2.num_virtual_shards = shard_counts[i];
    CHECK_RLK(rlk_logp_fwd(&d2, dx, dtgt, dmask, dlogp2, dlse2, dws, ws_bytes, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(logp2, dlogp2, sizeof(float) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(lse2, dlse2, sizeof(float) * n, hipMemcpyDeviceToHost));
    const int same = memcmp(logp, logp2, sizeof(float) * n) == 0 &&
                     memcmp(lse, lse2, sizeof(float) * n) == 0;
    printf("S=%d bitwise equal to S=1: %s\n", shard_counts[i], same ? "ok" : "FAIL");
    failures += !same;
  }

  int gather_ok = 1;
  for (int64_t r = 0; r < n; ++r) {
    if (!mask[r]) {
      uint32_t bits;
      memcpy(&bits, &logp[r], 4);
      gather_ok &= bits == 0u;
    } else {
      const float want = bf16_to_f32(x[r * ld + tgt[r]]) - lse[r];
      gather_ok &= memcmp(&want, &logp[r], 4) == 0;
    }
  }
  printf("logp = x[target] - LSE exactly, +0 on inactive rows: %s\n", gather_ok ? "ok" : "FAIL");
  failures += !gather_ok;

  CHECK_RLK(rlk_logp_bwd(&desc, dx, dtgt, dmask, dlse, dg, dd, ld, RLK_DTYPE_F32, dws, ws_bytes,
                         stream));
  float* d = malloc(sizeof(float) * n * ld);
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_HIP(hipMemcpy(d, dd, sizeof(float) * n * ld, hipMemcpyDeviceToHost));
  double worst = 0.0;
  int zeros_ok = 1;
  for (int64_t r = 0; r < n; ++r) {
    double sum = 0.0;
    for (int64_t j = 0; j < v_pad; ++j) {
      sum += d[r * ld + j];
      if ((!mask[r] || j >= v_real) && d[r * ld + j] != 0.0f) zeros_ok = 0;
    }
    const double rel = fabs(sum) / (fabs((double)g[r]) > 1.0 ? fabs((double)g[r]) : 1.0);
    if (rel > worst) worst = rel;
  }
  printf("backward rows sum to ~0 (worst %.2e), zeros where inactive or padded: %s\n", worst,
         (worst < 1e-4 && zeros_ok) ? "ok" : "FAIL");
  failures += !(worst < 1e-4 && zeros_ok);

  /* the one-launch calls: the same bits as the separate ones */
  {
    const size_t ws1_bytes = rlk_logp_fwd_bwd_workspace_bytes(&desc);
    const size_t wse_bytes = rlk_logp_ex_workspace_bytes(&desc);
    const size_t wsx_bytes = rlk_logp_fwd_bwd_ex_workspace_bytes(&desc);
    float* gl = malloc(sizeof(float) * n);
    float* gh = malloc(sizeof(float) * n);
    for (int64_t r = 0; r < n; ++r) {
      gl[r] = (float)((int)(next_u64() % 200) - 100) / 100.0f;
      gh[r] = (float)((int)(next_u64() % 200) - 100) / 100.0f;
    }
    void *dws1, *dwse, *dwsx, *dgl, *dgh, *dent, *dent2, *dd2, *dd3;
    CHECK_HIP(hipMalloc(&dws1, ws1_bytes));
    CHECK_HIP(hipMalloc(&dwse, wse_bytes));
    CHECK_HIP(hipMalloc(&dwsx, wsx_bytes));
    CHECK_HIP(hipMalloc(&dgl, sizeof(float) * n));
    CHECK_HIP(hipMalloc(&dgh, sizeof(float) * n));
    CHECK_HIP(hipMalloc(&dent, sizeof(float) * n));
    CHECK_HIP(hipMalloc(&dent2, sizeof(float) * n));
    CHECK_HIP(hipMalloc(&dd2, sizeof(float) * n * ld));
    CHECK_HIP(hipMalloc(&dd3, sizeof(float) * n * ld));
    CHECK_HIP(hipMemcpy(dgl, gl, sizeof(float) * n, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dgh, gh, sizeof(float) * n, hipMemcpyHostToDevice));
    float* d2 = malloc(sizeof(float) * n * ld);
    float* d3 = malloc(sizeof(float) * n * ld);
    float* ent = malloc(sizeof(float) * n);
    float* ent2 = malloc(sizeof(float) * n);

    CHECK_RLK(rlk_logp_fwd_bwd(&desc, dx, dtgt, dmask, dg, dlogp2, dlse2, dd2, ld, RLK_DTYPE_F32,
                               dws1, ws1_bytes, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(logp2, dlogp2, sizeof(float) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(lse2, dlse2, sizeof(float) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(d2, dd2, sizeof(float) * n * ld, hipMemcpyDeviceToHost));
    int same = memcmp(logp, logp2, sizeof(float) * n) == 0 &&
               memcmp(lse, lse2, sizeof(float) * n) == 0;
    for (int64_t r = 0; r < n; ++r)  /* columns [0, V_pad) of each row */
      same &= memcmp(d + r * ld, d2 + r * ld, sizeof(float) * v_pad) == 0;
    printf("rlk_logp_fwd_bwd bitwise equal to the two calls: %s\n", same ? "ok" : "FAIL");
    failures += !same;

    CHECK_RLK(rlk_logp_fwd_ex(&desc, dx, dtgt, dmask, dlogp, dlse, dent, dwse, wse_bytes, stream));
    CHECK_RLK(rlk_logp_bwd_ex(&desc, dx, dtgt, dmask, dlse, dent, dg, dgl, dgh, dd2, ld,
                              RLK_DTYPE_F32, dwse, wse_bytes, stream));
    CHECK_RLK(rlk_logp_fwd_bwd_ex(&desc, dx, dtgt, dmask, dg, dgl, dgh, dlogp2, dlse2, dent2, dd3,
                                  ld, RLK_DTYPE_F32, dwsx, wsx_bytes, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(logp, dlogp, sizeof(float) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(lse, dlse, sizeof(float) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(ent, dent, sizeof(float) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(logp2, dlogp2, sizeof(float) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(lse2, dlse2, sizeof(float) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(ent2, dent2, sizeof(float) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(d2, dd2, sizeof(float) * n * ld, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(d3, dd3, sizeof(float) * n * ld, hipMemcpyDeviceToHost));
    same = memcmp(logp, logp2, sizeof(float) * n) == 0 &&
           memcmp(lse, lse2, sizeof(float) * n) == 0 && memcmp(ent, ent2, sizeof(float) * n) == 0;
    for (int64_t r = 0; r < n; ++r)
      same &= memcmp(d2 + r * ld, d3 + r * ld, sizeof(float) * v_pad) == 0;
    printf("rlk_logp_fwd_bwd_ex bitwise equal to the two extended calls: %s\n",
           same ? "ok" : "FAIL");
    failures += !same;

    hipFree(dws1); hipFree(dwse); hipFree(dwsx); hipFree(dgl); hipFree(dgh); hipFree(dent);
    hipFree(dent2); hipFree(dd2); hipFree(dd3);
    free(gl); free(gh); free(d2); free(d3); free(ent); free(ent2);
  }

  rlk_logp_desc bad = desc;
  bad.num_vocab_tiles = 0;
  const rlk_status st = rlk_logp_fwd(&bad, dx, dtgt, dmask, dlogp, dlse, dws, ws_bytes, stream);
  const int err_ok = st == RLK_ERR_BAD_TILING && strlen(rlk_last_error_detail()) > 0;
  printf("host error reported (%s: %s): %s\n", rlk_status_string(st), rlk_last_error_detail(),
         err_ok ? "ok" : "FAIL");
  failures += !err_ok;

  CHECK_HIP(hipStreamDestroy(stream));
  hipFree(dx); hipFree(dtgt); hipFree(dmask); hipFree(dg); hipFree(dlogp); hipFree(dlse);
  hipFree(dlogp2); hipFree(dlse2); hipFree(dws); hipFree(dd);
  free(x); free(tgt); free(mask); free(g); free(logp); free(lse); free(logp2); free(lse2); free(d);
  printf("%s\n", failures ? "abi consumer: FAILED" : "abi consumer: all checks passed");
  return failures ? 1 : 0;
}
