/*
 * A plain C consumer of the library: no Python, no torch. It allocates device
 * memory with the HIP runtime's C API, plans and runs one dense and one
 * index-selected sparse decode through include/decode_attn.h, and checks both
 * against the fp64 oracle (oracle/decode_oracle.c, linked as liboracle.so;
 * test infrastructure) under the tolerance contract: |gpu - ref| <=
 * 2e-2 + 1e-2 |ref| elementwise and relative L2 <= 1e-2. Also checks that a
 * rejected feature fails closed with a status and a message.
 * Prints "c consumer ok" and exits 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "decode_attn.h"

int oracle_dense(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *out,
                 int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t capacity,
                 int64_t k_len, float scale, const int64_t *rows, int64_t nrows, int nthreads);
int oracle_sparse(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *sel,
                  int32_t topk, double *out, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                  int32_t kv_batch, int64_t capacity, int64_t k_len, float scale,
                  const int64_t *rows, int64_t nrows, int nthreads);

#define HIP_OK(x)                                                                  \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(2);                                                                     \
    }                                                                              \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform01(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}
static uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static void fill(uint16_t *x, size_t n) { /* roughly N(0, 1): sum of 4 uniforms */
  for (size_t i = 0; i < n; ++i) {
    const double s = uniform01() + uniform01() + uniform01() + uniform01() - 2.0;
    x[i] = bf16_rne((float)(s * 1.7320508));
  }
}

static int check(const char *what, const uint16_t *got, const double *ref, size_t n) {
  double num = 0.0, den = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double g = bf16_to_f32(got[i]), r = ref[i], err = fabs(g - r);
    if (!(err <= 2e-2 + 1e-2 * fabs(r))) {
      fprintf(stderr, "%s: element %zu got %g want %g\n", what, i, g, r);
      return 1;
    }
    num += (g - r) * (g - r);
    den += r * r;
  }
  if (den > 0 && sqrt(num / den) > 1e-2) {
    fprintf(stderr, "%s: relative L2 error %g\n", what, sqrt(num / den));
    return 1;
  }
  printf("%s: %zu elements within tolerance (relative L2 %.2e)\n", what, n,
         den > 0 ? sqrt(num / den) : 0.0);
  return 0;
}

static decode_attn_problem problem(int B, int Hq, int Hkv, int D, int64_t cap, int topk) {
  decode_attn_problem p;
  memset(&p, 0, sizeof p);
  p.batch = B;
  p.num_q_heads = Hq;
  p.num_kv_heads = Hkv;
  p.head_dim = D;
  p.seq_q = 1;
  p.capacity = cap;
  p.max_k_len = cap;
  p.topk_max = topk;
  p.kv_batch = topk ? 1 : 0;
  p.window_left = -1;
  p.window_right = -1;
  return p;
}

int main(void) {
  const int B = 2, Hq = 16, Hkv = 4, D = 128;
  const int64_t cap = 3000, k_len = 2500;
  const float scale = 0.088388347648f; /* 1/sqrt(128) in f32 */
  const size_t nq = (size_t)B * Hq * D, nkv = (size_t)B * Hkv * cap * D;
  uint16_t *q = malloc(nq * 2), *k = malloc(nkv * 2), *v = malloc(nkv * 2), *out = malloc(nq * 2);
  double *ref = malloc(nq * sizeof(double));
  fill(q, nq);
  fill(k, nkv);
  fill(v, nkv);

  void *dq, *dk, *dv, *dout, *ws = NULL;
  HIP_OK(hipMalloc(&dq, nq * 2));
  HIP_OK(hipMalloc(&dk, nkv * 2));
  HIP_OK(hipMalloc(&dv, nkv * 2));
  HIP_OK(hipMalloc(&dout, nq * 2));
  HIP_OK(hipMemcpy(dq, q, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, k, nkv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, v, nkv * 2, hipMemcpyHostToDevice));

  /* a rejected feature fails closed */
  decode_attn_problem bad = problem(B, Hq, Hkv, D, cap, 0);
  bad.has_alibi = 1;
  decode_attn_plan_t plan;
  if (decode_attn_plan(&bad, &plan) != DA_ERR_UNSUPPORTED || !strstr(decode_attn_last_error(), "alibi")) {
    fprintf(stderr, "ALiBi was not rejected\n");
    return 1;
  }
  printf("rejected: %s (%s)\n", decode_attn_status_str(DA_ERR_UNSUPPORTED), decode_attn_last_error());

  /* dense */
  decode_attn_problem p = problem(B, Hq, Hkv, D, cap, 0);
  if (decode_attn_plan(&p, &plan) != DA_OK) {
    fprintf(stderr, "plan: %s\n", decode_attn_last_error());
    return 1;
  }
  if (plan.workspace_bytes) HIP_OK(hipMalloc(&ws, plan.workspace_bytes));
  if (decode_attn_dense(&plan, dq, dk, dv, dout, scale, k_len, ws, plan.workspace_bytes, NULL) != DA_OK) {
    fprintf(stderr, "dense: %s\n", decode_attn_last_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(out, dout, nq * 2, hipMemcpyDeviceToHost));
  if (oracle_dense(q, k, v, ref, B, Hq, Hkv, D, cap, k_len, scale, NULL, 0, 4)) return 1;
  if (check("dense", out, ref, nq)) return 1;
  if (ws) HIP_OK(hipFree(ws));
  ws = NULL;

  /* sparse over KV set 0 (shared), 96 valid entries then -1 pads to topk 128 */
  const int topk = 128;
  int32_t *sel = malloc((size_t)B * topk * 4);
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < topk; ++t)
      sel[b * topk + t] = t < 96 ? (int32_t)((t * 37 + b * 11) % k_len) : -1;
  void *dsel;
  HIP_OK(hipMalloc(&dsel, (size_t)B * topk * 4));
  HIP_OK(hipMemcpy(dsel, sel, (size_t)B * topk * 4, hipMemcpyHostToDevice));
  decode_attn_problem ps = problem(B, Hq, Hkv, D, cap, topk);
  if (decode_attn_plan(&ps, &plan) != DA_OK) {
    fprintf(stderr, "sparse plan: %s\n", decode_attn_last_error());
    return 1;
  }
  if (plan.workspace_bytes) HIP_OK(hipMalloc(&ws, plan.workspace_bytes));
  if (decode_attn_sparse(&plan, dq, dk, dv, dsel, topk, dout, scale, k_len, ws,
                         plan.workspace_bytes, NULL) != DA_OK) {
    fprintf(stderr, "sparse: %s\n", decode_attn_last_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(out, dout, nq * 2, hipMemcpyDeviceToHost));
  /* the oracle sees KV set 0 only (kv_batch = 1) */
  if (oracle_sparse(q, k, v, sel, topk, ref, B, Hq, Hkv, D, 1, cap, k_len, scale, NULL, 0, 4))
    return 1;
  if (check("sparse", out, ref, nq)) return 1;

  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(dsel));
  if (ws) HIP_OK(hipFree(ws));
  free(q); free(k); free(v); free(out); free(ref); free(sel);
  printf("c consumer ok\n");
  return 0;
}
