/*
 * abi_demo.c -- the decode-attention library used from plain C (C11), with no
 * Python and no torch: only include/decode_attention.h, libdecode_attention.so
 * and the HIP runtime for device memory.  Test infrastructure: it links the fp64
 * C oracle (oracle/decode_oracle.c) to check what the library computes.
 *
 *   abi_demo host   status strings, workspace sizes and argument checks (no GPU)
 *   abi_demo gpu    GQA (paged, ragged, sinks) and MLA (causal MTP) calls on the
 *                   device at one and at several partitions, and the partition
 *                   pass + splitk_reduce() pair, each against the oracle
 *
 * Inputs come from a 64-bit linear congruential generator (Knuth's MMIX
 * constants) turned into approximately normal values by summing uniforms; they
 * are rounded to bf16 here and handed identically to both sides.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "decode_attention.h"

/* The oracle's entry point (oracle/decode_oracle.c). */
int oracle_decode_attention(const void* q, const void* k, const void* v, int dtype,
                            float k_scale, float v_scale, const uint32_t* page_table,
                            int page_size, int max_pages, const uint32_t* valid_length, int B,
                            int T, int H, int KVH, int D, int Dv, int S, float scale,
                            const float* sink, int causal, const uint32_t* q_offsets,
                            const int32_t* indices, int indices_stride,
                            const int32_t* topk_lengths, int64_t pool_rows,
                            const uint32_t* kv_offsets, const int64_t* rows, int64_t num_rows,
                            double* out, double* lse, int num_threads);

static int failures = 0;

#define CHECK(cond, ...)                     \
  do {                                       \
    if (!(cond)) {                           \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");                 \
      ++failures;                            \
    }                                        \
  } while (0)

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, \
              __LINE__);                                                          \
      exit(2);                                                                    \
    }                                                                             \
  } while (0)

/* ---- seeded inputs --------------------------------------------------------- */

static uint64_t lcg_state;
static double lcg_uniform(void) {
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(lcg_state >> 11) * (1.0 / 9007199254740992.0);
}
/* Irwin-Hall: the sum of 12 uniforms minus 6 has mean 0 and variance 1. */
static float lcg_normal(void) {
  double s = 0.0;
  for (int i = 0; i < 12; ++i) s += lcg_uniform();
  return (float)(s - 6.0);
}
/* float -> bf16 bits, round to nearest even (inputs are finite). */
static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}
static uint16_t* normal_bf16(size_t n) {
  uint16_t* a = (uint16_t*)malloc(n * sizeof(uint16_t));
  for (size_t i = 0; i < n; ++i) a[i] = to_bf16(lcg_normal());
  return a;
}

static void* to_device(const void* h, size_t bytes) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
  if (bytes) HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}

/* Max |gpu - oracle| over outputs (bf16) and over finite LSEs; LSE infinities must
 * agree. */
static void compare(const char* what, const uint16_t* out, const float* lse, const double* ref,
                    const double* ref_lse, size_t rows, int dv) {
  double err = 0.0, lerr = 0.0;
  for (size_t i = 0; i < rows * (size_t)dv; ++i) {
    double e = fabs(bf16_to_double(out[i]) - ref[i]);
    if (!(e <= err)) err = e; /* NaN-propagating max */
  }
  for (size_t r = 0; r < rows; ++r) {
    if (isinf(ref_lse[r]) || isinf(lse[r])) {
      CHECK(isinf(ref_lse[r]) && isinf(lse[r]), "%s: LSE infinity differs at row %zu", what, r);
      continue;
    }
    double e = fabs((double)lse[r] - ref_lse[r]);
    if (!(e <= lerr)) lerr = e;
  }
  printf("%-44s max|out-ref| %.3e  max|lse-ref| %.3e\n", what, err, lerr);
  CHECK(err <= 1e-2, "%s: output error %.3e", what, err);
  CHECK(lerr <= 1e-3, "%s: LSE error %.3e", what, lerr);
}

/* ---- host-only checks ------------------------------------------------------- */

static void host_checks(void) {
  CHECK(strcmp(decode_attention_status_string(DA_OK), "ok") == 0, "status string of DA_OK");
  CHECK(strcmp(decode_attention_status_string(-99), "unknown status") == 0, "unknown status");
  /* workspace: 256-byte queue section, then [P, rows, Dv], [P, rows], [P, rows], each
   * 256-byte aligned */
  size_t ws = decode_workspace_size(4, 2, 1, 8, 128);
  CHECK(ws == 256 + 4 * 16 * 128 * 4 + 2 * 256, "workspace size %zu", ws);
  CHECK(decode_workspace_o_offset(4, 2, 1, 8, 128) == 256, "o offset");
  /* argument checks return before anything is enqueued (no device is touched) */
  int rc = decode_attention(NULL, (void*)1, (void*)1, NULL, 0, 0, NULL, 1, 1, 8, 1, 64, 64,
                            0.1f, 1, NULL, DA_MASK_NONE, DA_BF16, (void*)1, NULL, NULL, 0, NULL);
  CHECK(rc == DA_ERR_INVALID_ARG, "null q: %d", rc);
  rc = decode_attention((void*)1, (void*)1, (void*)1, NULL, 0, 0, NULL, 1, 1, 8, 1, 96, 64, 0.1f,
                        1, NULL, DA_MASK_NONE, DA_BF16, (void*)1, NULL, NULL, 0, NULL);
  CHECK(rc == DA_ERR_UNSUPPORTED, "depth 96: %d", rc);
  rc = mla_decode((void*)1, (void*)1, NULL, 0, 0, NULL, 2, 1, 128, 64, 0.1f, 3, NULL,
                  DA_MASK_NONE, (void*)1, NULL, NULL, 0, NULL);
  CHECK(rc == DA_ERR_WORKSPACE, "MLA with P = 3 and no workspace: %d", rc);
  int P = decode_num_partitions(32, 1, 32, 8, 128, 128, 4096, 0, 256);
  CHECK(P == 1, "heuristic for the GQA problem on 256 CUs: %d", P);
  printf("host checks: %s\n", failures ? "FAILED" : "ok");
}

/* ---- device calls ------------------------------------------------------------ */

/* GQA: B = 3, 32 query / 4 KV heads, depth 128, 64-key pages, ragged, sinks. */
static void gqa_case(void) {
  const int B = 3, T = 1, H = 32, KVH = 4, D = 128, ps = 64, S = 700;
  const int max_pages = (S + ps - 1) / ps;
  const uint32_t lens[3] = {700, 129, 1};
  int need = 0;
  for (int b = 0; b < B; ++b) need += (int)((lens[b] + ps - 1) / ps);
  const int pages = need + 1; /* a spare page that no table entry names */
  uint32_t* table = (uint32_t*)malloc(sizeof(uint32_t) * B * max_pages);
  int next = 0;
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < max_pages; ++i)
      table[b * max_pages + i] =
          i < (int)((lens[b] + ps - 1) / ps) ? (uint32_t)(pages - 2 - next++) : (uint32_t)(pages - 1);
  const size_t nq = (size_t)B * T * H * D, nkv = (size_t)pages * ps * KVH * D;
  uint16_t* q = normal_bf16(nq);
  uint16_t* k = normal_bf16(nkv);
  uint16_t* v = normal_bf16(nkv);
  float sink[32];
  for (int h = 0; h < H; ++h) sink[h] = lcg_normal();
  const float scale = 0.08838834764831845f;

  const size_t rows = (size_t)B * T * H;
  double* ref = (double*)malloc(sizeof(double) * rows * D);
  double* ref_lse = (double*)malloc(sizeof(double) * rows);
  int rc = oracle_decode_attention(q, k, v, 1, 1.f, 1.f, table, ps, max_pages, lens, B, T, H,
                                   KVH, D, D, S, scale, sink, 0, NULL, NULL, 0, NULL, 0, NULL,
                                   NULL, (int64_t)rows, ref, ref_lse, 0);
  CHECK(rc == 0, "oracle (GQA): %d", rc);

  void *dq = to_device(q, nq * 2), *dk = to_device(k, nkv * 2), *dv = to_device(v, nkv * 2);
  void* dtable = to_device(table, sizeof(uint32_t) * B * max_pages);
  void* dlens = to_device(lens, sizeof(lens));
  void* dsink = to_device(sink, sizeof(float) * H);
  void *dout = NULL, *dlse = NULL, *dws = NULL;
  HIP_OK(hipMalloc(&dout, rows * D * 2));
  HIP_OK(hipMalloc(&dlse, rows * 4));
  uint16_t* out = (uint16_t*)malloc(rows * D * 2);
  float* lse = (float*)malloc(rows * 4);
  const int parts[3] = {1, 3, 0};
  for (int i = 0; i < 3; ++i) {
    int P = parts[i] ? parts[i]
                     : decode_num_partitions(B, T, H, KVH, D, D, S, 1, 0);
    size_t wsb = decode_workspace_size(P, B, T, H, D);
    HIP_OK(hipMalloc(&dws, wsb));
    HIP_OK(hipMemset(dws, 0, wsb)); /* the work-queue word starts at zero */
    rc = decode_attention(dq, dk, dv, (const uint32_t*)dtable, ps, max_pages,
                          (const uint32_t*)dlens, B, T, H, H / KVH, D, S, scale, P,
                          (const float*)dsink, DA_MASK_NONE, DA_BF16, dout, (float*)dlse, dws,
                          wsb, NULL);
    CHECK(rc == DA_OK, "decode_attention P=%d: %s", P, decode_attention_status_string(rc));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(out, dout, rows * D * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse, dlse, rows * 4, hipMemcpyDeviceToHost));
    char what[64];
    snprintf(what, sizeof what, "GQA paged ragged sinks, P=%d", P);
    compare(what, out, lse, ref, ref_lse, rows, D);
    HIP_OK(hipFree(dws));
  }

  /* the partition pass alone, then splitk_reduce() on its workspace */
  {
    const int P = 4;
    size_t wsb = decode_workspace_size(P, B, T, H, D);
    HIP_OK(hipMalloc(&dws, wsb));
    HIP_OK(hipMemset(dws, 0, wsb));
    rc = decode_attention_partials(dq, dk, dv, (const uint32_t*)dtable, ps, max_pages,
                                   (const uint32_t*)dlens, B, T, H, H / KVH, D, S, scale, P,
                                   DA_MASK_NONE, DA_BF16, dws, wsb, NULL);
    CHECK(rc == DA_OK, "partials: %s", decode_attention_status_string(rc));
    char* base = (char*)dws;
    rc = splitk_reduce((const float*)(base + decode_workspace_o_offset(P, B, T, H, D)),
                       (const float*)(base + decode_workspace_max_offset(P, B, T, H, D)),
                       (const float*)(base + decode_workspace_sum_offset(P, B, T, H, D)), P,
                       (int)rows, H, D, (const float*)dsink, dout, DA_BF16, (float*)dlse, NULL);
    CHECK(rc == DA_OK, "splitk_reduce: %s", decode_attention_status_string(rc));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(out, dout, rows * D * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse, dlse, rows * 4, hipMemcpyDeviceToHost));
    compare("GQA partials + splitk_reduce, P=4", out, lse, ref, ref_lse, rows, D);
    HIP_OK(hipFree(dws));
  }
  hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dtable); hipFree(dlens); hipFree(dsink);
  hipFree(dout); hipFree(dlse);
  free(q); free(k); free(v); free(table); free(ref); free(ref_lse); free(out); free(lse);
}

/* MLA: B = 2, two MTP tokens (causal), 128 heads, depth 576 / 512, 400 keys. */
static void mla_case(void) {
  const int B = 2, T = 2, H = 128, D = 576, Dv = 512, S = 400;
  const uint32_t lens[2] = {400, 45};
  const size_t nq = (size_t)B * T * H * D, nkv = (size_t)B * S * D;
  uint16_t* q = normal_bf16(nq);
  uint16_t* kv = normal_bf16(nkv);
  const float scale = 0.07216878364870322f; /* 1 / sqrt(192) */
  const size_t rows = (size_t)B * T * H;
  double* ref = (double*)malloc(sizeof(double) * rows * Dv);
  double* ref_lse = (double*)malloc(sizeof(double) * rows);
  int rc = oracle_decode_attention(q, kv, NULL, 1, 1.f, 1.f, NULL, 0, 0, lens, B, T, H, 1, D, Dv,
                                   S, scale, NULL, 1, NULL, NULL, 0, NULL, 0, NULL, NULL,
                                   (int64_t)rows, ref, ref_lse, 0);
  CHECK(rc == 0, "oracle (MLA): %d", rc);
  void *dq = to_device(q, nq * 2), *dkv = to_device(kv, nkv * 2);
  void* dlens = to_device(lens, sizeof(lens));
  void *dout = NULL, *dlse = NULL, *dws = NULL;
  HIP_OK(hipMalloc(&dout, rows * Dv * 2));
  HIP_OK(hipMalloc(&dlse, rows * 4));
  uint16_t* out = (uint16_t*)malloc(rows * Dv * 2);
  float* lse = (float*)malloc(rows * 4);
  for (int P = 1; P <= 3; P += 2) {
    size_t wsb = decode_workspace_size(P, B, T, H, Dv);
    HIP_OK(hipMalloc(&dws, wsb));
    HIP_OK(hipMemset(dws, 0, wsb));
    rc = mla_decode(dq, dkv, NULL, 0, 0, (const uint32_t*)dlens, B, T, H, S, scale, P, NULL,
                    DA_MASK_CAUSAL, dout, (float*)dlse, dws, wsb, NULL);
    CHECK(rc == DA_OK, "mla_decode P=%d: %s", P, decode_attention_status_string(rc));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(out, dout, rows * Dv * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse, dlse, rows * 4, hipMemcpyDeviceToHost));
    char what[64];
    snprintf(what, sizeof what, "MLA causal MTP (T=2), P=%d", P);
    compare(what, out, lse, ref, ref_lse, rows, Dv);
    HIP_OK(hipFree(dws));
  }
  hipFree(dq); hipFree(dkv); hipFree(dlens); hipFree(dout); hipFree(dlse);
  free(q); free(kv); free(ref); free(ref_lse); free(out); free(lse);
}

int main(int argc, char** argv) {
  lcg_state = 20260601ull;
  const int gpu = argc > 1 && strcmp(argv[1], "gpu") == 0;
  host_checks();
  if (gpu) {
    HIP_OK(hipSetDevice(0));
    gqa_case();
    mla_case();
  }
  printf("%s\n", failures ? "FAILED" : "PASSED");
  return failures ? 1 : 0;
}
