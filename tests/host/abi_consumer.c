/*
 * abi_consumer.c -- a plain C99 program that drives libkda through include/kda.h
 * only (no Python, no C++), on one GPU.
 *
 * Inputs are synthetic (a 64-bit LCG; q and k unit-norm per (token, head),
 * v in (-1, 1), g in (-0.05, 0), beta in (0.2, 0.8)), rounded to bf16 with
 * round-to-nearest-even.  The program checks properties that need no
 * reference values:
 *   1. prefill of [0, 1024) with a checkpoint at 512, then a restore of that
 *      checkpoint into a fresh page and a resumed prefill of [512, 1024) from
 *      it: the resumed outputs and final state equal the uninterrupted ones
 *      bit for bit (page "Cache de préfixe hybride KDA–MLA", section
 *      "Le fonctionnement du prefill": a hit resumes from the stored state);
 *   2. a decode step in place and the same step into a fresh page from an
 *      equal state give equal outputs and states bit for bit;
 *   3. an invalid call (chunk size 32) returns KDA_ERR_SHAPE with a message
 *      and leaves the device untouched.
 * Exit status 0 and a line "abi_consumer: OK" on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda.h"

#define H 2
#define D 128
#define T 1024
#define B 512

#define CHECK_HIP(x)                                                      \
  do {                                                                    \
    hipError_t e_ = (x);                                                  \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
      exit(2);                                                            \
    }                                                                     \
  } while (0)
#define CHECK_KDA(x)                                                      \
  do {                                                                    \
    kda_status s_ = (x);                                                  \
    if (s_ != KDA_OK) {                                                   \
      fprintf(stderr, "kda status %d at %s:%d: %s\n", (int)s_, __FILE__, __LINE__, kda_last_error()); \
      exit(3);                                                            \
    }                                                                     \
  } while (0)

static uint64_t g_rng = 0x4B44412D41424931ull;
static double uni(void) { /* uniform in [0, 1) from a 64-bit LCG (Knuth's MMIX constants) */
  g_rng = g_rng * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(g_rng >> 11) * (1.0 / 9007199254740992.0);
}

static uint16_t to_bf16(float f) { /* round to nearest even; inputs here are finite */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void* dev_copy(const void* host, size_t n) {
  void* p = NULL;
  CHECK_HIP(hipMalloc(&p, n));
  CHECK_HIP(hipMemcpy(p, host, n, hipMemcpyHostToDevice));
  return p;
}

int main(void) {
  const size_t nv = (size_t)T * H * D;
  uint16_t* hq = malloc(nv * 2);
  uint16_t* hk = malloc(nv * 2);
  uint16_t* hv = malloc(nv * 2);
  uint16_t* hg = malloc(nv * 2);
  uint16_t* hb = malloc((size_t)T * H * 2);
  if (!hq || !hk || !hv || !hg || !hb) return 4;
  for (size_t r = 0; r < (size_t)T * H; ++r) {
    double q[D], k[D], nq = 0.0, nk = 0.0;
    for (int c = 0; c < D; ++c) {
      q[c] = uni() - 0.5;
      k[c] = uni() - 0.5;
      nq += q[c] * q[c];
      nk += k[c] * k[c];
    }
    for (int c = 0; c < D; ++c) {
      hq[r * D + c] = to_bf16((float)(q[c] / sqrt(nq)));
      hk[r * D + c] = to_bf16((float)(k[c] / sqrt(nk)));
      hv[r * D + c] = to_bf16((float)(2.0 * uni() - 1.0));
      hg[r * D + c] = to_bf16((float)(-0.05 * uni()));
    }
    hb[r] = to_bf16((float)(0.2 + 0.6 * uni()));
  }
  void* q = dev_copy(hq, nv * 2);
  void* k = dev_copy(hk, nv * 2);
  void* v = dev_copy(hv, nv * 2);
  void* g = dev_copy(hg, nv * 2);
  void* beta = dev_copy(hb, (size_t)T * H * 2);

  /* pages: 0 final (uninterrupted), 1 checkpoint at B, 2 restored, 3 final (resumed), 4 decode copy */
  kda_pool pool;
  pool.page_bytes = (int64_t)H * D * D * 4;
  pool.num_pages = 5;
  pool.num_heads = H;
  pool.d_k = D;
  pool.d_v = D;
  CHECK_HIP(hipMalloc(&pool.base, (size_t)pool.page_bytes * pool.num_pages));
  CHECK_HIP(hipMemset(pool.base, 0, (size_t)pool.page_bytes * pool.num_pages));
  CHECK_KDA(kda_pool_check(&pool));

  void *o_a = NULL, *o_b = NULL;
  CHECK_HIP(hipMalloc(&o_a, nv * 2));
  CHECK_HIP(hipMalloc(&o_b, nv * 2));
  const size_t wsb = kda_prefill_workspace_bytes(&pool, T, 1, 1, KDA_BF16);
  if (wsb == 0) return 5;
  void* ws = NULL;
  CHECK_HIP(hipMalloc(&ws, wsb));

  /* 1. uninterrupted [0, T) with a checkpoint at B */
  const int64_t cu_a[2] = {0, T};
  const int32_t out_a[1] = {0}, ck_cu[2] = {0, 1}, ck_page[1] = {1};
  const int64_t ck_pos[1] = {B};
  CHECK_KDA(kda_prefill_chunked(&pool, q, k, v, g, beta, KDA_BF16, o_a, KDA_BF16, 1, cu_a, NULL, NULL,
                                out_a, ck_cu, ck_pos, ck_page, 64, 512, ws, wsb, NULL));
  /* restore the checkpoint into a fresh page, resume [B, T) from it */
  const int32_t src[1] = {1}, dst[1] = {2};
  CHECK_KDA(kda_checkpoint_restore(&pool, src, dst, 1, NULL));
  const int64_t cu_b[2] = {0, T - B}, sp_b[1] = {B};
  const int32_t in_b[1] = {2}, out_b[1] = {3};
  const size_t off = (size_t)B * H * D * 2;
  CHECK_KDA(kda_prefill_chunked(&pool, (const char*)q + off, (const char*)k + off, (const char*)v + off,
                                (const char*)g + off, (const char*)beta + (size_t)B * H * 2, KDA_BF16,
                                o_b, KDA_BF16, 1, cu_b, sp_b, in_b, out_b, NULL, NULL, NULL, 64, 512, ws,
                                wsb, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  const size_t half = (size_t)(T - B) * H * D * 2;
  unsigned char* ha = malloc(half);
  unsigned char* hbuf = malloc(half);
  CHECK_HIP(hipMemcpy(ha, (const char*)o_a + off, half, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hbuf, o_b, half, hipMemcpyDeviceToHost));
  if (memcmp(ha, hbuf, half) != 0) {
    fprintf(stderr, "resumed outputs differ from the uninterrupted run\n");
    return 6;
  }
  const size_t sb = (size_t)pool.page_bytes;
  unsigned char* s0 = malloc(sb);
  unsigned char* s3 = malloc(sb);
  CHECK_HIP(hipMemcpy(s0, (const char*)pool.base + 0 * sb, sb, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(s3, (const char*)pool.base + 3 * sb, sb, hipMemcpyDeviceToHost));
  if (memcmp(s0, s3, sb) != 0) {
    fprintf(stderr, "resumed final state differs from the uninterrupted one\n");
    return 7;
  }
  int finite = 1;
  for (size_t i = 0; i < sb / 4; ++i) {
    float f;
    memcpy(&f, s0 + 4 * i, 4);
    if (!isfinite(f)) finite = 0;
  }
  if (!finite) {
    fprintf(stderr, "non-finite final state\n");
    return 8;
  }

  /* 2. decode: page 0 in place, page 3 (equal state) into page 4 */
  int32_t hp_in[2] = {0, 3}, hp_out[2] = {0, 4};
  int32_t *p_in = NULL, *p_out = NULL;
  CHECK_HIP(hipMalloc((void**)&p_in, sizeof(hp_in)));
  CHECK_HIP(hipMalloc((void**)&p_out, sizeof(hp_out)));
  CHECK_HIP(hipMemcpy(p_in, hp_in, sizeof(hp_in), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(p_out, hp_out, sizeof(hp_out), hipMemcpyHostToDevice));
  /* both requests take the same token: rows 0 and 1 of a 2-request batch hold token 0's inputs twice */
  const size_t tok = (size_t)H * D * 2;
  void *dq = NULL, *dk = NULL, *dv = NULL, *dg = NULL, *db = NULL, *od = NULL;
  CHECK_HIP(hipMalloc(&dq, 2 * tok));
  CHECK_HIP(hipMalloc(&dk, 2 * tok));
  CHECK_HIP(hipMalloc(&dv, 2 * tok));
  CHECK_HIP(hipMalloc(&dg, 2 * tok));
  CHECK_HIP(hipMalloc(&db, 2 * H * 2));
  CHECK_HIP(hipMalloc(&od, 2 * tok));
  for (int r = 0; r < 2; ++r) {
    CHECK_HIP(hipMemcpy((char*)dq + r * tok, hq, tok, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy((char*)dk + r * tok, hk, tok, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy((char*)dv + r * tok, hv, tok, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy((char*)dg + r * tok, hg, tok, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy((char*)db + r * H * 2, hb, H * 2, hipMemcpyHostToDevice));
  }
  CHECK_KDA(kda_decode_step(&pool, dq, dk, dv, dg, db, KDA_BF16, od, KDA_BF16, 2, p_in, p_out, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  unsigned char* ho = malloc(2 * tok);
  CHECK_HIP(hipMemcpy(ho, od, 2 * tok, hipMemcpyDeviceToHost));
  if (memcmp(ho, ho + tok, tok) != 0) {
    fprintf(stderr, "decode outputs differ between in-place and fresh-page requests\n");
    return 9;
  }
  CHECK_HIP(hipMemcpy(s0, (const char*)pool.base + 0 * sb, sb, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(s3, (const char*)pool.base + 4 * sb, sb, hipMemcpyDeviceToHost));
  if (memcmp(s0, s3, sb) != 0) {
    fprintf(stderr, "decode states differ between in-place and fresh-page requests\n");
    return 10;
  }

  /* 3. an invalid call is rejected before anything runs */
  kda_status st = kda_prefill_chunked(&pool, q, k, v, g, beta, KDA_BF16, o_a, KDA_BF16, 1, cu_a, NULL,
                                      NULL, out_a, NULL, NULL, NULL, 32, 512, ws, wsb, NULL);
  if (st != KDA_ERR_SHAPE || kda_last_error()[0] == '\0') {
    fprintf(stderr, "chunk size 32 gave status %d (%s)\n", (int)st, kda_last_error());
    return 11;
  }

  printf("abi_consumer: OK (resume bitwise, restore, in-place decode, rejection; library version %d.%d)\n",
         (int)(kda_version() >> 16), (int)(kda_version() & 0xffff));
  return 0;
}
