/*
 * Exercises every oracle function on ragged, seeded inputs so that the
 * oracle can be run under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitized.py builds and runs it).  Exits 0 when every
 * call returned and every output is finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ULL;

static double uniform(void) { /* xorshift64*, enough for test inputs */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 0x2545F4914F6CDD1DULL) >> 11) * 0x1p-53;
}

static float* vec(int64_t n, double scale, int positive) {
  float* p = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i)
    p[i] = (float)(positive ? 1e-8 + scale * uniform() : scale * (uniform() - 0.5));
  return p;
}

static int finite_all(const float* p, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static int run_table(const int64_t* numels, int32_t L, int32_t C, int32_t W) {
  int64_t N = 0;
  for (int32_t l = 0; l < L; ++l) N += numels[l];
  const int64_t K = (N + C - 1) / C;
  oracle_hparams hp = {0.9f, 0.999f, 1e-8f, 1e-3f, 0.0f, 0.01f, 10.0f, 0.5f, 4.0f, 0.1f, 0, 0.0f, 0};
  float *x = vec(N, 0.04, 0), *m = vec(N, 0.0, 0), *v = vec(N, 0.0, 0), *vf = vec(N, 0.0, 0);
  float* err_s = vec(N, 0.0, 0);
  float** g = (float**)malloc(sizeof(float*) * (size_t)W);
  float** e = (float**)malloc(sizeof(float*) * (size_t)W);
  uint32_t** bw = (uint32_t**)malloc(sizeof(uint32_t*) * (size_t)W);
  float** sw = (float**)malloc(sizeof(float*) * (size_t)W);
  for (int32_t w = 0; w < W; ++w) {
    g[w] = vec(N, 0.04, 0);
    e[w] = vec(N, 0.0, 0);
    bw[w] = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(K * C / 32));
    sw[w] = (float*)malloc(sizeof(float) * (size_t)K);
  }
  uint32_t* bs = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(K * C / 32));
  float* ss = (float*)malloc(sizeof(float) * (size_t)K);
  float *c_sum = vec(L, 0.0, 0), *c_out = vec(L, 0.0, 0), *c_avg = vec(L, 0.0, 0), *f_prev = vec(L, 0.0, 0);
  int ok = 1;
  for (int t = 1; t <= 3; ++t) {
    hp.bias_step = t;
    hp.weight_decay = 0.01f;
    hp.c_avg_decay = 0.9f;
    oracle_warmup_step(L, numels, W, (const float* const*)g, x, m, v, c_sum, c_out, &hp);
  }
  hp.bias_step = 0;
  oracle_freeze(L, N, W, v, vf, e, err_s, c_sum, 3, c_avg, f_prev, &hp);
  for (int r = 0; r < 2; ++r) {
    hp.rho_mode = r;
    oracle_compressed_step(L, numels, C, W, (const float* const*)g, e, err_s, x, m, v, vf, c_avg,
                           f_prev, c_out, bw, sw, bs, ss, &hp, ORACLE_ONEBIT);
    oracle_compressed_step(L, numels, C, W, (const float* const*)g, e, err_s, x, m, v, vf, c_avg,
                           f_prev, NULL, NULL, NULL, NULL, NULL, &hp, ORACLE_IDENTITY);
  }
  ok &= finite_all(x, N) && finite_all(m, N) && finite_all(vf, N) && finite_all(ss, K);
  /* codec pieces */
  float* out = vec(N, 0.0, 0);
  float scratch_in[1];
  (void)scratch_in;
  oracle_compress_ef(N, C, x, err_s, bs, ss);
  oracle_average_packed(N, C, W, (const uint32_t* const*)bw, (const float* const*)sw, err_s, bs, ss);
  oracle_average(N, C, W, (const uint32_t* const*)bw, (const float* const*)sw, out);
  oracle_decompress(N, C, bs, ss, out);
  ok &= finite_all(out, N);
  /* 1-bit Adam */
  hp.weight_decay = 0.0f;
  hp.bias_step = 1;
  oracle_adam_warmup_step(N, W, (const float* const*)g, x, m, v, &hp);
  hp.bias_step = 0;
  oracle_adam_compressed_step(N, C, W, (const float* const*)g, e, err_s, x, m, v, bw, sw, bs, ss,
                              &hp, ORACLE_ONEBIT);
  oracle_adam_compressed_step(N, C, W, (const float* const*)g, e, err_s, x, m, v, NULL, NULL, NULL,
                              NULL, &hp, ORACLE_IDENTITY);
  ok &= finite_all(x, N);
  /* sparse stage */
  const int32_t nb = C / 64;
  for (int32_t nsel = 1; nsel <= nb; nsel += nb - 1) {
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    for (int64_t k = 0; k < K; ++k) sel[k] = (int32_t)(uniform() * nb);
    float** vw = (float**)malloc(sizeof(float*) * (size_t)W);
    for (int32_t w = 0; w < W; ++w) vw[w] = (float*)malloc(sizeof(float) * (size_t)(K * nsel * 64));
    float* vs = (float*)malloc(sizeof(float) * (size_t)(K * nsel * 64));
    oracle_sparse_step(L, numels, C, W, nsel, sel, (const float* const*)g, e, x, m, v, vf, c_avg,
                       vw, vs, &hp);
    ok &= finite_all(vs, K * nsel * 64) && finite_all(x, N);
    for (int32_t w = 0; w < W; ++w) free(vw[w]);
    free(vw);
    free(vs);
    free(sel);
  }
  /* chunk scale on its own */
  float* tmp = (float*)malloc(sizeof(float) * (size_t)C);
  ok &= isfinite(oracle_chunk_scale(x, N < C ? N : C, C, tmp));
  free(tmp);
  for (int32_t w = 0; w < W; ++w) {
    free(g[w]);
    free(e[w]);
    free(bw[w]);
    free(sw[w]);
  }
  free(g); free(e); free(bw); free(sw); free(bs); free(ss);
  free(x); free(m); free(v); free(vf); free(err_s); free(out);
  free(c_sum); free(c_out); free(c_avg); free(f_prev);
  return ok;
}

int main(void) {
  const int64_t t1[] = {1};
  const int64_t t2[] = {10, 20, 30};
  const int64_t t3[] = {1, 3, 4095, 4097, 100, 8192, 17};
  const int64_t t4[] = {1024 * 3};
  int ok = 1;
  for (int32_t C = 1024; C <= 4096; C *= 4) {
    ok &= run_table(t1, 1, C, 1);
    ok &= run_table(t2, 3, C, 3);
    ok &= run_table(t3, 7, C, 4);
    ok &= run_table(t4, 1, C, 2);
  }
  if (!ok) {
    fprintf(stderr, "oracle driver: a non-finite output\n");
    return 1;
  }
  printf("oracle driver ok\n");
  return 0;
}
