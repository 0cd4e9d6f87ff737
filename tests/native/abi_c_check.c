/*
 * The C ABI of libonebit.so used from plain C, without Python: a caller that
 * has only include/onebit.h and the HIP runtime.  It builds a ragged layer
 * table, runs two 1-bit LAMB compression-stage steps and one 1-bit Adam
 * compression step on the GPU through the C entry points, runs the CPU
 * oracle on the same seeded inputs, and compares every output bit for bit
 * (this stage has no order-dependent sum, so x and c are exact too).  Then
 * it runs one more LAMB step as W simulated GPUs would, through the per-GPU
 * entry points (each worker's compression, each GPU's chunk range as server,
 * one replica's statistics and update), and checks it against the fused
 * step on a copy of the state; then one step through the allocation-free
 * entry point against the fused step with a workspace, and three warmup
 * steps with the parameters' squared norm carried against three that read
 * x.  It also checks a few argument errors.
 * Test infrastructure: it links the library, the oracle and the host input
 * generator; prints PASS and returns 0, or names the first mismatch and
 * returns 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "onebit.h"
#include "oracle.h"

void synth_fill_normal(uint64_t seed, uint64_t stream, int64_t offset, int64_t n, double mean,
                       double std, float* out);
void synth_fill_uniform(uint64_t seed, uint64_t stream, int64_t offset, int64_t n, double lo,
                        double hi, float* out);

#define L_TENSORS 5
#define W 3
#define C 4096
#define STEPS 2

static int failures = 0;

static void hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    printf("abi_c_check: %s: %s\n", what, hipGetErrorString(e));
    fflush(stdout);
    exit(2);
  }
}

static void rc_ok(int rc, const char* what) {
  if (rc != ONEBIT_OK) {
    printf("abi_c_check: %s returned %d: %s\n", what, rc, onebit_last_error());
    fflush(stdout);
    exit(2);
  }
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  hip_ok(hipMalloc(&p, bytes ? bytes : 16), "hipMalloc");
  hip_ok(hipMemset(p, 0, bytes ? bytes : 16), "hipMemset");
  return p;
}

static void up(void* d, const void* h, size_t bytes) {
  hip_ok(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice), "hipMemcpy H2D");
}

static void* down(const void* d, size_t bytes) {
  void* h = malloc(bytes);
  hip_ok(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost), "hipMemcpy D2H");
  return h;
}

/* Bitwise comparison of a device array with the expected host copy. */
static void same(const char* name, const void* d, const void* h, size_t bytes) {
  void* g = down(d, bytes);
  if (memcmp(g, h, bytes) != 0) {
    const uint32_t* a = (const uint32_t*)g;
    const uint32_t* b = (const uint32_t*)h;
    size_t i = 0;
    while (i < bytes / 4 && a[i] == b[i]) ++i;
    printf("abi_c_check: %s differs at word %zu (got 0x%08x, expected 0x%08x)\n", name, i, a[i],
           b[i]);
    ++failures;
  }
  free(g);
}

static uint64_t stream_id(uint64_t array, uint64_t step, uint64_t worker) {
  return (array << 40) | (step << 20) | worker;
}

int main(void) {
  const int64_t numels[L_TENSORS] = {3 * C + 100, 1, 777, 2 * C, 5};
  int64_t N = 0;
  for (int l = 0; l < L_TENSORS; ++l) N += numels[l];
  const int64_t K = (N + C - 1) / C, words = K * C / 32;
  const size_t fb = (size_t)N * 4, wb = (size_t)words * 4, sb = (size_t)K * 4,
               lb = (size_t)L_TENSORS * 4;

  onebit_hparams hp;
  memset(&hp, 0, sizeof hp);
  hp.beta1 = 0.9f; hp.beta2 = 0.999f; hp.eta = 1e-8f; hp.lr = 1e-3f;
  hp.c_min = 0.01f; hp.c_max = 10.0f; hp.f_min = 0.5f; hp.f_max = 4.0f; hp.kappa = 0.1f;
  oracle_hparams ohp;
  memset(&ohp, 0, sizeof ohp);
  ohp.beta1 = hp.beta1; ohp.beta2 = hp.beta2; ohp.eta = hp.eta; ohp.lr = hp.lr;
  ohp.c_min = hp.c_min; ohp.c_max = hp.c_max; ohp.f_min = hp.f_min; ohp.f_max = hp.f_max;
  ohp.kappa = hp.kappa;

  /* host state: x ~ N(0, 0.02), m ~ N(0, 1e-3), v_frozen = v_fresh ~ U(1e-8, 1e-4) */
  float *x = malloc(fb), *m = malloc(fb), *vz = malloc(fb), *vf = malloc(fb), *es = calloc(N, 4);
  float *g[W], *e[W];
  synth_fill_normal(0, stream_id(1, 0, 0), 0, N, 0.0, 0.02, x);
  synth_fill_normal(0, stream_id(2, 0, 0), 0, N, 0.0, 1e-3, m);
  synth_fill_uniform(0, stream_id(3, 0, 0), 0, N, 1e-8, 1e-4, vz);
  memcpy(vf, vz, fb);
  float c_avg[L_TENSORS], f_prev[L_TENSORS], c_out[L_TENSORS];
  for (int l = 0; l < L_TENSORS; ++l) { c_avg[l] = 1.0f; f_prev[l] = 1.0f; c_out[l] = 0.0f; }
  uint32_t *bw[W], *bs = malloc(wb);
  float *sw[W], *ss = malloc(sb);

  /* device state, same values */
  onebit_layer_table* table = NULL;
  rc_ok(onebit_layer_table_create(numels, L_TENSORS, C, &table), "onebit_layer_table_create");
  int64_t tN = 0, tK = 0, tS = 0;
  rc_ok(onebit_layer_table_info(table, &tN, &tK, &tS), "onebit_layer_table_info");
  if (tN != N || tK != K) { printf("abi_c_check: table info %lld %lld\n", (long long)tN, (long long)tK); return 1; }
  size_t wsb = 0;
  rc_ok(onebit_workspace_size(table, W, &wsb), "onebit_workspace_size");
  float *dx = dev_alloc(fb), *dm = dev_alloc(fb), *dvz = dev_alloc(fb), *dvf = dev_alloc(fb),
        *des = dev_alloc(fb);
  float *dg[W], *de[W], *dsw[W];
  uint32_t* dbw[W];
  for (int w = 0; w < W; ++w) {
    g[w] = malloc(fb); e[w] = calloc(N, 4); bw[w] = malloc(wb); sw[w] = malloc(sb);
    dg[w] = dev_alloc(fb); de[w] = dev_alloc(fb); dbw[w] = dev_alloc(wb); dsw[w] = dev_alloc(sb);
  }
  uint32_t* dbs = dev_alloc(wb);
  float *dss = dev_alloc(sb), *dcavg = dev_alloc(lb), *dfprev = dev_alloc(lb), *dcout = dev_alloc(lb);
  void* dws = dev_alloc(wsb);
  int32_t* dstatus = dev_alloc(4);
  up(dx, x, fb); up(dm, m, fb); up(dvz, vz, fb); up(dvf, vf, fb);
  up(dcavg, c_avg, lb); up(dfprev, f_prev, lb);

  for (int step = 0; step < STEPS; ++step) {
    for (int w = 0; w < W; ++w) {
      synth_fill_normal(0, stream_id(4, (uint64_t)step, (uint64_t)w), 0, N, 0.0, 1e-3, g[w]);
      up(dg[w], g[w], fb);
    }
    rc_ok(onebit_lamb_compressed_step(table, W, (const float* const*)dg, de, des, dx, dm, dvz, dvf,
                                      dcavg, dfprev, dcout, dbw, dsw, dbs, dss, &hp, dws, dstatus,
                                      NULL),
          "onebit_lamb_compressed_step");
    oracle_compressed_step(L_TENSORS, numels, C, W, (const float* const*)g, e, es, x, m, vz, vf,
                           c_avg, f_prev, c_out, bw, sw, bs, ss, &ohp, ORACLE_ONEBIT);
    hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize");
    char name[64];
    same("x", dx, x, fb); same("m", dm, m, fb); same("v_fresh", dvf, vf, fb);
    same("err_s", des, es, fb); same("bits_s", dbs, bs, wb); same("scales_s", dss, ss, sb);
    same("f_prev", dfprev, f_prev, lb); same("c", dcout, c_out, lb);
    for (int w = 0; w < W; ++w) {
      snprintf(name, sizeof name, "err_w[%d]", w); same(name, de[w], e[w], fb);
      snprintf(name, sizeof name, "bits_w[%d]", w); same(name, dbw[w], bw[w], wb);
      snprintf(name, sizeof name, "scales_w[%d]", w); same(name, dsw[w], sw[w], sb);
    }
  }

  /* 1-bit Adam on the same buffers, flat (no layer table) */
  for (int w = 0; w < W; ++w) {
    synth_fill_normal(0, stream_id(4, 7, (uint64_t)w), 0, N, 0.0, 1e-3, g[w]);
    up(dg[w], g[w], fb);
  }
  rc_ok(onebit_adam_compressed_step(N, C, W, (const float* const*)dg, de, des, dx, dm, dvz, dbw,
                                    dsw, dbs, dss, &hp, dstatus, NULL),
        "onebit_adam_compressed_step");
  oracle_adam_compressed_step(N, C, W, (const float* const*)g, e, es, x, m, vz, bw, sw, bs, ss, &ohp,
                              ORACLE_ONEBIT);
  hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize");
  same("adam x", dx, x, fb); same("adam m", dm, m, fb); same("adam err_s", des, es, fb);
  same("adam bits_s", dbs, bs, wb); same("adam scales_s", dss, ss, sb);

  /* one GPU's share, W simulated GPUs: the same step through the per-GPU
   * entry points on copies of the state, against the fused step */
  {
    float *sx = dev_alloc(fb), *sm = dev_alloc(fb), *svf = dev_alloc(fb), *ses = dev_alloc(fb),
          *sfp = dev_alloc(lb), *sco = dev_alloc(lb), *se[W], *ssw[W], *sss = dev_alloc(sb);
    uint32_t *sbw[W], *sbs = dev_alloc(wb);
    void* sws = dev_alloc(wsb);
    hip_ok(hipMemcpy(sx, dx, fb, hipMemcpyDeviceToDevice), "copy");
    hip_ok(hipMemcpy(sm, dm, fb, hipMemcpyDeviceToDevice), "copy");
    hip_ok(hipMemcpy(svf, dvf, fb, hipMemcpyDeviceToDevice), "copy");
    hip_ok(hipMemcpy(ses, des, fb, hipMemcpyDeviceToDevice), "copy");
    hip_ok(hipMemcpy(sfp, dfprev, lb, hipMemcpyDeviceToDevice), "copy");
    for (int w = 0; w < W; ++w) {
      se[w] = dev_alloc(fb); sbw[w] = dev_alloc(wb); ssw[w] = dev_alloc(sb);
      hip_ok(hipMemcpy(se[w], de[w], fb, hipMemcpyDeviceToDevice), "copy");
      synth_fill_normal(0, stream_id(4, 9, (uint64_t)w), 0, N, 0.0, 1e-3, g[w]);
      up(dg[w], g[w], fb);
    }
    /* the fused step on the original state */
    rc_ok(onebit_lamb_compressed_step(table, W, (const float* const*)dg, de, des, dx, dm, dvz, dvf,
                                      dcavg, dfprev, dcout, dbw, dsw, dbs, dss, &hp, dws, dstatus,
                                      NULL),
          "onebit_lamb_compressed_step (fused)");
    /* 1. every GPU compresses its own worker's momentum */
    for (int w = 0; w < W; ++w)
      rc_ok(onebit_worker_compress(N, C, dg[w], se[w], sm, NULL, NULL, sbw[w], ssw[w], &hp, dstatus,
                                   NULL),
            "onebit_worker_compress");
    /* 3. GPU p serves chunks [K*p/W, K*(p+1)/W) */
    for (int p = 0; p < W; ++p) {
      const int64_t k0 = K * p / W, k1 = K * (p + 1) / W;
      if (k1 == k0) continue;
      const int64_t lo = k0 * C, hi = k1 * C < N ? k1 * C : N;
      const uint32_t* rb[W];
      const float* rs[W];
      for (int w = 0; w < W; ++w) { rb[w] = sbw[w] + k0 * C / 32; rs[w] = ssw[w] + k0; }
      rc_ok(onebit_average_packed(hi - lo, C, W, rb, rs, ses + lo, sbs + k0 * C / 32, sss + k0,
                                  dstatus, NULL),
            "onebit_average_packed (range)");
    }
    /* 5. one replica: statistics, then the update */
    rc_ok(onebit_lamb_rescale_stats(table, sbs, sss, sm, NULL, NULL, dvz, svf, &hp, sws, NULL),
          "onebit_lamb_rescale_stats");
    rc_ok(onebit_lamb_rescale_update(table, sbs, sss, sx, sm, dvz, dcavg, sfp, sco, &hp, sws,
                                     dstatus, NULL),
          "onebit_lamb_rescale_update");
    hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize");
    void* h;
#define SAME_DEV(name, a, b, bytes)                     \
    h = down(b, bytes);                                 \
    same(name, a, h, bytes);                            \
    free(h)
    SAME_DEV("share x", sx, dx, fb); SAME_DEV("share m", sm, dm, fb);
    SAME_DEV("share v_fresh", svf, dvf, fb); SAME_DEV("share err_s", ses, des, fb);
    SAME_DEV("share bits_s", sbs, dbs, wb); SAME_DEV("share scales_s", sss, dss, sb);
    SAME_DEV("share f_prev", sfp, dfprev, lb); SAME_DEV("share c", sco, dcout, lb);
    for (int w = 0; w < W; ++w) {
      SAME_DEV("share err_w", se[w], de[w], fb); SAME_DEV("share bits_w", sbw[w], dbw[w], wb);
    }
#undef SAME_DEV
  }

  /* the allocation-free step on a copy of the state, against the fused step
   * with a workspace on the original */
  {
    float *ax = dev_alloc(fb), *am = dev_alloc(fb), *avf = dev_alloc(fb), *aes = dev_alloc(fb),
          *afp = dev_alloc(lb), *aco = dev_alloc(lb), *ae[W], *asw[W], *ass = dev_alloc(sb);
    uint32_t *abw[W], *abs_ = dev_alloc(wb);
    hip_ok(hipMemcpy(ax, dx, fb, hipMemcpyDeviceToDevice), "copy");
    hip_ok(hipMemcpy(am, dm, fb, hipMemcpyDeviceToDevice), "copy");
    hip_ok(hipMemcpy(avf, dvf, fb, hipMemcpyDeviceToDevice), "copy");
    hip_ok(hipMemcpy(aes, des, fb, hipMemcpyDeviceToDevice), "copy");
    hip_ok(hipMemcpy(afp, dfprev, lb, hipMemcpyDeviceToDevice), "copy");
    for (int w = 0; w < W; ++w) {
      ae[w] = dev_alloc(fb); abw[w] = dev_alloc(wb); asw[w] = dev_alloc(sb);
      hip_ok(hipMemcpy(ae[w], de[w], fb, hipMemcpyDeviceToDevice), "copy");
      synth_fill_normal(0, stream_id(4, 11, (uint64_t)w), 0, N, 0.0, 1e-3, g[w]);
      up(dg[w], g[w], fb);
    }
    rc_ok(onebit_lamb_compressed_step(table, W, (const float* const*)dg, de, des, dx, dm, dvz, dvf,
                                      dcavg, dfprev, dcout, dbw, dsw, dbs, dss, &hp, dws, dstatus,
                                      NULL),
          "onebit_lamb_compressed_step (workspace)");
    rc_ok(onebit_lamb_compressed_step_noalloc(table, W, (const float* const*)dg, ae, aes, ax, am,
                                              dvz, avf, dcavg, afp, aco, abw, asw, abs_, ass, &hp,
                                              dstatus, NULL),
          "onebit_lamb_compressed_step_noalloc");
    hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize");
    void* h;
#define SAME_DEV(name, a, b, bytes)                     \
    h = down(b, bytes);                                 \
    same(name, a, h, bytes);                            \
    free(h)
    SAME_DEV("noalloc x", ax, dx, fb); SAME_DEV("noalloc m", am, dm, fb);
    SAME_DEV("noalloc v_fresh", avf, dvf, fb); SAME_DEV("noalloc err_s", aes, des, fb);
    SAME_DEV("noalloc bits_s", abs_, dbs, wb); SAME_DEV("noalloc scales_s", ass, dss, sb);
    SAME_DEV("noalloc f_prev", afp, dfprev, lb); SAME_DEV("noalloc c", aco, dcout, lb);
    for (int w = 0; w < W; ++w) {
      SAME_DEV("noalloc err_w", ae[w], de[w], fb); SAME_DEV("noalloc bits_w", abw[w], dbw[w], wb);
    }
  }

  /* the warmup with the parameters' squared norm carried between steps,
   * against the warmup that reads x every step: three steps from m = v = 0 */
  {
    float *wx = dev_alloc(fb), *wm = dev_alloc(fb), *wv = dev_alloc(fb), *wcs = dev_alloc(lb),
          *wco = dev_alloc(lb);
    float *qx = dev_alloc(fb), *qm = dev_alloc(fb), *qv = dev_alloc(fb), *qcs = dev_alloc(lb),
          *qco = dev_alloc(lb);
    double* x_sq = dev_alloc((size_t)tS * 8);
    up(wx, x, fb);
    up(qx, x, fb);
    for (int step = 0; step < 3; ++step) {
      for (int w = 0; w < W; ++w) {
        synth_fill_normal(0, stream_id(4, 20 + (uint64_t)step, (uint64_t)w), 0, N, 0.0, 0.02, g[w]);
        up(dg[w], g[w], fb);
      }
      rc_ok(onebit_lamb_warmup_step(table, W, (const float* const*)dg, wx, wm, wv, wcs, wco, &hp,
                                    dws, dstatus, NULL),
            "onebit_lamb_warmup_step");
      rc_ok(onebit_lamb_warmup_step_carry(table, W, (const float* const*)dg, qx, qm, qv, qcs, qco,
                                          x_sq, step > 0, &hp, dws, dstatus, NULL),
            "onebit_lamb_warmup_step_carry");
    }
    hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize");
    void* h;
    SAME_DEV("carry x", qx, wx, fb); SAME_DEV("carry m", qm, wm, fb);
    SAME_DEV("carry v", qv, wv, fb); SAME_DEV("carry c_sum", qcs, wcs, lb);
    SAME_DEV("carry c", qco, wco, lb);
#undef SAME_DEV
  }

  int32_t status = -1;
  hip_ok(hipMemcpy(&status, dstatus, 4, hipMemcpyDeviceToHost), "status");
  if (status != 0) { printf("abi_c_check: status %d\n", status); ++failures; }

  /* argument errors come back as codes, before anything is enqueued */
  if (onebit_compress_ef(N, C, (const float*)((char*)dx + 4), des, dbs, dss, NULL, NULL) !=
      ONEBIT_EALIGN) { printf("abi_c_check: misaligned input not rejected\n"); ++failures; }
  if (onebit_compress_ef(N, 3000, dx, des, dbs, dss, NULL, NULL) != ONEBIT_EUNSUPPORTED) {
    printf("abi_c_check: chunk 3000 not rejected\n"); ++failures;
  }
  if (onebit_lamb_compressed_step(table, 17, (const float* const*)dg, de, des, dx, dm, dvz, dvf,
                                  dcavg, dfprev, dcout, NULL, NULL, dbs, dss, &hp, dws, NULL,
                                  NULL) != ONEBIT_EUNSUPPORTED) {
    printf("abi_c_check: W = 17 not rejected\n"); ++failures;
  }
  if (onebit_last_error()[0] == '\0') { printf("abi_c_check: empty error message\n"); ++failures; }

  rc_ok(onebit_layer_table_destroy(table), "onebit_layer_table_destroy");
  printf("abi_c_check: %s (N = %lld, K = %lld, W = %d, %d LAMB steps, one Adam step, one "
         "LAMB step through the per-GPU entry points, one allocation-free step, three carried "
         "warmup steps)\n",
         failures ? "FAIL" : "PASS", (long long)N, (long long)K, W, STEPS);
  return failures ? 1 : 0;
}
