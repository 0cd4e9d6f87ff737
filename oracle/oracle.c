/*
 * CPU oracle for the 1-bit LAMB step.  TEST INFRASTRUCTURE ONLY (see
 * oracle.h).  Plain single-threaded loops, no blocking, no fusion: each
 * function takes the steps in the order the method states them.
 *
 * Notation: (+) (-) (*) (/) are fp32 operations, rounded one at a time, in the
 * order the parentheses give.  a1 = 1-beta1, a2 = 1-beta2, kp = 1+kappa,
 * km = 1-kappa (each one fp32 operation).  The page text ("1-bit LAMB",
 * arXiv 2104.06069) names the symbols but its equations are missing; the
 * steps are the following readings of it.
 *
 * LAMB warmup step (Background on LAMB; footnotes 3 and 4):
 *   W1  gbar_i = ((g_0,i (+) g_1,i) (+) ...) (/) W     full-precision average
 *   W2  m_i = (beta1 (*) m_i) (+) (a1 (*) gbar_i)
 *   W3  v_i = (beta2 (*) v_i) (+) (a2 (*) (gbar_i (*) gbar_i))
 *   W4  u_i = m_i (/) (sqrt(v_i) (+) eta)               no bias correction
 *   W5  per tensor l: X = sum x_i^2, U = sum u_i^2 in double, sequential,
 *       over the parameters before this step's update;
 *       r = 1 if X == 0 or U == 0, else fp32(sqrt(X)/sqrt(U)) (double);
 *       c_l = min(max(r, c_min), c_max)   (clip of the whole ratio, fn 4);
 *       c_sum_l = c_sum_l (+) c_l
 *   W6  x_i = x_i (-) ((gamma (*) c_l) (*) u_i)
 *
 * Freeze (1-bit Adam's frozen variance, Related work): v stays as v_frozen;
 *   v_fresh = v; c_avg_l = c_sum_l (/) T_w; f_prev_l = 1; e_w = e_s = 0.
 *
 * Compression step (Introduction, Related work, Sections 4 and 5):
 *   C1  z_w,i = ((beta1 (*) m_i) (+) (a1 (*) g_w,i)) (+) e_w,i
 *       the worker's local momentum plus its previous compression error
 *   C2  s_w,k = sqrt(S) (/) sqrt((float) n_k), S = canonical pairwise tree
 *       of z^2 over the chunk's C slots, zero beyond n_k:
 *       t[j] = z_j (*) z_j; for h = C/2, C/4, ..., 1: t[j] = t[j] (+) t[j+h]
 *       (a norm-preserving scale: ||C[z]|| = ||z||)
 *   C3  bit = [z >= 0] (so +0 and -0 give +1), sigma = +-1
 *   C4  e_w,i = bit ? z (-) s : z (+) s          (e = z - C[z])
 *   C5  a_i = ((sigma_0 s_0 (+) sigma_1 s_1) (+) ...) (/) W ;  y_i = a_i (+) e_s,i
 *       the average step of the compressed allreduce
 *   C6  the average is recompressed with its own error buffer e_s by C2-C4
 *       before the scatter step: s', bits', e_s; mhat_i = sigma'_i s'_k
 *   C7  ghat_i = (mhat_i (-) (beta1 (*) m_i)) (/) a1     reconstructed gradient
 *   C8  vf_i = (beta2 (*) vf_i) (+) (a2 (*) (ghat_i (*) ghat_i))
 *   C9  q_i = (sqrt(v_frozen,i) (+) eta) (/) (sqrt(vf_i) (+) eta);
 *       rho_l = max over the tensor's elements of q_i (NaN if any q_i is
 *       NaN: a sign cannot encode an undefined value, so such a tensor has
 *       no defined factor; C10's fminf then drops it and f is clamped by
 *       f_max and kp (*) f_prev alone)
 *   C10 f = min(rho_l, f_max, kp (*) f_prev_l); f = max(f, f_min, km (*) f_prev_l);
 *       f_prev_l = f; c_l = c_avg_l (*) f          stabilized soft thresholds
 *   C11 x_i = x_i (-) ((gamma (*) c_l) (*) (mhat_i (/) (sqrt(v_frozen,i) (+) eta)));
 *       m_i = mhat_i
 *
 * Variant readings (each off by default; the page leaves these points open):
 *   bias correction (bias_step = t >= 1; Adam's, which the page does not
 *       mention): bc1 = fp32(1 - beta1^t), bc2 = fp32(1 - beta2^t), both
 *       evaluated in double from the fp32 betas;
 *       W4' u_i = (m_i (/) bc1) (/) (sqrt(v_i (/) bc2) (+) eta)
 *   weight decay (lambda != 0; footnote 3 omits it; LAMB's usual form):
 *       W4'' u_i = u_i (+) (lambda (*) x_i)  with x before the update, so it
 *       enters the trust ratio; in the compression stage
 *       C11' x_i = x_i (-) ((gamma (*) c_l) (*) ((mhat_i (/) (sqrt(v_frozen,i)
 *            (+) eta)) (+) (lambda (*) x_i)))
 *   EMA of the warmup coefficient (c_avg_decay = d in (0,1)):
 *       W5' c_sum_l = (d (*) c_sum_l) (+) ((1 (-) d) (*) c_l), and at the
 *       freeze c_avg_l = c_sum_l (/) fp32(1 - d^T_w) (double power)
 *   norm-ratio factor (rho_mode = 1):
 *       C9' Qz = sum (sqrt(v_frozen,i) (+) eta)^2, Qf = sum (sqrt(vf_i) (+) eta)^2
 *       in double, sequential; rho_l = 1 if either is 0, else
 *       fp32(sqrt(Qz)/sqrt(Qf)) (double)
 *
 * 1-bit Adam (the 1-bit Adam page's abstract; 1-bit LAMB's Related Work):
 *   warmup  W1-W4 (or W4' with bias correction) as above, then
 *           x_i = x_i (-) (gamma (*) u_i)  (plain Adam, no layerwise
 *           coefficient; weight decay is not part of this mode)
 *   compression  C1-C6 as above, then
 *           x_i = x_i (-) (gamma (*) (mhat_i (/) (sqrt(v_frozen,i) (+) eta)));
 *           m_i = mhat_i          (frozen variance, no rescale)
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int64_t num_chunks(int64_t n, int32_t C) { return (n + C - 1) / C; }

/* Bias-correction divisors of warmup step t (1 when t == 0). */
static float bias_divisor(float beta, int32_t t) {
  return t >= 1 ? (float)(1.0 - pow((double)beta, (double)t)) : 1.0f;
}

static void* xmalloc(size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p) abort();
  return p;
}

static int sign_bit(const uint32_t* bits, int32_t C, int64_t k, int64_t j) {
  const uint32_t word = bits[k * (C / 32) + j / 32];
  return (int)((word >> (j % 32)) & 1u);
}

/* C2 */
float oracle_chunk_scale(const float* z, int64_t n, int32_t C, float* t) {
  for (int64_t j = 0; j < C; ++j) t[j] = j < n ? z[j] * z[j] : 0.0f;
  for (int64_t h = C / 2; h >= 1; h /= 2)
    for (int64_t j = 0; j < h; ++j) t[j] = t[j] + t[j + h];
  return sqrtf(t[0]) / sqrtf((float)n);
}

/* C2-C4 applied to z, one chunk: writes the chunk's sign words, returns s,
 * and replaces z by the compression error. */
static float compress_chunk(float* z, int64_t n, int32_t C, uint32_t* words, float* scratch) {
  const float s = oracle_chunk_scale(z, n, C, scratch);
  for (int64_t q = 0; q < C / 32; ++q) words[q] = 0u;
  for (int64_t j = 0; j < n; ++j) {
    const int bit = z[j] >= 0.0f;
    if (bit) words[j / 32] |= 1u << (j % 32);
    z[j] = bit ? z[j] - s : z[j] + s;
  }
  return s;
}

void oracle_compress_ef(int64_t n, int32_t C, const float* in, float* err, uint32_t* bits,
                        float* scales) {
  float* z = (float*)xmalloc(sizeof(float) * (size_t)C);
  float* scratch = (float*)xmalloc(sizeof(float) * (size_t)C);
  const int64_t K = num_chunks(n, C);
  for (int64_t k = 0; k < K; ++k) {
    const int64_t base = k * C;
    const int64_t nk = n - base < C ? n - base : C;
    for (int64_t j = 0; j < nk; ++j) z[j] = in[base + j] + err[base + j];
    scales[k] = compress_chunk(z, nk, C, bits + k * (C / 32), scratch);
    for (int64_t j = 0; j < nk; ++j) err[base + j] = z[j];
  }
  free(z);
  free(scratch);
}

void oracle_decompress(int64_t n, int32_t C, const uint32_t* bits, const float* scales, float* out) {
  const int64_t K = num_chunks(n, C);
  for (int64_t k = 0; k < K; ++k) {
    const int64_t base = k * C;
    const int64_t nk = n - base < C ? n - base : C;
    for (int64_t j = 0; j < nk; ++j) out[base + j] = sign_bit(bits, C, k, j) ? scales[k] : -scales[k];
  }
}

/* C5, first half */
void oracle_average(int64_t n, int32_t C, int32_t W, const uint32_t* const* bits_w,
                    const float* const* scales_w, float* a) {
  const int64_t K = num_chunks(n, C);
  for (int64_t k = 0; k < K; ++k) {
    const int64_t base = k * C;
    const int64_t nk = n - base < C ? n - base : C;
    for (int64_t j = 0; j < nk; ++j) {
      float acc = sign_bit(bits_w[0], C, k, j) ? scales_w[0][k] : -scales_w[0][k];
      for (int32_t w = 1; w < W; ++w)
        acc = acc + (sign_bit(bits_w[w], C, k, j) ? scales_w[w][k] : -scales_w[w][k]);
      a[base + j] = acc / (float)W;
    }
  }
}

/* C5 second half and C6 */
void oracle_average_packed(int64_t n, int32_t C, int32_t W, const uint32_t* const* bits_w,
                           const float* const* scales_w, float* err_s, uint32_t* bits_out,
                           float* scales_out) {
  float* y = (float*)xmalloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  oracle_average(n, C, W, bits_w, scales_w, y);
  for (int64_t i = 0; i < n; ++i) y[i] = y[i] + err_s[i];
  float* scratch = (float*)xmalloc(sizeof(float) * (size_t)C);
  const int64_t K = num_chunks(n, C);
  for (int64_t k = 0; k < K; ++k) {
    const int64_t base = k * C;
    const int64_t nk = n - base < C ? n - base : C;
    scales_out[k] = compress_chunk(y + base, nk, C, bits_out + k * (C / 32), scratch);
    for (int64_t j = 0; j < nk; ++j) err_s[base + j] = y[base + j];
  }
  free(scratch);
  free(y);
}

void oracle_warmup_step(int32_t L, const int64_t* numels, int32_t W, const float* const* grads,
                        float* x, float* m, float* v, float* c_sum, float* c_out,
                        const oracle_hparams* hp) {
  const float a1 = 1.0f - hp->beta1;
  const float a2 = 1.0f - hp->beta2;
  int64_t N = 0;
  for (int32_t l = 0; l < L; ++l) N += numels[l];

  /* W1-W3 */
  for (int64_t i = 0; i < N; ++i) {
    float gsum = grads[0][i];
    for (int32_t w = 1; w < W; ++w) gsum = gsum + grads[w][i];
    const float gbar = gsum / (float)W;
    m[i] = (hp->beta1 * m[i]) + (a1 * gbar);
    v[i] = (hp->beta2 * v[i]) + (a2 * (gbar * gbar));
  }

  /* W4 (W4' and W4'' when enabled) */
  float* u = (float*)xmalloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
  const float bc1 = bias_divisor(hp->beta1, hp->bias_step);
  const float bc2 = bias_divisor(hp->beta2, hp->bias_step);
  for (int64_t i = 0; i < N; ++i) {
    if (hp->bias_step >= 1)
      u[i] = (m[i] / bc1) / (sqrtf(v[i] / bc2) + hp->eta);
    else
      u[i] = m[i] / (sqrtf(v[i]) + hp->eta);
    if (hp->weight_decay != 0.0f) u[i] = u[i] + (hp->weight_decay * x[i]);
  }

  /* W5 */
  float* c = (float*)xmalloc(sizeof(float) * (size_t)L);
  int64_t off = 0;
  for (int32_t l = 0; l < L; ++l) {
    double X = 0.0, U = 0.0;
    for (int64_t i = off; i < off + numels[l]; ++i) {
      X += (double)x[i] * (double)x[i];
      U += (double)u[i] * (double)u[i];
    }
    const float r = (X == 0.0 || U == 0.0) ? 1.0f : (float)(sqrt(X) / sqrt(U));
    c[l] = fminf(fmaxf(r, hp->c_min), hp->c_max);
    if (hp->c_avg_decay > 0.0f)
      c_sum[l] = (hp->c_avg_decay * c_sum[l]) + ((1.0f - hp->c_avg_decay) * c[l]);
    else
      c_sum[l] = c_sum[l] + c[l];
    if (c_out) c_out[l] = c[l];
    off += numels[l];
  }

  /* W6 */
  off = 0;
  for (int32_t l = 0; l < L; ++l) {
    const float step = hp->lr * c[l];
    for (int64_t i = off; i < off + numels[l]; ++i) x[i] = x[i] - (step * u[i]);
    off += numels[l];
  }
  free(c);
  free(u);
}

void oracle_freeze(int32_t L, int64_t N, int32_t W, const float* v, float* v_fresh,
                   float* const* err_w, float* err_s, const float* c_sum, int32_t T_w, float* c_avg,
                   float* f_prev, const oracle_hparams* hp) {
  const float d = hp ? hp->c_avg_decay : 0.0f;
  const float den = d > 0.0f ? (float)(1.0 - pow((double)d, (double)T_w)) : (float)T_w;
  for (int64_t i = 0; i < N; ++i) v_fresh[i] = v[i];
  for (int32_t w = 0; w < W; ++w)
    for (int64_t i = 0; i < N; ++i) err_w[w][i] = 0.0f;
  for (int64_t i = 0; i < N; ++i) err_s[i] = 0.0f;
  for (int32_t l = 0; l < L; ++l) {
    c_avg[l] = c_sum[l] / den;
    f_prev[l] = 1.0f;
  }
}

void oracle_compressed_step(int32_t L, const int64_t* numels, int32_t C, int32_t W,
                            const float* const* grads, float* const* err_w, float* err_s, float* x,
                            float* m, const float* v_frozen, float* v_fresh, const float* c_avg,
                            float* f_prev, float* c_out, uint32_t* const* bits_w,
                            float* const* scales_w, uint32_t* bits_s, float* scales_s,
                            const oracle_hparams* hp, int32_t compressor) {
  const float a1 = 1.0f - hp->beta1;
  const float a2 = 1.0f - hp->beta2;
  const float kp = 1.0f + hp->kappa;
  const float km = 1.0f - hp->kappa;
  int64_t N = 0;
  for (int32_t l = 0; l < L; ++l) N += numels[l];
  const int64_t K = num_chunks(N, C);
  const size_t nbuf = (size_t)(N > 0 ? N : 1);

  float* mhat = (float*)xmalloc(sizeof(float) * nbuf);
  float* in = (float*)xmalloc(sizeof(float) * nbuf);

  if (compressor == ORACLE_IDENTITY) {
    /* C1-C6 with C[z] = z: the errors stay 0 and the server's average is
     * forwarded as is. */
    for (int64_t i = 0; i < N; ++i) {
      float acc = 0.0f;
      for (int32_t w = 0; w < W; ++w) {
        const float z = ((hp->beta1 * m[i]) + (a1 * grads[w][i])) + err_w[w][i];
        acc = w == 0 ? z : acc + z;
      }
      mhat[i] = (acc / (float)W) + err_s[i];
    }
  } else {
    uint32_t** bw = (uint32_t**)xmalloc(sizeof(uint32_t*) * (size_t)W);
    float** sw = (float**)xmalloc(sizeof(float*) * (size_t)W);
    for (int32_t w = 0; w < W; ++w) {
      bw[w] = bits_w && bits_w[w] ? bits_w[w]
                                  : (uint32_t*)xmalloc(sizeof(uint32_t) * (size_t)(K * C / 32 + 1));
      sw[w] = scales_w && scales_w[w] ? scales_w[w] : (float*)xmalloc(sizeof(float) * (size_t)(K + 1));
    }
    uint32_t* bs = bits_s ? bits_s : (uint32_t*)xmalloc(sizeof(uint32_t) * (size_t)(K * C / 32 + 1));
    float* ss = scales_s ? scales_s : (float*)xmalloc(sizeof(float) * (size_t)(K + 1));

    /* C1-C4, worker by worker */
    for (int32_t w = 0; w < W; ++w) {
      for (int64_t i = 0; i < N; ++i) in[i] = (hp->beta1 * m[i]) + (a1 * grads[w][i]);
      oracle_compress_ef(N, C, in, err_w[w], bw[w], sw[w]);
    }
    /* C5-C6 */
    oracle_average_packed(N, C, W, (const uint32_t* const*)bw, (const float* const*)sw, err_s, bs, ss);
    oracle_decompress(N, C, bs, ss, mhat);

    for (int32_t w = 0; w < W; ++w) {
      if (!(bits_w && bits_w[w])) free(bw[w]);
      if (!(scales_w && scales_w[w])) free(sw[w]);
    }
    if (!bits_s) free(bs);
    if (!scales_s) free(ss);
    free(bw);
    free(sw);
  }

  /* C7-C9 (C9' when rho_mode = 1) */
  float* rho = (float*)xmalloc(sizeof(float) * (size_t)L);
  int64_t off = 0;
  for (int32_t l = 0; l < L; ++l) {
    float r = 0.0f;
    double Qz = 0.0, Qf = 0.0;
    for (int64_t i = off; i < off + numels[l]; ++i) {
      const float ghat = (mhat[i] - (hp->beta1 * m[i])) / a1;
      v_fresh[i] = (hp->beta2 * v_fresh[i]) + (a2 * (ghat * ghat));
      const float q = (sqrtf(v_frozen[i]) + hp->eta) / (sqrtf(v_fresh[i]) + hp->eta);
      /* the maximum of a set holding an undefined ratio is undefined: one
       * NaN anywhere in the tensor makes rho_l NaN (q > NaN is false, so
       * once r is NaN it stays NaN) */
      r = (i == off || isnan(q) || q > r) ? q : r;
      const double dz = (double)(sqrtf(v_frozen[i]) + hp->eta);
      const double df = (double)(sqrtf(v_fresh[i]) + hp->eta);
      Qz += dz * dz;
      Qf += df * df;
    }
    if (hp->rho_mode == 1) r = (Qz == 0.0 || Qf == 0.0) ? 1.0f : (float)(sqrt(Qz) / sqrt(Qf));
    rho[l] = r;
    off += numels[l];
  }

  /* C10 */
  float* c = (float*)xmalloc(sizeof(float) * (size_t)L);
  for (int32_t l = 0; l < L; ++l) {
    float f = fminf(fminf(rho[l], hp->f_max), kp * f_prev[l]);
    f = fmaxf(fmaxf(f, hp->f_min), km * f_prev[l]);
    f_prev[l] = f;
    c[l] = c_avg[l] * f;
    if (c_out) c_out[l] = c[l];
  }

  /* C11 */
  off = 0;
  for (int32_t l = 0; l < L; ++l) {
    const float step = hp->lr * c[l];
    for (int64_t i = off; i < off + numels[l]; ++i) {
      if (hp->weight_decay != 0.0f)
        x[i] = x[i] - (step * ((mhat[i] / (sqrtf(v_frozen[i]) + hp->eta)) + (hp->weight_decay * x[i])));
      else
        x[i] = x[i] - (step * (mhat[i] / (sqrtf(v_frozen[i]) + hp->eta)));
      m[i] = mhat[i];
    }
    off += numels[l];
  }

  free(c);
  free(rho);
  free(in);
  free(mhat);
}

/* ---- 1-bit Adam ------------------------------------------------------ */

void oracle_adam_warmup_step(int64_t n, int32_t W, const float* const* grads, float* x, float* m,
                             float* v, const oracle_hparams* hp) {
  const float a1 = 1.0f - hp->beta1;
  const float a2 = 1.0f - hp->beta2;
  /* W1-W3 */
  for (int64_t i = 0; i < n; ++i) {
    float gsum = grads[0][i];
    for (int32_t w = 1; w < W; ++w) gsum = gsum + grads[w][i];
    const float gmean = gsum / (float)W;
    m[i] = (hp->beta1 * m[i]) + (a1 * gmean);
    v[i] = (hp->beta2 * v[i]) + (a2 * (gmean * gmean));
  }
  /* W4 (W4' with bias correction) and the Adam update */
  const float bc1 = bias_divisor(hp->beta1, hp->bias_step);
  const float bc2 = bias_divisor(hp->beta2, hp->bias_step);
  for (int64_t i = 0; i < n; ++i) {
    const float u = hp->bias_step >= 1 ? (m[i] / bc1) / (sqrtf(v[i] / bc2) + hp->eta)
                                       : m[i] / (sqrtf(v[i]) + hp->eta);
    x[i] = x[i] - (hp->lr * u);
  }
}

void oracle_adam_compressed_step(int64_t n, int32_t C, int32_t W, const float* const* grads,
                                 float* const* err_w, float* err_s, float* x, float* m,
                                 const float* v_frozen, uint32_t* const* bits_w,
                                 float* const* scales_w, uint32_t* bits_s, float* scales_s,
                                 const oracle_hparams* hp, int32_t compressor) {
  const float a1 = 1.0f - hp->beta1;
  const int64_t K = num_chunks(n, C);
  const size_t nbuf = (size_t)(n > 0 ? n : 1);
  float* mhat = (float*)xmalloc(sizeof(float) * nbuf);
  float* in = (float*)xmalloc(sizeof(float) * nbuf);

  if (compressor == ORACLE_IDENTITY) {
    for (int64_t i = 0; i < n; ++i) {
      float acc = 0.0f;
      for (int32_t w = 0; w < W; ++w) {
        const float z = ((hp->beta1 * m[i]) + (a1 * grads[w][i])) + err_w[w][i];
        acc = w == 0 ? z : acc + z;
      }
      mhat[i] = (acc / (float)W) + err_s[i];
    }
  } else {
    uint32_t** bw = (uint32_t**)xmalloc(sizeof(uint32_t*) * (size_t)W);
    float** sw = (float**)xmalloc(sizeof(float*) * (size_t)W);
    for (int32_t w = 0; w < W; ++w) {
      bw[w] = bits_w && bits_w[w] ? bits_w[w]
                                  : (uint32_t*)xmalloc(sizeof(uint32_t) * (size_t)(K * C / 32 + 1));
      sw[w] = scales_w && scales_w[w] ? scales_w[w] : (float*)xmalloc(sizeof(float) * (size_t)(K + 1));
    }
    uint32_t* bs = bits_s ? bits_s : (uint32_t*)xmalloc(sizeof(uint32_t) * (size_t)(K * C / 32 + 1));
    float* ss = scales_s ? scales_s : (float*)xmalloc(sizeof(float) * (size_t)(K + 1));

    /* C1-C4, worker by worker */
    for (int32_t w = 0; w < W; ++w) {
      const float* gw = grads[w];
      for (int64_t i = 0; i < n; ++i) in[i] = (hp->beta1 * m[i]) + (a1 * gw[i]);
      oracle_compress_ef(n, C, in, err_w[w], bw[w], sw[w]);
    }
    /* C5-C6 */
    oracle_average_packed(n, C, W, (const uint32_t* const*)bw, (const float* const*)sw, err_s, bs, ss);
    oracle_decompress(n, C, bs, ss, mhat);

    for (int32_t w = 0; w < W; ++w) {
      if (!(bits_w && bits_w[w])) free(bw[w]);
      if (!(scales_w && scales_w[w])) free(sw[w]);
    }
    if (!bits_s) free(bs);
    if (!scales_s) free(ss);
    free(bw);
    free(sw);
  }

  /* momentum SGD preconditioned by the frozen variance */
  for (int64_t i = 0; i < n; ++i) {
    x[i] = x[i] - (hp->lr * (mhat[i] / (sqrtf(v_frozen[i]) + hp->eta)));
    m[i] = mhat[i];
  }
  free(in);
  free(mhat);
}

/* ---- SLAMB-style sparse compression stage ----------------------------- */

/* Position of element j of a chunk among the transmitted values, or -1. */
static int64_t sparse_slot(int64_t j, int32_t C, int32_t nsel, int32_t first_block) {
  const int64_t nb = C / 64;
  const int64_t rel = ((j / 64) - first_block + nb) % nb;
  return rel < nsel ? rel * 64 + j % 64 : -1;
}

void oracle_sparse_step(int32_t L, const int64_t* numels, int32_t C, int32_t W, int32_t nsel,
                        const int32_t* sel, const float* const* grads, float* const* err_w,
                        float* x, float* m, const float* v_frozen, float* v_fresh,
                        const float* c_avg, float* const* vals_w, float* vals_s,
                        const oracle_hparams* hp) {
  const float a1 = 1.0f - hp->beta1;
  const float a2 = 1.0f - hp->beta2;
  int64_t N = 0;
  for (int32_t l = 0; l < L; ++l) N += numels[l];
  const int64_t K = num_chunks(N, C);
  const int64_t per = (int64_t)nsel * 64;
  float* mhat = (float*)xmalloc(sizeof(float) * (size_t)(N > 0 ? N : 1));

  /* the transmitted arrays start at 0 (positions past the buffer's end) */
  for (int64_t q = 0; q < K * per; ++q) vals_s[q] = 0.0f;
  for (int32_t w = 0; w < W; ++w)
    if (vals_w && vals_w[w])
      for (int64_t q = 0; q < K * per; ++q) vals_w[w][q] = 0.0f;

  /* S1-S4, element by element, workers in order */
  for (int64_t i = 0; i < N; ++i) {
    const int64_t k = i / C;
    const int64_t slot = sparse_slot(i - k * C, C, nsel, sel[k]);
    float acc = 0.0f;
    for (int32_t w = 0; w < W; ++w) {
      const float z = ((hp->beta1 * m[i]) + (a1 * grads[w][i])) + err_w[w][i];
      if (slot >= 0) {
        if (vals_w && vals_w[w]) vals_w[w][k * per + slot] = z;
        acc = w == 0 ? z : acc + z;
        err_w[w][i] = 0.0f;
      } else {
        err_w[w][i] = z;
      }
    }
    if (slot >= 0) {
      mhat[i] = acc / (float)W;
      vals_s[k * per + slot] = mhat[i];
    } else {
      mhat[i] = 0.0f;
    }
  }

  /* S5-S6 */
  int64_t off = 0;
  for (int32_t l = 0; l < L; ++l) {
    const float step = hp->lr * c_avg[l];
    for (int64_t i = off; i < off + numels[l]; ++i) {
      const int64_t k = i / C;
      if (sparse_slot(i - k * C, C, nsel, sel[k]) >= 0) {
        const float gh = (mhat[i] - (hp->beta1 * m[i])) / a1;
        v_fresh[i] = (hp->beta2 * v_fresh[i]) + (a2 * (gh * gh));
        const float dz = sqrtf(v_frozen[i]) + hp->eta;
        const float q = dz / (sqrtf(v_fresh[i]) + hp->eta);
        const float r = fminf(fmaxf(q, hp->f_min), hp->f_max);
        x[i] = x[i] - (step * (r * (mhat[i] / dz)));
      }
      m[i] = mhat[i];
    }
    off += numels[l];
  }
  free(mhat);
}
