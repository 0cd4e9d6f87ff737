/*
 * Counter-based synthetic variates, shared by the host fill (synth.c) and the
 * device fill (synth_dev.hip).  This file holds no arithmetic of the 1-bit
 * LAMB method: it only turns (seed, stream, element index) into a normal or a
 * uniform number, so that the CPU oracle and the GPU library can be handed the
 * same inputs, and any slice of a large array can be regenerated on its own.
 *
 * Definition (all integer arithmetic is modulo 2^64):
 *   mix(z)      SplitMix64 output function (Steele, Lea & Flood, "Fast
 *               splittable pseudorandom number generators", OOPSLA 2014, with
 *               the 64-bit finaliser constants of their reference code):
 *                 z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *                 z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31
 *   key         mix(seed ^ mix(stream + GAMMA)),  GAMMA = 0x9E3779B97F4A7C15
 *   x1, x2      mix(key + (2i+1)*GAMMA), mix(key + (2i+2)*GAMMA)
 *   u1          ((x1 >> 11) + 1) * 2^-53            in (0, 1]
 *   u2          (x2 >> 11) * 2^-53                  in [0, 1)
 *   normal(i)   sqrt(-2 ln u1) * cos(2 pi u2)       (Box & Muller 1958)
 *   uniform(i)  (x1 >> 11) * 2^-53                  in [0, 1)
 *
 * ln, sqrt and cos are evaluated here with IEEE double +, -, *, / only, in a
 * fixed order and with floating-point contraction disabled, so that the host
 * and the device produce bit-identical doubles (and therefore bit-identical
 * fp32 values after the final round-to-nearest conversion):
 *   ln(M 2^-53)  exponent/mantissa split m in [sqrt(1/2), sqrt(2)], then
 *                ln m = 2 atanh(s), s = (m-1)/(m+1), odd series to s^23
 *   sqrt(a)      bit-level first guess, then 6 Heron (Newton) iterations
 *   cos(2 pi u)  quadrant from the top two bits of u, Taylor series of cos
 *                and sin on [0, pi/2) to degree 22/23
 * The accuracy of these routines is about 1e-15, far below what matters for
 * synthetic data; only their reproducibility matters.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#ifndef SYNTH_QUAL
#define SYNTH_QUAL static inline
#endif

#if defined(__clang__)
#define SYNTH_NO_CONTRACT _Pragma("clang fp contract(off)")
#else
#define SYNTH_NO_CONTRACT
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

SYNTH_QUAL uint64_t synth_mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

SYNTH_QUAL uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return synth_mix64(seed ^ synth_mix64(stream + SYNTH_GAMMA));
}

SYNTH_QUAL double synth_from_bits(uint64_t b) {
  union { uint64_t u; double d; } c;
  c.u = b;
  return c.d;
}

SYNTH_QUAL uint64_t synth_to_bits(double d) {
  union { uint64_t u; double d; } c;
  c.d = d;
  return c.u;
}

/* ln(M * 2^-53) for integer M in [1, 2^53]. */
SYNTH_QUAL double synth_ln_unit(uint64_t M) {
  SYNTH_NO_CONTRACT
  int e = 63 - __builtin_clzll(M);                       /* M = 2^e * m, m in [1,2) */
  double m = (double)M * synth_from_bits((uint64_t)(1023 - e) << 52);
  if (m > 0x1.6a09e667f3bcdp+0) {                        /* m > sqrt(2) */
    m = m * 0.5;
    e = e + 1;
  }
  double f = m - 1.0;
  double s = f / (2.0 + f);
  double t = s * s;
  double p = 0x1.642c8590b2164p-5;                       /* 1/23 */
  p = p * t + 0x1.8618618618618p-5;                      /* 1/21 */
  p = p * t + 0x1.af286bca1af28p-5;                      /* 1/19 */
  p = p * t + 0x1.e1e1e1e1e1e1ep-5;                      /* 1/17 */
  p = p * t + 0x1.1111111111111p-4;                      /* 1/15 */
  p = p * t + 0x1.3b13b13b13b14p-4;                      /* 1/13 */
  p = p * t + 0x1.745d1745d1746p-4;                      /* 1/11 */
  p = p * t + 0x1.c71c71c71c71cp-4;                      /* 1/9  */
  p = p * t + 0x1.2492492492492p-3;                      /* 1/7  */
  p = p * t + 0x1.999999999999ap-3;                      /* 1/5  */
  p = p * t + 0x1.5555555555555p-2;                      /* 1/3  */
  p = p * t + 1.0;
  double lnm = (2.0 * s) * p;
  return (double)(e - 53) * 0x1.62e42fefa39efp-1 + lnm;  /* ln 2 */
}

/* sqrt(a) for a >= 0 by Heron's iteration from a bit-level first guess. */
SYNTH_QUAL double synth_sqrt(double a) {
  SYNTH_NO_CONTRACT
  if (!(a > 0.0)) return 0.0;
  double y = synth_from_bits((synth_to_bits(a) >> 1) + 0x1FF8000000000000ULL);
  for (int it = 0; it < 6; ++it) y = 0.5 * (y + a / y);
  return y;
}

/* cos(2 pi N 2^-53) for integer N in [0, 2^53). */
SYNTH_QUAL double synth_cos2pi(uint64_t N) {
  SYNTH_NO_CONTRACT
  unsigned q = (unsigned)(N >> 51);                      /* quadrant 0..3 */
  double r = (double)(N & ((1ULL << 51) - 1)) * 0x1p-51; /* [0,1) within it */
  double th = r * 0x1.921fb54442d18p+0;                  /* r * pi/2 */
  double t = th * th;
  if (q == 0 || q == 2) {
    double c = -0x1.0ce396db7f853p-70;
    c = c * t + 0x1.e542ba4020225p-62;
    c = c * t + -0x1.6827863b97d97p-53;
    c = c * t + 0x1.ae7f3e733b81fp-45;
    c = c * t + -0x1.93974a8c07c9dp-37;
    c = c * t + 0x1.1eed8eff8d898p-29;
    c = c * t + -0x1.27e4fb7789f5cp-22;
    c = c * t + 0x1.a01a01a01a01ap-16;
    c = c * t + -0x1.6c16c16c16c17p-10;
    c = c * t + 0x1.5555555555555p-5;
    c = c * t + -0x1.0000000000000p-1;
    c = c * t + 1.0;
    return q == 0 ? c : -c;
  } else {
    double s = -0x1.761b41316381ap-75;
    s = s * t + 0x1.71b8ef6dcf572p-66;
    s = s * t + -0x1.2f49b46814157p-57;
    s = s * t + 0x1.952c77030ad4ap-49;
    s = s * t + -0x1.ae7f3e733b81fp-41;
    s = s * t + 0x1.6124613a86d09p-33;
    s = s * t + -0x1.ae64567f544e4p-26;
    s = s * t + 0x1.71de3a556c734p-19;
    s = s * t + -0x1.a01a01a01a01ap-13;
    s = s * t + 0x1.1111111111111p-7;
    s = s * t + -0x1.5555555555555p-3;
    s = s * t + 1.0;
    s = s * th;
    return q == 1 ? -s : s;                              /* cos(pi/2+x) = -sin x */
  }
}

/* Standard normal variate number i of the stream keyed by `key`. */
SYNTH_QUAL double synth_normal(uint64_t key, uint64_t i) {
  SYNTH_NO_CONTRACT
  uint64_t x1 = synth_mix64(key + (2 * i + 1) * SYNTH_GAMMA);
  uint64_t x2 = synth_mix64(key + (2 * i + 2) * SYNTH_GAMMA);
  double ln_u1 = synth_ln_unit((x1 >> 11) + 1);
  double R = synth_sqrt(-2.0 * ln_u1);
  return R * synth_cos2pi(x2 >> 11);
}

/* Uniform variate in [0,1) number i of the stream keyed by `key`. */
SYNTH_QUAL double synth_uniform(uint64_t key, uint64_t i) {
  SYNTH_NO_CONTRACT
  uint64_t x1 = synth_mix64(key + (2 * i + 1) * SYNTH_GAMMA);
  return (double)(x1 >> 11) * 0x1p-53;
}

/* The fp32 values handed to both sides. */
SYNTH_QUAL float synth_normal_f32(uint64_t key, uint64_t i, double mean, double std) {
  SYNTH_NO_CONTRACT
  return (float)(mean + std * synth_normal(key, i));
}

SYNTH_QUAL float synth_uniform_f32(uint64_t key, uint64_t i, double lo, double hi) {
  SYNTH_NO_CONTRACT
  return (float)(lo + (hi - lo) * synth_uniform(key, i));
}

#endif /* SYNTH_CORE_H */
