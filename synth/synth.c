/*
 * Host fill of seeded synthetic arrays (test and benchmark infrastructure).
 * Every value is a pure function of (seed, stream, element index) defined in
 * synth_core.h, so any window of an array can be regenerated on its own and
 * matches what synth_dev.hip writes on the device.  OpenMP only splits the
 * index range; the values do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "synth_core.h"

void synth_fill_normal(uint64_t seed, uint64_t stream, int64_t offset, int64_t n,
                       double mean, double std, float* out) {
  const uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j)
    out[j] = synth_normal_f32(key, (uint64_t)(offset + j), mean, std);
}

void synth_fill_uniform(uint64_t seed, uint64_t stream, int64_t offset, int64_t n,
                        double lo, double hi, float* out) {
  const uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j)
    out[j] = synth_uniform_f32(key, (uint64_t)(offset + j), lo, hi);
}

/* Raw doubles, for tests of the generator itself. */
void synth_normal_f64(uint64_t seed, uint64_t stream, int64_t offset, int64_t n, double* out) {
  const uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = synth_normal(key, (uint64_t)(offset + j));
}

/* Per-tensor multipliers 10^U(lo_exp10, hi_exp10), one per tensor, host only
 * (the same doubles are then passed to the host and the device fills). */
void synth_layer_log_scales(uint64_t seed, uint64_t stream, int32_t L, double lo_exp10,
                            double hi_exp10, double* out) {
  const uint64_t key = synth_key(seed, stream);
  for (int32_t l = 0; l < L; ++l)
    out[l] = pow(10.0, lo_exp10 + (hi_exp10 - lo_exp10) * synth_uniform(key, (uint64_t)l));
}

/* out[j] = uniform integer in [0, nb) number offset+j of the stream: the top
 * 32 bits of the keyed draw, scaled to the range by a multiply and shift. */
void synth_fill_index(uint64_t seed, uint64_t stream, int64_t offset, int64_t n, int32_t nb,
                      int32_t* out) {
  const uint64_t key = synth_key(seed, stream);
  for (int64_t j = 0; j < n; ++j) {
    const uint64_t x = synth_mix64(key + (2 * (uint64_t)(offset + j) + 1) * SYNTH_GAMMA);
    out[j] = (int32_t)(((x >> 32) * (uint64_t)nb) >> 32);
  }
}

/* Scalar reference pieces of the generator, exposed for its own tests. */
double synth_ln_unit_host(uint64_t M) { return synth_ln_unit(M); }
double synth_sqrt_host(double a) { return synth_sqrt(a); }
double synth_cos2pi_host(uint64_t N) { return synth_cos2pi(N); }
uint64_t synth_mix64_host(uint64_t z) { return synth_mix64(z); }

int synth_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
