/*
 * synth_host.c -- host build of the seeded input generator (see synth_rng.h
 * for the generator's definition).  Fills host arrays; OpenMP over blocks.
 * Holds none of the MoE method's arithmetic.
 */
#include <stddef.h>
#include <stdint.h>

#include "synth_rng.h"

/* Raw Philox4x64-10 block, for known-answer tests. */
void syn_philox_block(uint64_t n, uint64_t k0, uint64_t k1, uint64_t out[4]) {
  syn_philox4x64_10(n, k0, k1, out);
}

/* The transcendental helpers, exposed for tests against libm. */
double syn_ln_host(double u) { return syn_ln(u); }
double syn_sqrt_host(double a) { return syn_sqrt(a); }
void syn_sincos_2pi_host(double v, double *s, double *c) { syn_sincos_2pi(v, s, c); }

/* Elements [first, first + count) of the normal tensor (seed, tid), scaled by
 * sigma and rounded to fp32 (out_f32) or further to bf16 (out_bf16).
 * Exactly one of out_f32 / out_bf16 is non-NULL. */
void syn_normal_fill(float *out_f32, uint16_t *out_bf16, int64_t first, int64_t count,
                     uint64_t seed, uint64_t tid, double sigma) {
  if (count <= 0) return;
  int64_t b0 = first / 4, b1 = (first + count - 1) / 4;
#pragma omp parallel for schedule(static)
  for (int64_t b = b0; b <= b1; ++b) {
    double z[4];
    syn_normal4(seed, tid, (uint64_t)b, z);
    for (int w = 0; w < 4; ++w) {
      int64_t flat = b * 4 + w;
      if (flat < first || flat >= first + count) continue;
      float v = (float)(sigma * z[w]);
      if (out_f32) out_f32[flat - first] = v;
      else out_bf16[flat - first] = syn_f32_to_bf16_rne(v);
    }
  }
}

/* Elements [first, first + count) of the uniform tensor (seed, tid) mapped to
 * lo + (hi - lo) * u, u in (0, 1], rounded to fp32. */
void syn_uniform_fill(float *out, int64_t first, int64_t count, uint64_t seed, uint64_t tid,
                      double lo, double hi) {
  if (count <= 0) return;
  int64_t b0 = first / 4, b1 = (first + count - 1) / 4;
#pragma omp parallel for schedule(static)
  for (int64_t b = b0; b <= b1; ++b) {
    double u[4];
    syn_uniform4(seed, tid, (uint64_t)b, u);
    for (int w = 0; w < 4; ++w) {
      int64_t flat = b * 4 + w;
      if (flat < first || flat >= first + count) continue;
      out[flat - first] = (float)(lo + (hi - lo) * u[w]);
    }
  }
}

uint16_t syn_bf16_from_f32(float f) { return syn_f32_to_bf16_rne(f); }
