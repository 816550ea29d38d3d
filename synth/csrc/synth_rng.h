/*
 * synth_rng.h -- seeded, counter-based input generator shared by the host
 * build (gcc, synth_host.c) and the device build (hipcc, synth_gpu.hip) of
 * the `synth` module.  It produces the synthetic activations, weights and
 * biases of the MoE workloads; it holds none of the MoE method's arithmetic.
 *
 * Generator definition (both builds must agree bit for bit):
 *   - Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 *     easy as 1, 2, 3", SC'11).  Key = (seed, tensor_id); the 64-bit block
 *     counter n occupies word 0 of the 256-bit counter, words 1..3 are 0.
 *     One block yields four 64-bit words r0..r3.
 *   - Element `flat` of a tensor uses block flat/4 and word flat%4.
 *   - Uniform in (0,1]:  U(r) = ((r >> 11) + 1) * 2^-53   (exact in double).
 *     Angle fraction in [0,1): V(r) = (r >> 11) * 2^-53.
 *   - Normal: Box--Muller on the word pair (r0,r1) for words 0,1 and (r2,r3)
 *     for words 2,3: R = sqrt(-2 ln U(r_even)), phi = 2*pi*V(r_odd);
 *     even word -> R cos(phi), odd word -> R sin(phi).
 *   - ln, sqrt, sin and cos are computed below with IEEE add, subtract and
 *     multiply only (no library calls, no fused multiply-add: both builds
 *     compile this file with -ffp-contract=off), so the host and device
 *     results are identical.  Their accuracy (~1e-15 relative) is far beyond
 *     what a synthetic input needs; determinism is the point.
 *   - Final value: (float)(sigma * z) with sigma passed in as a double, then
 *     optionally rounded to bfloat16 by round-to-nearest-even on the bits.
 */
#ifndef SYNTH_RNG_H
#define SYNTH_RNG_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYN_FN __host__ __device__ static inline
#else
#define SYN_FN static inline
#endif

/* Philox4x64 multipliers and Weyl key increments (SC'11, Table 2). */
#define SYN_PHILOX_M0 0xD2E7470EE14C6C93ull
#define SYN_PHILOX_M1 0xCA5A826395121157ull
#define SYN_PHILOX_W0 0x9E3779B97F4A7C15ull
#define SYN_PHILOX_W1 0xBB67AE8584CAA73Bull

SYN_FN void syn_mulhilo64(uint64_t a, uint64_t b, uint64_t *hi, uint64_t *lo) {
#if defined(__HIP_DEVICE_COMPILE__)
  *lo = a * b;
  *hi = __umul64hi(a, b);
#else
  unsigned __int128 p = (unsigned __int128)a * b;
  *lo = (uint64_t)p;
  *hi = (uint64_t)(p >> 64);
#endif
}

/* One Philox4x64-10 block for counter (n, 0, 0, 0) and key (k0, k1). */
SYN_FN void syn_philox4x64_10(uint64_t n, uint64_t k0, uint64_t k1, uint64_t r[4]) {
  uint64_t c0 = n, c1 = 0, c2 = 0, c3 = 0;
  for (int round = 0; round < 10; ++round) {
    uint64_t hi0, lo0, hi1, lo1;
    syn_mulhilo64(SYN_PHILOX_M0, c0, &hi0, &lo0);
    syn_mulhilo64(SYN_PHILOX_M1, c2, &hi1, &lo1);
    uint64_t n0 = hi1 ^ c1 ^ k0;
    uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += SYN_PHILOX_W0;
    k1 += SYN_PHILOX_W1;
  }
  r[0] = c0; r[1] = c1; r[2] = c2; r[3] = c3;
}

SYN_FN double syn_bits_to_double(uint64_t b) {
  union { uint64_t u; double d; } v;
  v.u = b;
  return v.d;
}

SYN_FN uint64_t syn_double_to_bits(double d) {
  union { uint64_t u; double d; } v;
  v.d = d;
  return v.u;
}

SYN_FN double syn_unit_open0(uint64_t r) { /* (0, 1] */
  return (double)((r >> 11) + 1ull) * 0x1p-53;
}

SYN_FN double syn_unit_open1(uint64_t r) { /* [0, 1) */
  return (double)(r >> 11) * 0x1p-53;
}

/* Natural log for u in (0, 1]: u = 2^e * m with m in [1/sqrt2, sqrt2),
 * ln(m) = 2 atanh(s), s = (m-1)/(m+1), the reciprocal 1/(m+1) by Newton
 * iteration.  Coefficients are 1/(2n+1) as exact hex literals. */
SYN_FN double syn_ln(double u) {
  uint64_t b = syn_double_to_bits(u);
  int e = (int)((b >> 52) & 0x7ffull) - 1023;
  double m = syn_bits_to_double((b & 0x000fffffffffffffull) | 0x3ff0000000000000ull);
  if (m > 0x1.6a09e667f3bcdp+0) { /* sqrt(2) */
    m = m * 0.5;
    e += 1;
  }
  double f = m - 1.0;
  double den = 2.0 + f;                 /* in [1.70, 2.42] */
  double rcp = 0.5;                     /* |1 - den*rcp| <= 0.21 */
  for (int i = 0; i < 6; ++i) rcp = rcp * (2.0 - den * rcp);
  double s = f * rcp;
  double s2 = s * s;                    /* <= 0.0295 */
  double p = 0x1.47ae147ae147bp-5;      /* 1/25 */
  p = p * s2 + 0x1.642c8590b2164p-5;    /* 1/23 */
  p = p * s2 + 0x1.8618618618618p-5;    /* 1/21 */
  p = p * s2 + 0x1.af286bca1af28p-5;    /* 1/19 */
  p = p * s2 + 0x1.e1e1e1e1e1e1ep-5;    /* 1/17 */
  p = p * s2 + 0x1.1111111111111p-4;    /* 1/15 */
  p = p * s2 + 0x1.3b13b13b13b14p-4;    /* 1/13 */
  p = p * s2 + 0x1.745d1745d1746p-4;    /* 1/11 */
  p = p * s2 + 0x1.c71c71c71c71cp-4;    /* 1/9 */
  p = p * s2 + 0x1.2492492492492p-3;    /* 1/7 */
  p = p * s2 + 0x1.999999999999ap-3;    /* 1/5 */
  p = p * s2 + 0x1.5555555555555p-2;    /* 1/3 */
  p = p * s2 + 1.0;
  return (double)e * 0x1.62e42fefa39efp-1 + 2.0 * s * p; /* ln 2 */
}

/* sqrt(a) for a >= 0 by Newton iteration on 1/sqrt(a). */
SYN_FN double syn_sqrt(double a) {
  if (a <= 0.0) return 0.0;
  double y = syn_bits_to_double(0x5FE6EB50C7B537A9ull - (syn_double_to_bits(a) >> 1));
  for (int i = 0; i < 6; ++i) y = y * (1.5 - 0.5 * a * y * y);
  return a * y;
}

/* sin and cos of 2*pi*v for v in [0, 1): exact quadrant split, then Taylor
 * series on [0, pi/2) with coefficients (-1)^n/(2n+1)! and (-1)^n/(2n)!. */
SYN_FN void syn_sincos_2pi(double v, double *sn, double *cs) {
  double t = v * 4.0;                   /* exact */
  int q = (int)t;                       /* 0..3 */
  double r = t - (double)q;             /* exact, in [0, 1) */
  double th = r * 0x1.921fb54442d18p+0; /* pi/2 */
  double t2 = th * th;
  double ps = 0x1.3f3ccdd165fa9p-84;
  ps = ps * t2 - 0x1.761b41316381ap-75;
  ps = ps * t2 + 0x1.71b8ef6dcf572p-66;
  ps = ps * t2 - 0x1.2f49b46814157p-57;
  ps = ps * t2 + 0x1.952c77030ad4ap-49;
  ps = ps * t2 - 0x1.ae7f3e733b81fp-41;
  ps = ps * t2 + 0x1.6124613a86d09p-33;
  ps = ps * t2 - 0x1.ae64567f544e4p-26;
  ps = ps * t2 + 0x1.71de3a556c734p-19;
  ps = ps * t2 - 0x1.a01a01a01a01ap-13;
  ps = ps * t2 + 0x1.1111111111111p-7;
  ps = ps * t2 - 0x1.5555555555555p-3;
  ps = ps * t2 + 1.0;
  double s = th * ps;
  double pc = 0x1.f2cf01972f578p-80;
  pc = pc * t2 - 0x1.0ce396db7f853p-70;
  pc = pc * t2 + 0x1.e542ba4020225p-62;
  pc = pc * t2 - 0x1.6827863b97d97p-53;
  pc = pc * t2 + 0x1.ae7f3e733b81fp-45;
  pc = pc * t2 - 0x1.93974a8c07c9dp-37;
  pc = pc * t2 + 0x1.1eed8eff8d898p-29;
  pc = pc * t2 - 0x1.27e4fb7789f5cp-22;
  pc = pc * t2 + 0x1.a01a01a01a01ap-16;
  pc = pc * t2 - 0x1.6c16c16c16c17p-10;
  pc = pc * t2 + 0x1.5555555555555p-5;
  pc = pc * t2 - 0.5;
  pc = pc * t2 + 1.0;
  double c = pc;
  switch (q) {
    case 0: *sn = s;  *cs = c;  break;
    case 1: *sn = c;  *cs = -s; break;
    case 2: *sn = -s; *cs = -c; break;
    default: *sn = -c; *cs = s; break;
  }
}

/* Four consecutive normals (elements 4n .. 4n+3) of tensor (seed, tid). */
SYN_FN void syn_normal4(uint64_t seed, uint64_t tid, uint64_t n, double z[4]) {
  uint64_t r[4];
  syn_philox4x64_10(n, seed, tid, r);
  for (int p = 0; p < 2; ++p) {
    double rad = syn_sqrt(-2.0 * syn_ln(syn_unit_open0(r[2 * p])));
    double sn, cs;
    syn_sincos_2pi(syn_unit_open1(r[2 * p + 1]), &sn, &cs);
    z[2 * p] = rad * cs;
    z[2 * p + 1] = rad * sn;
  }
}

/* Four consecutive uniforms in (0, 1] (elements 4n .. 4n+3). */
SYN_FN void syn_uniform4(uint64_t seed, uint64_t tid, uint64_t n, double u[4]) {
  uint64_t r[4];
  syn_philox4x64_10(n, seed, tid, r);
  for (int w = 0; w < 4; ++w) u[w] = syn_unit_open0(r[w]);
}

SYN_FN uint16_t syn_f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t u = v.u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#endif /* SYNTH_RNG_H */
