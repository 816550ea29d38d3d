/*
 * oracle.c -- plain, slow CPU definition of the zero-computation-expert MoE
 * forward.  TEST INFRASTRUCTURE ONLY: used by tests/, by the smoke check and
 * by the benchmark's CPU-baseline leg, never by the GPU product path.  It
 * shares no code, header or table with the HIP library.
 *
 * Sources (the pages that describe the method):
 *   [LCF-arch]  LongCat-Flash technical-report summary (zhangjingwei.cn page),
 *               section 2 "architecture", item 1 "zero-computation experts":
 *               tokens pick among FFN experts and Z zero-computation experts;
 *               a zero-computation expert only returns its input, at no
 *               compute cost; an expert-specific bias, adjusted by a
 *               controller, shifts the routing scores so the share of FFN vs
 *               zero experts stays on target.
 *   [LCF-cfg]   same page, section 2, model-configuration paragraph: 512 FFN
 *               experts of width 2048 and 256 zero experts per layer, 12
 *               experts per token, hidden size 6144.
 *   [LCF-infra] same page, section 5 "training infrastructure", numerical
 *               precision item: BF16 results are judged against a CPU FP32
 *               ground truth.  The oracle therefore computes in fp32, with
 *               bfloat16 inputs widened exactly.
 *   [KOL]       cnouyi.fund thread summarising the same report: the zero
 *               expert acts as a "sink" for easy tokens; balancing is an
 *               aux-loss-free bias in the style of DeepSeek-V3.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - routing score = softmax over all N+Z router logits (fp32, max-shifted);
 *   - the bias is added to the softmax probability and used for selection
 *     only; the gate of a selected expert is its unbiased probability, with
 *     no renormalisation and no scale;
 *   - an FFN expert is SwiGLU with three matrices and no biases:
 *       y = W_down (silu(W_gate x) * (W_up x)),  silu(z) = z / (1 + e^-z);
 *   - top-k order: biased score descending, equal scores -> lower index;
 *   - output = (sum of zero-slot gates) * x + sum_j gate_j * y_j, the FFN
 *     terms added in ascending slot order.
 *
 * Every sum is a plain left-to-right fp32 sum in ascending index order.
 * Build: gcc -O2 -fopenmp -ffp-contract=off (OpenMP only splits tokens).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* Exact widening of an element of an fp32 or bfloat16 array to fp32. */
static float orc_ld(const void *p, int64_t i, int dt) {
  if (dt == ORC_F32) return ((const float *)p)[i];
  uint32_t b = (uint32_t)((const uint16_t *)p)[i] << 16;
  float f;
  memcpy(&f, &b, sizeof f);
  return f;
}

/* Step 1 of [LCF-arch]: router logits l[t,e] = sum_i x[t,i] * W_router[e,i]. */
void oracle_router_logits(int64_t T, int d, int E, const void *x, const void *w_router, int dt,
                          float *logits) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int i = 0; i < d; ++i)
        acc += orc_ld(x, t * (int64_t)d + i, dt) * orc_ld(w_router, (int64_t)e * d + i, dt);
      logits[t * (int64_t)E + e] = acc;
    }
  }
}

/* Softmax of one token's logits over all E experts (FFN and zero together). */
static void orc_softmax(int E, const float *l, float *p) {
  float m = l[0];
  for (int e = 1; e < E; ++e)
    if (l[e] > m) m = l[e];
  float sum = 0.0f;
  for (int e = 0; e < E; ++e) sum += expf(l[e] - m);
  for (int e = 0; e < E; ++e) p[e] = expf(l[e] - m) / sum;
}

/* Steps 1-2 of [LCF-arch] from given logits: p = softmax(l); s = p + bias;
 * idx = the k experts of largest s (ties -> lower index), listed by s
 * descending; gate_j = routed_scale * p[idx_j]; margin = s_(k) - s_(k+1)
 * (+inf if k == E).  probs (nullable) receives p (unscaled).
 * routed_scale: [LITE] (the LongCat-Flash-Lite article, part 02) fuses the
 * router's logits, softmax, top-k and a scaling step into one kernel; the
 * pages do not say what is scaled.  Reading: every selected slot's gate is
 * multiplied by one constant (FFN and zero slots alike, as the router does
 * not tell them apart); selection does not depend on it; 1 is the unscaled
 * method, and multiplying by 1 is exact. */
void oracle_route_from_logits(int64_t T, int E, int k, const float *logits, const float *bias,
                              int32_t *idx, float *gate, float *margin, float *probs,
                              float routed_scale) {
#pragma omp parallel
  {
    float *p = (float *)malloc(sizeof(float) * (size_t)E);
    float *s = (float *)malloc(sizeof(float) * (size_t)E);
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      orc_softmax(E, logits + t * (int64_t)E, p);
      for (int e = 0; e < E; ++e) {
        s[e] = p[e] + bias[e];
        taken[e] = 0;
      }
      float last = 0.0f;
      /* selection by repeated argmax: strictly greater wins, so the lowest
       * index wins among equal scores */
      for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e)
          if (!taken[e] && (best < 0 || s[e] > s[best])) best = e;
        taken[best] = 1;
        idx[t * k + j] = best;
        gate[t * k + j] = routed_scale * p[best];
        last = s[best];
      }
      if (margin) {
        if (k >= E) {
          margin[t] = INFINITY;
        } else {
          int nxt = -1;
          for (int e = 0; e < E; ++e)
            if (!taken[e] && (nxt < 0 || s[e] > s[nxt])) nxt = e;
          margin[t] = last - s[nxt];
        }
      }
      if (probs) memcpy(probs + t * (int64_t)E, p, sizeof(float) * (size_t)E);
    }
    free(p);
    free(s);
    free(taken);
  }
}

/* Per-expert selection counts over all E experts ([LCF-arch], the quantity
 * the bias controller consumes). */
void oracle_counts(int64_t T, int k, int E, const int32_t *idx, int32_t *counts) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) counts[idx[t * k + j]] += 1;
}

/* One SwiGLU FFN expert on one token: y = Wd (silu(Wg x) * (Wu x)).
 * wg, wu: [I, d]; wd: [d, I]; h: scratch of I floats. */
static void orc_expert(int d, int I, const float *x, const void *wg, const void *wu,
                       const void *wd, int dt, float *h, float *y) {
  for (int r = 0; r < I; ++r) {
    float g = 0.0f, u = 0.0f;
    for (int c = 0; c < d; ++c) {
      g += orc_ld(wg, (int64_t)r * d + c, dt) * x[c];
      u += orc_ld(wu, (int64_t)r * d + c, dt) * x[c];
    }
    h[r] = (g / (1.0f + expf(-g))) * u;
  }
  for (int i = 0; i < d; ++i) {
    float acc = 0.0f;
    for (int r = 0; r < I; ++r) acc += orc_ld(wd, (int64_t)i * I + r, dt) * h[r];
    y[i] = acc;
  }
}

/* Steps 3-5 of [LCF-arch] for one token with given routing: zero-expert slots
 * (idx >= N) add gate * x (identity expert); FFN slots add gate * FFN(x).
 * wg[j], wu[j], wd[j] point at the matrices of the expert in slot j (unused
 * for zero slots).  out: d floats, in fp32. */
void oracle_token_output(int d, int I, int N, int k, const void *x_row, int dt,
                         const int32_t *idx, const float *gate, const void *const *wg,
                         const void *const *wu, const void *const *wd, float *out) {
  float *xf = (float *)malloc(sizeof(float) * (size_t)d);
  float *y = (float *)malloc(sizeof(float) * (size_t)d);
  float *h = (float *)malloc(sizeof(float) * (size_t)(I > 0 ? I : 1));
  for (int i = 0; i < d; ++i) xf[i] = orc_ld(x_row, i, dt);
  float zsum = 0.0f;
  for (int j = 0; j < k; ++j)
    if (idx[j] >= N) zsum += gate[j];
  for (int i = 0; i < d; ++i) out[i] = zsum * xf[i];
  for (int j = 0; j < k; ++j) {
    if (idx[j] >= N) continue;
    orc_expert(d, I, xf, wg[j], wu[j], wd[j], dt, h, y);
    for (int i = 0; i < d; ++i) out[i] += gate[j] * y[i];
  }
  free(xf);
  free(y);
  free(h);
}

/* Steps 3-5 for tokens [0, T) given their routing; full weight tensors
 * w_gate/w_up [N, I, d], w_down [N, d, I]. */
void oracle_combine_given_routing(int64_t T, int d, int I, int N, int k, const void *x, int dt,
                                  const int32_t *idx, const float *gate, const void *w_gate,
                                  const void *w_up, const void *w_down, float *out) {
  size_t es = dt == ORC_F32 ? 4 : 2;
  size_t per = (size_t)I * (size_t)d * es;
#pragma omp parallel
  {
    const void **pg = (const void **)malloc(sizeof(void *) * (size_t)k);
    const void **pu = (const void **)malloc(sizeof(void *) * (size_t)k);
    const void **pd = (const void **)malloc(sizeof(void *) * (size_t)k);
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      for (int j = 0; j < k; ++j) {
        int e = idx[t * k + j];
        int ffn = e < N;
        pg[j] = ffn ? (const char *)w_gate + (size_t)e * per : NULL;
        pu[j] = ffn ? (const char *)w_up + (size_t)e * per : NULL;
        pd[j] = ffn ? (const char *)w_down + (size_t)e * per : NULL;
      }
      oracle_token_output(d, I, N, k, (const char *)x + (size_t)t * (size_t)d * es, dt,
                          idx + t * k, gate + t * k, pg, pu, pd, out + t * (int64_t)d);
    }
    free(pg);
    free(pu);
    free(pd);
  }
}

/* Step 3 for a list of (token, FFN expert) pairs: y[i] = Wd (silu(Wg x) *
 * (Wu x)) for pair i, whose token row x_rows[i] (the inputs' dtype, d
 * elements) and expert matrices wg[i], wu[i] ([I, d]) and wd[i] ([d, I]) are
 * given by pointer.  The arithmetic is the per-slot expert of
 * oracle_token_output, so a check can hold a few experts in memory at a time
 * and still reproduce that function bit for bit.  y: [n, d] fp32. */
void oracle_ffn_pairs(int64_t n, int d, int I, int dt, const void *const *x_rows,
                      const void *const *wg, const void *const *wu, const void *const *wd,
                      float *y) {
#pragma omp parallel
  {
    float *xf = (float *)malloc(sizeof(float) * (size_t)d);
    float *h = (float *)malloc(sizeof(float) * (size_t)(I > 0 ? I : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
      for (int c = 0; c < d; ++c) xf[c] = orc_ld(x_rows[i], c, dt);
      orc_expert(d, I, xf, wg[i], wu[i], wd[i], dt, h, y + i * (int64_t)d);
    }
    free(xf);
    free(h);
  }
}

/* Steps 4-5 of [LCF-arch] with the FFN slots' expert outputs given:
 * out[t] = (sum of zero-slot gates) * x[t] + sum_j gate_j * y[t, j], the FFN
 * terms added in ascending slot order (the combine of oracle_token_output).
 * y_slots: [T, k, d] fp32; rows of zero slots (idx >= N) are not read. */
void oracle_combine_slots(int64_t T, int d, int N, int k, const void *x, int dt,
                          const int32_t *idx, const float *gate, const float *y_slots,
                          float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const int32_t *it = idx + t * k;
    const float *gt = gate + t * k;
    float *o = out + t * (int64_t)d;
    float zsum = 0.0f;
    for (int j = 0; j < k; ++j)
      if (it[j] >= N) zsum += gt[j];
    for (int i = 0; i < d; ++i) o[i] = zsum * orc_ld(x, t * (int64_t)d + i, dt);
    for (int j = 0; j < k; ++j) {
      if (it[j] >= N) continue;
      const float *y = y_slots + (t * (int64_t)k + j) * (int64_t)d;
      for (int i = 0; i < d; ++i) o[i] += gt[j] * y[i];
    }
  }
}

/* The whole forward: logits, routing, counts and output (fp32). */
void oracle_forward(int64_t T, int d, int I, int N, int Z, int k, int dt, const void *x,
                    const void *w_router, const float *bias, const void *w_gate,
                    const void *w_up, const void *w_down, float *out, int32_t *counts,
                    int32_t *idx, float *gate, float *margin, float routed_scale) {
  int E = N + Z;
  float *logits = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * (size_t)E);
  oracle_router_logits(T, d, E, x, w_router, dt, logits);
  oracle_route_from_logits(T, E, k, logits, bias, idx, gate, margin, NULL, routed_scale);
  oracle_counts(T, k, E, idx, counts);
  oracle_combine_given_routing(T, d, I, N, k, x, dt, idx, gate, w_gate, w_up, w_down, out);
  free(logits);
}

/* Bias controller (the step after the forward that consumes `counts`).
 * [LCF-arch] computation-budget control, and [LCF] section 1 "main
 * contributions": an expert-specific bias, adjusted by a PID controller,
 * keeps the average share of FFN vs zero experts near its target.  [KOL]:
 * the balancing is aux-loss-free, a bias update with a decaying step.  The
 * pages give no formula or gains; this is the plain incremental PID on the
 * per-token load error of each expert:
 *   e   = (target[e] - counts[e]) / T                   (selections per token)
 *   u   = ki*e + kp*(e - e1) + kd*((e - e1) - (e1 - e2))  (e1, e2: previous two e)
 *   bias[e] += lr * u                                   (mode 0)
 *   bias[e] += lr * sign(e)                             (mode 1, sign update)
 * The caller supplies lr (its decay schedule) and the per-expert target.  An
 * under-selected expert (e > 0) gets a larger bias, hence more selections.
 * state[2*E] = (e1, e2) per expert, updated in place; NULL means "no history"
 * (e1 = e2 = e).  All fp32, in this order, with no contraction. */
void oracle_bias_update(int E, int64_t T, const int32_t *counts, const float *target, float *bias,
                        float *state, float lr, float ki, float kp, float kd, int mode) {
  const float tf = (float)T;
  for (int e = 0; e < E; ++e) {
    const float err = (target[e] - (float)counts[e]) / tf;
    float step;
    if (mode == 1) {
      const float s = err > 0.0f ? 1.0f : (err < 0.0f ? -1.0f : 0.0f);
      step = lr * s;
    } else {
      const float e1 = state ? state[2 * e] : err;
      const float e2 = state ? state[2 * e + 1] : err;
      const float a = err - e1;
      const float b = e1 - e2;
      const float dd = a - b;
      float u = ki * err;
      u = u + kp * a;
      u = u + kd * dd;
      step = lr * u;
    }
    bias[e] = bias[e] + step;
    if (state) {
      state[2 * e + 1] = state[2 * e];
      state[2 * e] = err;
    }
  }
}

/* ------------------------------------------------------------------------
 * Block-scaled FP8 experts.
 * [LCF] section 6 "inference and deployment", custom kernels, quantization
 * item: fine-grained block quantization as in DeepSeek-V3, activations per
 * [1,128] block and weights per [128,128] block.  Readings (the pages name
 * neither the format nor the scale rule):
 *   - FP8 = OCP E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits,
 *     subnormals, largest finite 448, no infinities;
 *   - conversion rounds to nearest, ties to even, and saturates at +-448;
 *   - a block's scale is a power of two, the smallest 2^e >= amax / 448
 *     (e >= -127; 1 for an all-zero block), and q = E4M3(v / scale), so the
 *     block's largest magnitude lands in (224, 448] and dividing by the
 *     scale is exact.  (DeepSeek-V3 keeps fp32 scales; a power-of-two scale
 *     is one exponent byte per block, which the gfx950 FP8 matrix
 *     instructions apply in hardware, and loses at most one bit of the
 *     block's range.);
 *   - a GEMM adds, per 128-wide K block, (scale_a * scale_b) times the fp32
 *     sum of the products of the quantized values;
 *   - the router stays in the inputs' dtype; x is quantized per [1,128]
 *     before the gate/up projections, the SwiGLU activations per [1,128]
 *     before the down projection; a zero expert returns the unquantized x.
 * ------------------------------------------------------------------------ */

/* E4M3 byte of a finite fp32 value (round to nearest even, saturate). */
uint8_t oracle_e4m3_from_f32(float v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const float a = fabsf(v);
  if (a > 448.0f) return sign | 0x7E;
  if (a < 0.015625f) {                     /* below 2^-6: subnormal steps of 2^-9 */
    const float m = rintf(a * 512.0f);     /* exact scaling; rint = ties to even */
    return sign | (uint8_t)m;              /* m == 8 is the smallest normal, 0x08 */
  }
  int e;
  const float f = frexpf(a, &e);           /* a = f * 2^e, f in [0.5, 1) */
  const float mm = rintf((f * 2.0f - 1.0f) * 8.0f);  /* 3 mantissa bits, exact operands */
  int ex = e - 1 + 7, man = (int)mm;
  if (man == 8) {
    man = 0;
    ++ex;
  }
  return sign | (uint8_t)((ex << 3) | man);
}

float oracle_e4m3_to_f32(uint8_t q) {
  const int e = (q >> 3) & 15, m = q & 7;
  const float a = e == 0 ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
  return (q & 0x80) ? -a : a;
}

/* Block scale: the smallest power of two >= amax / 448, not below 2^-127;
 * 1 when amax is 0. */
static float orc_block_scale(float amax) {
  if (!(amax > 0.0f)) return 1.0f;
  int E;
  const float f = frexpf(amax / 448.0f, &E); /* r = f * 2^E, f in [0.5, 1) */
  int e = f == 0.5f ? E - 1 : E;
  if (e < -127) e = -127;
  return ldexpf(1.0f, e);
}

/* src [nmat, rows, K] (fp32 or bf16) -> q [nmat, rows, K] E4M3 bytes and
 * s [nmat, rows / block_rows, K / 128] fp32 scales (blocks of block_rows x
 * 128; block_rows = 128 for weights, 1 for activations). */
void oracle_quantize_fp8(const void *src, int dt, int64_t nmat, int rows, int K, int block_rows,
                         uint8_t *q, float *s) {
  const int nrb = rows / block_rows, nkb = K / 128;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nmat * nrb * nkb; ++b) {
    const int64_t m = b / ((int64_t)nrb * nkb);
    const int rb = (int)((b / nkb) % nrb), kb = (int)(b % nkb);
    float amax = 0.0f;
    for (int r = rb * block_rows; r < (rb + 1) * block_rows; ++r)
      for (int c = kb * 128; c < (kb + 1) * 128; ++c) {
        const float a = fabsf(orc_ld(src, (m * rows + r) * (int64_t)K + c, dt));
        amax = a > amax ? a : amax;
      }
    const float scale = orc_block_scale(amax);
    s[b] = scale;
    for (int r = rb * block_rows; r < (rb + 1) * block_rows; ++r)
      for (int c = kb * 128; c < (kb + 1) * 128; ++c) {
        const int64_t i = (m * rows + r) * (int64_t)K + c;
        q[i] = oracle_e4m3_from_f32(orc_ld(src, i, dt) / scale);
      }
  }
}

/* The value of every E4M3 byte (oracle_e4m3_to_f32 of each), so that the
 * dot products below look values up instead of decoding each byte again. */
static void orc_e4m3_table(float *lut) {
  for (int q = 0; q < 256; ++q) lut[q] = oracle_e4m3_to_f32((uint8_t)q);
}

/* One row of a block-scaled GEMM: sum over K blocks of
 * (sa[kb] * sb[kb]) * (sum of the quantized products in the block).
 * lut: orc_e4m3_table. */
static float orc_dot_fp8(int K, const uint8_t *qa, const float *sa, const uint8_t *qb,
                         const float *sb, const float *lut) {
  float acc = 0.0f;
  for (int kb = 0; kb < K / 128; ++kb) {
    float blk = 0.0f;
    for (int c = kb * 128; c < (kb + 1) * 128; ++c) blk += lut[qa[c]] * lut[qb[c]];
    const float sc = sa[kb] * sb[kb];
    acc += blk * sc;
  }
  return acc;
}

/* Quantize one fp32 row of K (multiple of 128) per [1,128] block. */
static void orc_quant_row(int K, const float *v, uint8_t *q, float *s) {
  for (int kb = 0; kb < K / 128; ++kb) {
    float amax = 0.0f;
    for (int c = kb * 128; c < (kb + 1) * 128; ++c) amax = fabsf(v[c]) > amax ? fabsf(v[c]) : amax;
    const float scale = orc_block_scale(amax);
    s[kb] = scale;
    for (int c = kb * 128; c < (kb + 1) * 128; ++c) q[c] = oracle_e4m3_from_f32(v[c] / scale);
  }
}

/* One FFN expert on a quantized token: g, u (block-scaled GEMMs against
 * W_gate/W_up, scales [I/128, d/128]), h = silu(g) * u, h quantized per
 * [1,128], y = block-scaled GEMM against W_down (scales [d/128, I/128]). */
static void orc_expert_fp8(int d, int I, const uint8_t *qx, const float *sx, const uint8_t *qwg,
                           const float *swg, const uint8_t *qwu, const float *swu,
                           const uint8_t *qwd, const float *swd, float *h, uint8_t *qh,
                           float *sh, float *y) {
  const int dkb = d / 128, ikb = I / 128;
  float lut[256];
  orc_e4m3_table(lut);
  for (int r = 0; r < I; ++r) {
    const float g =
        orc_dot_fp8(d, qwg + (int64_t)r * d, swg + (int64_t)(r / 128) * dkb, qx, sx, lut);
    const float u =
        orc_dot_fp8(d, qwu + (int64_t)r * d, swu + (int64_t)(r / 128) * dkb, qx, sx, lut);
    h[r] = (g / (1.0f + expf(-g))) * u;
  }
  orc_quant_row(I, h, qh, sh);
  for (int i = 0; i < d; ++i)
    y[i] = orc_dot_fp8(I, qwd + (int64_t)i * I, swd + (int64_t)(i / 128) * ikb, qh, sh, lut);
}

/* Steps 3-5 for one token with given routing, FP8 experts.  Pointer arrays
 * hold, per slot j, the expert's quantized matrices and scales (unused for
 * zero slots).  x_row in the inputs' dtype; out: d floats. */
void oracle_token_output_fp8(int d, int I, int N, int k, const void *x_row, int dt,
                             const int32_t *idx, const float *gate, const uint8_t *const *qwg,
                             const float *const *swg, const uint8_t *const *qwu,
                             const float *const *swu, const uint8_t *const *qwd,
                             const float *const *swd, float *out) {
  float *x = (float *)malloc(sizeof(float) * (size_t)d);
  uint8_t *qx = (uint8_t *)malloc((size_t)d);
  float *sx = (float *)malloc(sizeof(float) * (size_t)(d / 128));
  float *h = (float *)malloc(sizeof(float) * (size_t)(I > 0 ? I : 1));
  uint8_t *qh = (uint8_t *)malloc((size_t)(I > 0 ? I : 1));
  float *sh = (float *)malloc(sizeof(float) * (size_t)(I / 128 > 0 ? I / 128 : 1));
  float *y = (float *)malloc(sizeof(float) * (size_t)d);
  for (int c = 0; c < d; ++c) x[c] = orc_ld(x_row, c, dt);
  orc_quant_row(d, x, qx, sx);
  float zsum = 0.0f;
  for (int j = 0; j < k; ++j)
    if (idx[j] >= N) zsum += gate[j];
  for (int c = 0; c < d; ++c) out[c] = zsum * x[c];
  for (int j = 0; j < k; ++j) {
    if (idx[j] >= N) continue;
    orc_expert_fp8(d, I, qx, sx, qwg[j], swg[j], qwu[j], swu[j], qwd[j], swd[j], h, qh, sh, y);
    for (int c = 0; c < d; ++c) out[c] += gate[j] * y[c];
  }
  free(x);
  free(qx);
  free(sx);
  free(h);
  free(qh);
  free(sh);
  free(y);
}

/* Step 3 with FP8 experts for a list of (token, FFN expert) pairs: pair i's
 * token row (the inputs' dtype) is quantized per [1,128] and run through its
 * expert's quantized matrices, exactly as one FFN slot of
 * oracle_token_output_fp8.  y: [n, d] fp32. */
void oracle_ffn_pairs_fp8(int64_t n, int d, int I, int dt, const void *const *x_rows,
                          const uint8_t *const *qwg, const float *const *swg,
                          const uint8_t *const *qwu, const float *const *swu,
                          const uint8_t *const *qwd, const float *const *swd, float *y) {
#pragma omp parallel
  {
    float *x = (float *)malloc(sizeof(float) * (size_t)d);
    uint8_t *qx = (uint8_t *)malloc((size_t)d);
    float *sx = (float *)malloc(sizeof(float) * (size_t)(d / 128 > 0 ? d / 128 : 1));
    float *h = (float *)malloc(sizeof(float) * (size_t)(I > 0 ? I : 1));
    uint8_t *qh = (uint8_t *)malloc((size_t)(I > 0 ? I : 1));
    float *sh = (float *)malloc(sizeof(float) * (size_t)(I / 128 > 0 ? I / 128 : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
      for (int c = 0; c < d; ++c) x[c] = orc_ld(x_rows[i], c, dt);
      orc_quant_row(d, x, qx, sx);
      orc_expert_fp8(d, I, qx, sx, qwg[i], swg[i], qwu[i], swu[i], qwd[i], swd[i], h, qh, sh,
                     y + i * (int64_t)d);
    }
    free(x);
    free(qx);
    free(sx);
    free(h);
    free(qh);
    free(sh);
  }
}

/* All tokens with given routing; weights q [N, rows, K] with scales
 * [N, rows/128, K/128] (W_gate/W_up rows I, K d; W_down rows d, K I). */
void oracle_combine_given_routing_fp8(int64_t T, int d, int I, int N, int k, const void *x, int dt,
                                      const int32_t *idx, const float *gate, const uint8_t *qwg,
                                      const float *swg, const uint8_t *qwu, const float *swu,
                                      const uint8_t *qwd, const float *swd, float *out) {
  const size_t es = dt == ORC_F32 ? 4 : 2;
  const size_t per = (size_t)I * (size_t)d, sper = (size_t)(I / 128) * (size_t)(d / 128);
#pragma omp parallel
  {
    const uint8_t **pg = (const uint8_t **)malloc(sizeof(void *) * (size_t)k);
    const uint8_t **pu = (const uint8_t **)malloc(sizeof(void *) * (size_t)k);
    const uint8_t **pd = (const uint8_t **)malloc(sizeof(void *) * (size_t)k);
    const float **sg = (const float **)malloc(sizeof(void *) * (size_t)k);
    const float **su = (const float **)malloc(sizeof(void *) * (size_t)k);
    const float **sd = (const float **)malloc(sizeof(void *) * (size_t)k);
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      for (int j = 0; j < k; ++j) {
        const int e = idx[t * k + j];
        const int ffn = e < N;
        pg[j] = ffn ? qwg + (size_t)e * per : NULL;
        pu[j] = ffn ? qwu + (size_t)e * per : NULL;
        pd[j] = ffn ? qwd + (size_t)e * per : NULL;
        sg[j] = ffn ? swg + (size_t)e * sper : NULL;
        su[j] = ffn ? swu + (size_t)e * sper : NULL;
        sd[j] = ffn ? swd + (size_t)e * sper : NULL;
      }
      oracle_token_output_fp8(d, I, N, k, (const char *)x + (size_t)t * (size_t)d * es, dt,
                              idx + t * k, gate + t * k, pg, sg, pu, su, pd, sd,
                              out + t * (int64_t)d);
    }
    free(pg);
    free(pu);
    free(pd);
    free(sg);
    free(su);
    free(sd);
  }
}

/* The whole FP8-expert forward: routing as in oracle_forward, then the
 * block-scaled experts. */
void oracle_forward_fp8(int64_t T, int d, int I, int N, int Z, int k, int dt, const void *x,
                        const void *w_router, const float *bias, const uint8_t *qwg,
                        const float *swg, const uint8_t *qwu, const float *swu,
                        const uint8_t *qwd, const float *swd, float *out, int32_t *counts,
                        int32_t *idx, float *gate, float *margin, float routed_scale) {
  int E = N + Z;
  float *logits = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * (size_t)E);
  oracle_router_logits(T, d, E, x, w_router, dt, logits);
  oracle_route_from_logits(T, E, k, logits, bias, idx, gate, margin, NULL, routed_scale);
  oracle_counts(T, k, E, idx, counts);
  oracle_combine_given_routing_fp8(T, d, I, N, k, x, dt, idx, gate, qwg, swg, qwu, swu, qwd, swd,
                                   out);
  free(logits);
}

/* ------------------------------------------------------------------------
 * Backward of the block (training).
 * [LCF] section 5 "training infrastructure": the backward's grouped GEMMs,
 * the weight-gradient GEMMs with the fp32 accumulation fused into them
 * ("GemmAdd") and a deterministic scatter-add for gradient aggregation.
 * The pages give the kernels, not the formulas; the formulas are the chain
 * rule applied to the forward above, with the routing held fixed (the
 * top-k selection and the bias are not differentiated; the bias moves only
 * through the controller):
 *   zero slot j:  dgate_j = <dout, x>;                dx += gate_j dout
 *   FFN slot j, expert e (g = Wg x, u = Wu x, s = sigmoid(g), h = g s u):
 *     v = Wd^T dout;  dgate_j = <v, h>;  dh = gate_j v;
 *     dg = dh u s (1 + g (1 - s));  du = dh g s;
 *     dx += Wg^T dg + Wu^T du;
 *     dWd[e] += (gate_j dout) h^T;  dWg[e] += dg x^T;  dWu[e] += du x^T
 *   router (p = softmax(l), gate_j = routed_scale * p[idx_j]):
 *     dp[e] = routed_scale * dgate_j where idx_j = e, else 0;
 *     dl = p * (dp - <p, dp>);  dx += Wr^T dl;  dWr += dl x^T
 * Weight gradients are accumulated into the caller's fp32 arrays.  Every sum
 * runs in ascending index order; weight gradients add tokens in ascending
 * order.
 * ------------------------------------------------------------------------ */

/* One token: dx (d floats), dgate (k), dl (E: gradient of the router
 * logits); per-slot h, dg, du ([k, I] each, rows of zero slots untouched).
 * wg/wu/wd[j]: the matrices of the expert in slot j (unused for zero slots). */
void oracle_token_backward(int d, int I, int N, int E, int k, const void *x_row, int dt,
                           const void *w_router, const int32_t *idx, const float *gate,
                           const float *dout, const void *const *wg, const void *const *wu,
                           const void *const *wd, float *dx, float *dgate, float *dl,
                           float *h_s, float *dg_s, float *du_s, float routed_scale) {
  float *x = (float *)malloc(sizeof(float) * (size_t)d);
  float *l = (float *)malloc(sizeof(float) * (size_t)E);
  float *p = (float *)malloc(sizeof(float) * (size_t)E);
  float *dp = (float *)malloc(sizeof(float) * (size_t)E);
  for (int c = 0; c < d; ++c) x[c] = orc_ld(x_row, c, dt);
  /* forward quantities: logits and probabilities of this token */
  for (int e = 0; e < E; ++e) {
    float acc = 0.0f;
    for (int c = 0; c < d; ++c) acc += x[c] * orc_ld(w_router, (int64_t)e * d + c, dt);
    l[e] = acc;
  }
  orc_softmax(E, l, p);
  float zsum = 0.0f;
  for (int j = 0; j < k; ++j)
    if (idx[j] >= N) zsum += gate[j];
  for (int c = 0; c < d; ++c) dx[c] = zsum * dout[c];
  for (int j = 0; j < k; ++j) {
    const int e = idx[j];
    if (e >= N) {
      float acc = 0.0f;
      for (int c = 0; c < d; ++c) acc += dout[c] * x[c];
      dgate[j] = acc;
      continue;
    }
    float *h = h_s + (int64_t)j * I, *dg = dg_s + (int64_t)j * I, *du = du_s + (int64_t)j * I;
    float dgj = 0.0f;
    for (int r = 0; r < I; ++r) {
      float g = 0.0f, u = 0.0f, vr = 0.0f;
      for (int c = 0; c < d; ++c) {
        g += orc_ld(wg[j], (int64_t)r * d + c, dt) * x[c];
        u += orc_ld(wu[j], (int64_t)r * d + c, dt) * x[c];
      }
      for (int c = 0; c < d; ++c) vr += orc_ld(wd[j], (int64_t)c * I + r, dt) * dout[c];
      const float s = 1.0f / (1.0f + expf(-g));
      h[r] = g * s * u;
      dgj += vr * h[r];
      const float dh = gate[j] * vr;
      dg[r] = dh * u * s * (1.0f + g * (1.0f - s));
      du[r] = dh * g * s;
    }
    dgate[j] = dgj;
    for (int c = 0; c < d; ++c) {
      float acc = dx[c];
      for (int r = 0; r < I; ++r) acc += orc_ld(wg[j], (int64_t)r * d + c, dt) * dg[r];
      for (int r = 0; r < I; ++r) acc += orc_ld(wu[j], (int64_t)r * d + c, dt) * du[r];
      dx[c] = acc;
    }
  }
  /* router: softmax backward through the selected gates */
  for (int e = 0; e < E; ++e) dp[e] = 0.0f;
  for (int j = 0; j < k; ++j) dp[idx[j]] = routed_scale * dgate[j]; /* gate_j = scale * p */
  float pdp = 0.0f;
  for (int e = 0; e < E; ++e) pdp += p[e] * dp[e];
  for (int e = 0; e < E; ++e) dl[e] = p[e] * (dp[e] - pdp);
  for (int c = 0; c < d; ++c) {
    float acc = 0.0f;
    for (int e = 0; e < E; ++e) acc += orc_ld(w_router, (int64_t)e * d + c, dt) * dl[e];
    dx[c] += acc;
  }
  free(x);
  free(l);
  free(p);
  free(dp);
}

/* The whole backward for tokens [0, T) with given routing (idx, gate from
 * the forward) and output gradient dout [T, d] (fp32).  dx [T, d] is
 * overwritten; dw_router [E, d], dw_gate / dw_up [N, I, d] and dw_down
 * [N, d, I] (fp32) are accumulated into. */
void oracle_backward(int64_t T, int d, int I, int N, int Z, int k, int dt, const void *x,
                     const void *w_router, const void *w_gate, const void *w_up,
                     const void *w_down, const int32_t *idx, const float *gate,
                     const float *dout, float *dx, float *dw_router, float *dw_gate,
                     float *dw_up, float *dw_down, float routed_scale) {
  const int E = N + Z;
  const size_t es = dt == ORC_F32 ? 4 : 2;
  const size_t per = (size_t)I * (size_t)d * es;
  const size_t Ts = (size_t)(T > 0 ? T : 1), Is = (size_t)(I > 0 ? I : 1);
  float *dl = (float *)malloc(sizeof(float) * Ts * (size_t)E);
  float *dgate = (float *)malloc(sizeof(float) * Ts * (size_t)k);
  float *h = (float *)malloc(sizeof(float) * Ts * (size_t)k * Is);
  float *dg = (float *)malloc(sizeof(float) * Ts * (size_t)k * Is);
  float *du = (float *)malloc(sizeof(float) * Ts * (size_t)k * Is);
#pragma omp parallel
  {
    const void **pg = (const void **)malloc(sizeof(void *) * (size_t)k);
    const void **pu = (const void **)malloc(sizeof(void *) * (size_t)k);
    const void **pd = (const void **)malloc(sizeof(void *) * (size_t)k);
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      for (int j = 0; j < k; ++j) {
        const int e = idx[t * k + j];
        const int ffn = e < N;
        pg[j] = ffn ? (const char *)w_gate + (size_t)e * per : NULL;
        pu[j] = ffn ? (const char *)w_up + (size_t)e * per : NULL;
        pd[j] = ffn ? (const char *)w_down + (size_t)e * per : NULL;
      }
      const size_t so = (size_t)t * (size_t)k * Is;
      oracle_token_backward(d, I, N, E, k, (const char *)x + (size_t)t * (size_t)d * es, dt,
                            w_router, idx + t * k, gate + t * k, dout + t * (int64_t)d, pg, pu,
                            pd, dx + t * (int64_t)d, dgate + t * k, dl + t * (int64_t)E, h + so,
                            dg + so, du + so, routed_scale);
    }
    free(pg);
    free(pu);
    free(pd);
  }
  /* expert weight gradients, one expert at a time, tokens ascending */
#pragma omp parallel for schedule(dynamic, 1)
  for (int e = 0; e < N; ++e) {
    float *gwg = dw_gate + (int64_t)e * I * d, *gwu = dw_up + (int64_t)e * I * d;
    float *gwd = dw_down + (int64_t)e * d * I;
    for (int64_t t = 0; t < T; ++t) {
      for (int j = 0; j < k; ++j) {
        if (idx[t * k + j] != e) continue;
        const size_t so = ((size_t)t * (size_t)k + (size_t)j) * Is;
        for (int r = 0; r < I; ++r)
          for (int c = 0; c < d; ++c) {
            const float xc = orc_ld(x, t * (int64_t)d + c, dt);
            gwg[(int64_t)r * d + c] += dg[so + r] * xc;
            gwu[(int64_t)r * d + c] += du[so + r] * xc;
          }
        const float gt = gate[t * k + j];
        for (int c = 0; c < d; ++c) {
          const float dy = gt * dout[t * (int64_t)d + c];
          for (int r = 0; r < I; ++r) gwd[(int64_t)c * I + r] += dy * h[so + r];
        }
      }
    }
  }
  /* router weight gradient, tokens ascending */
#pragma omp parallel for schedule(static)
  for (int e = 0; e < E; ++e)
    for (int64_t t = 0; t < T; ++t) {
      const float g = dl[t * (int64_t)E + e];
      for (int c = 0; c < d; ++c)
        dw_router[(int64_t)e * d + c] += g * orc_ld(x, t * (int64_t)d + c, dt);
    }
  free(dl);
  free(dgate);
  free(h);
  free(dg);
  free(du);
}

/* Rows of one expert's weight gradients from the tokens routed to it (for
 * sampled checks at sizes where the whole backward is too slow): given the
 * n routed tokens' x (dtype, [n, d]), dout ([n, d] fp32) and gates, in
 * ascending token order, the gradient contributions of this call for row r:
 * dwg_row = dWg[e][r, :], dwu_row = dWu[e][r, :] (d floats each) and
 * dwd_col = dWd[e][:, r] (d floats), each summed over the n tokens. */
void oracle_expert_wgrad_row(int d, int I, int n, const void *x_rows, int dt,
                             const float *dout_rows, const float *gates, const void *wg,
                             const void *wu, const void *wd, int r, float *dwg_row,
                             float *dwu_row, float *dwd_col) {
  for (int c = 0; c < d; ++c) dwg_row[c] = dwu_row[c] = dwd_col[c] = 0.0f;
  for (int i = 0; i < n; ++i) {
    float g = 0.0f, u = 0.0f, vr = 0.0f;
    for (int c = 0; c < d; ++c) {
      const float xc = orc_ld(x_rows, (int64_t)i * d + c, dt);
      g += orc_ld(wg, (int64_t)r * d + c, dt) * xc;
      u += orc_ld(wu, (int64_t)r * d + c, dt) * xc;
    }
    for (int c = 0; c < d; ++c) vr += orc_ld(wd, (int64_t)c * I + r, dt) * dout_rows[(int64_t)i * d + c];
    const float s = 1.0f / (1.0f + expf(-g));
    const float h = g * s * u;
    const float dh = gates[i] * vr;
    const float dg = dh * u * s * (1.0f + g * (1.0f - s));
    const float du = dh * g * s;
    for (int c = 0; c < d; ++c) {
      const float xc = orc_ld(x_rows, (int64_t)i * d + c, dt);
      dwg_row[c] += dg * xc;
      dwu_row[c] += du * xc;
      dwd_col[c] += gates[i] * dout_rows[(int64_t)i * d + c] * h;
    }
  }
}

/* The dense FFN path of the layer ([LCF] section 2, shortcut-connected MoE
 * and the model-configuration paragraph: a dense SwiGLU FFN block beside the
 * MoE, intermediate width 12288 at the production shape):
 * out[t] = W2 (silu(W1 x[t]) * (W3 x[t])), W1 / W3 [I, d], W2 [d, I]. */
void oracle_dense_ffn(int64_t T, int d, int I, const void *x, int dt, const void *w1,
                      const void *w3, const void *w2, float *out) {
  const size_t es = dt == ORC_F32 ? 4 : 2;
#pragma omp parallel
  {
    float *xf = (float *)malloc(sizeof(float) * (size_t)d);
    float *h = (float *)malloc(sizeof(float) * (size_t)(I > 0 ? I : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      const void *xr = (const char *)x + (size_t)t * (size_t)d * es;
      for (int c = 0; c < d; ++c) xf[c] = orc_ld(xr, c, dt);
      orc_expert(d, I, xf, w1, w3, w2, dt, h, out + t * (int64_t)d);
    }
    free(xf);
    free(h);
  }
}
