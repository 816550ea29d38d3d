// bias.hip -- the bias controller that consumes the forward's per-expert
// selection counts.
//
// LongCat-Flash technical-report summary page, section 2 "architecture",
// computation-budget control (and section 1, main contributions): an
// expert-specific bias, adjusted by a PID controller, keeps the average
// share of FFN vs zero-computation experts near its target.  The cnouyi.fund
// thread on the same report describes the balancing as aux-loss-free, with a
// decaying update.  The pages give no formula or gains; this library's
// reading is an incremental PID on each expert's per-token load error,
//   e = (target[e] - counts[e]) / T,
//   u = ki*e + kp*(e - e1) + kd*((e - e1) - (e1 - e2)),   bias[e] += lr*u,
// or, in sign mode, bias[e] += lr*sign(e).  One thread per expert, fp32 in
// exactly that order with no contraction, so the result is bit-reproducible.
#include "moe_zc.h"
#include "moe_zc_internal.h"

#include <cmath>

namespace moezc {

__global__ void __launch_bounds__(256)
    bias_update_kernel(int E, float tf, const int32_t *__restrict__ counts,
                       const float *__restrict__ target, float *__restrict__ bias,
                       float *__restrict__ state, float lr, float ki, float kp, float kd, int mode) {
#pragma clang fp contract(off)
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const float err = (target[e] - static_cast<float>(counts[e])) / tf;
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

}  // namespace moezc

extern "C" int moe_zc_bias_update(int32_t E, int64_t T, const int32_t *counts, const float *target,
                                  float *bias, float *state, float lr, float ki, float kp, float kd,
                                  int32_t mode, void *stream) {
  if (E < 1 || T < 1 || !counts || !target || !bias || (mode != 0 && mode != 1))
    return MOE_ZC_EINVAL;
  if (!std::isfinite(lr) || !std::isfinite(ki) || !std::isfinite(kp) || !std::isfinite(kd))
    return MOE_ZC_EINVAL;
  const uintptr_t mis = (reinterpret_cast<uintptr_t>(counts) | reinterpret_cast<uintptr_t>(target) |
                         reinterpret_cast<uintptr_t>(bias) | reinterpret_cast<uintptr_t>(state)) & 3u;
  if (mis) return MOE_ZC_EALIGN;
  const unsigned grid = static_cast<unsigned>((static_cast<int64_t>(E) + 255) / 256);
  hipLaunchKernelGGL(moezc::bias_update_kernel, dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), E, static_cast<float>(T), counts, target,
                     bias, state, lr, ki, kp, kd, mode);
  return hipGetLastError() == hipSuccess ? MOE_ZC_OK : MOE_ZC_EHIP;
}
