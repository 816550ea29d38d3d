/*
 * synth_gpu.hip -- device build of the seeded input generator (see
 * synth_rng.h for its definition).  Fills device buffers on a stream; values
 * are bit-identical to the host build.  Holds none of the MoE method's
 * arithmetic.  Compiled with -ffp-contract=off.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_rng.h"

__global__ void __launch_bounds__(256) syn_normal_kernel(float *out_f32, uint16_t *out_bf16,
                                                         int64_t first, int64_t count,
                                                         uint64_t seed, uint64_t tid,
                                                         double sigma) {
  int64_t b0 = first / 4;
  int64_t nblk = (first + count - 1) / 4 - b0 + 1;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nblk;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t b = b0 + i;
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

__global__ void __launch_bounds__(256) syn_uniform_kernel(float *out, int64_t first, int64_t count,
                                                          uint64_t seed, uint64_t tid, double lo,
                                                          double hi) {
  int64_t b0 = first / 4;
  int64_t nblk = (first + count - 1) / 4 - b0 + 1;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nblk;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t b = b0 + i;
    double u[4];
    syn_uniform4(seed, tid, (uint64_t)b, u);
    for (int w = 0; w < 4; ++w) {
      int64_t flat = b * 4 + w;
      if (flat < first || flat >= first + count) continue;
      out[flat - first] = (float)(lo + (hi - lo) * u[w]);
    }
  }
}

static unsigned syn_grid(int64_t nblk) {
  int64_t g = (nblk + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

extern "C" int syn_normal_fill_device(float *out_f32, uint16_t *out_bf16, int64_t first,
                                      int64_t count, uint64_t seed, uint64_t tid, double sigma,
                                      void *stream) {
  if (count <= 0) return 0;
  if ((out_f32 == nullptr) == (out_bf16 == nullptr)) return -1;
  int64_t nblk = (first + count - 1) / 4 - first / 4 + 1;
  hipLaunchKernelGGL(syn_normal_kernel, dim3(syn_grid(nblk)), dim3(256), 0,
                     (hipStream_t)stream, out_f32, out_bf16, first, count, seed, tid, sigma);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int syn_uniform_fill_device(float *out, int64_t first, int64_t count, uint64_t seed,
                                       uint64_t tid, double lo, double hi, void *stream) {
  if (count <= 0) return 0;
  int64_t nblk = (first + count - 1) / 4 - first / 4 + 1;
  hipLaunchKernelGGL(syn_uniform_kernel, dim3(syn_grid(nblk)), dim3(256), 0,
                     (hipStream_t)stream, out, first, count, seed, tid, lo, hi);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
