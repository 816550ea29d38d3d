// fp8.hip -- block quantization to E4M3 with power-of-two block scales.
//
// LongCat-Flash technical-report summary page, section 6 "inference and
// deployment", custom kernels, quantization item: DeepSeek-V3-style blocks,
// activations per [1,128], weights per [128,128].  This library's reading:
// a block's scale is the smallest power of two 2^e >= amax / 448 (e >= -127;
// e = 0 for an all-zero block), stored as the E8M0 byte e + 127; each value
// becomes E4M3(v * 2^-e), rounded to nearest even (the gfx950 conversion
// instruction; the scaling by a power of two is exact).
//   weights:     [nmat, rows, K] -> blocks of 128 rows x 128 columns
//   activations: [rows, K]       -> blocks of 1 row x 128 columns
#include "moe_zc.h"
#include "moe_zc_internal.h"

namespace moezc {

// Smallest power of two >= amax / 448 as an exponent, clamped to -127; 0
// when amax is 0.
__device__ __forceinline__ int quant_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  const float r = amax / 448.0f;
  const uint32_t b = __float_as_uint(r);
  const int ex = static_cast<int>((b >> 23) & 0xFF);
  const uint32_t man = b & 0x7FFFFFu;
  int e;
  if (ex == 0) {  // subnormal ratio man * 2^-149
    const int lg = 31 - __clz(man);
    e = (man == (1u << lg) ? lg : lg + 1) - 149;
  } else {
    e = ex - 127 + (man != 0u ? 1 : 0);
  }
  return e < -127 ? -127 : e;
}

__device__ __forceinline__ float exp2_neg(int e) {  // 2^-e, e in [-127, 127]
  return e <= 126 ? __uint_as_float(static_cast<uint32_t>(127 - e) << 23)
                  : __uint_as_float(1u << 22);
}

template <typename T>
__device__ __forceinline__ void load8(const T *p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t *p, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4 *>(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float *p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ uint2 pack8_e4m3(const float (&v)[8], float inv) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * inv, v[1] * inv, 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * inv, v[3] * inv, lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4] * inv, v[5] * inv, 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6] * inv, v[7] * inv, hi, true);
  return make_uint2(static_cast<uint32_t>(lo), static_cast<uint32_t>(hi));
}

// One workgroup (256 threads) per 128 x 128 block: thread t covers row t / 2,
// columns (t % 2) * 64 .. + 63 of the block.
template <typename T>
__global__ void __launch_bounds__(256) quant_w_kernel(const T *__restrict__ src, int rows, int K,
                                                      uint8_t *__restrict__ q,
                                                      uint8_t *__restrict__ sexp) {
  __shared__ float s_max[4];
  const int nrb = rows / 128, nkb = K / 128;
  const int64_t b = blockIdx.x;
  const int64_t m = b / (static_cast<int64_t>(nrb) * nkb);
  const int rb = static_cast<int>((b / nkb) % nrb), kb = static_cast<int>(b % nkb);
  const int row = rb * 128 + (threadIdx.x >> 1);
  const int col = kb * 128 + (threadIdx.x & 1) * 64;
  const int64_t base = (m * rows + row) * static_cast<int64_t>(K) + col;
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    load8<T>(src + base + i * 8, v[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const int e = quant_exponent(amax);
  const float inv = exp2_neg(e);
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<uint2 *>(q + base + i * 8) = pack8_e4m3(v[i], inv);
  if (threadIdx.x == 0) sexp[b] = static_cast<uint8_t>(e + 127);
}

// Activations: one 16-lane group per [1,128] block (8 values per lane); a
// workgroup of 256 threads covers 16 blocks, in row-major block order.
template <typename T>
__global__ void __launch_bounds__(256) quant_rows_kernel(const T *__restrict__ src, int64_t nblocks,
                                                         int K, uint8_t *__restrict__ q,
                                                         uint8_t *__restrict__ sexp) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  if (b >= nblocks) return;  // uniform within the 16-lane group
  const int nkb = K / 128;
  const int64_t row = b / nkb;
  const int kb = static_cast<int>(b % nkb);
  const int64_t base = row * K + kb * 128 + (threadIdx.x & 15) * 8;
  float v[8];
  load8<T>(src + base, v);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
  const int e = quant_exponent(amax);
  *reinterpret_cast<uint2 *>(q + base) = pack8_e4m3(v, exp2_neg(e));
  if ((threadIdx.x & 15) == 0) sexp[b] = static_cast<uint8_t>(e + 127);
}

static hipError_t launch_quant(const void *src, int dtype, int64_t nmat, int rows, int K,
                               int block_rows, uint8_t *q, uint8_t *sexp, hipStream_t s) {
  if (block_rows == 128) {
    const int64_t nblk = nmat * (rows / 128) * (K / 128);
    if (nblk == 0) return hipSuccess;
    if (dtype == MOE_ZC_BF16)
      hipLaunchKernelGGL(quant_w_kernel<bf16_t>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0,
                         s, static_cast<const bf16_t *>(src), rows, K, q, sexp);
    else
      hipLaunchKernelGGL(quant_w_kernel<float>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0,
                         s, static_cast<const float *>(src), rows, K, q, sexp);
  } else {
    const int64_t nblk = nmat * rows * (K / 128);
    if (nblk == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>((nblk + 15) / 16);
    if (dtype == MOE_ZC_BF16)
      hipLaunchKernelGGL(quant_rows_kernel<bf16_t>, dim3(grid), dim3(256), 0, s,
                         static_cast<const bf16_t *>(src), nblk, K, q, sexp);
    else
      hipLaunchKernelGGL(quant_rows_kernel<float>, dim3(grid), dim3(256), 0, s,
                         static_cast<const float *>(src), nblk, K, q, sexp);
  }
  return hipGetLastError();
}

// x's exponents in permuted row order, K-block-major: sxp[kb * ldt + row] =
// sx[tok[row] * nkb + kb] for the P = meta[1] permuted rows, one thread per
// row (consecutive threads on consecutive rows, so each store instruction
// writes consecutive bytes), so that the expert GEMMs read one step's
// exponents of a tile's rows as consecutive bytes.  A row's nkb source bytes
// are read 16 at a time when nkb is a multiple of 16 (then every source row
// is 16-byte aligned).  One thread per byte instead: 17 us at prod.
__global__ void __launch_bounds__(256) gather_exp_kernel(const uint8_t *__restrict__ sx,
                                                         const int32_t *__restrict__ tok,
                                                         const int32_t *__restrict__ meta,
                                                         int nkb, int64_t ldt,
                                                         uint8_t *__restrict__ sxp) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (row >= meta[1]) return;
  const uint8_t *src = sx + static_cast<int64_t>(tok[row]) * nkb;
  if ((nkb & 15) == 0) {
    for (int kb0 = 0; kb0 < nkb; kb0 += 16) {
      const uint4 v = *reinterpret_cast<const uint4 *>(src + kb0);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 16; ++i)
        sxp[static_cast<int64_t>(kb0 + i) * ldt + row] =
            static_cast<uint8_t>(w[i >> 2] >> ((i & 3) * 8));
    }
  } else {
    for (int kb = 0; kb < nkb; ++kb) sxp[static_cast<int64_t>(kb) * ldt + row] = src[kb];
  }
}

// The forward's activation quantization: x [T, d] -> qx, sx, then sx's rows
// gathered into the experts' permuted row order.
hipError_t launch_quant_x(const Plan &p, hipStream_t s) {
  hipError_t e = launch_quant(p.x, p.dtype, 1, static_cast<int>(p.T), p.d, 1,
                              static_cast<uint8_t *>(p.qx), p.sx, s);
  if (e != hipSuccess || p.pmax == 0) return e;
  const int nkb = p.d / 128;
  hipLaunchKernelGGL(gather_exp_kernel, dim3(static_cast<unsigned>((p.pmax + 255) / 256)),
                     dim3(256), 0, s, p.sx, p.tok, p.meta, nkb, p.pmax, p.sxp);
  return hipGetLastError();
}

}  // namespace moezc

extern "C" int moe_zc_quantize_fp8(const void *src, int32_t dtype, int64_t nmat, int32_t rows,
                                   int32_t K, int32_t block_rows, uint8_t *q, uint8_t *scale_exp,
                                   void *stream) {
  if (dtype != MOE_ZC_F32 && dtype != MOE_ZC_BF16) return MOE_ZC_EDTYPE;
  if (nmat < 0 || rows < 0 || K < 0 || (block_rows != 1 && block_rows != 128)) return MOE_ZC_EINVAL;
  if (rows % block_rows != 0 || K % 128 != 0) return MOE_ZC_EALIGN;
  if (nmat == 0 || rows == 0 || K == 0) return MOE_ZC_OK;
  if (!src || !q || !scale_exp) return MOE_ZC_EINVAL;
  const int64_t blocks = nmat * (rows / block_rows) * (K / 128);
  if (block_rows == 128 && blocks >= (int64_t(1) << 31)) return MOE_ZC_EINVAL;
  if (block_rows == 1 && (blocks + 15) / 16 >= (int64_t(1) << 31)) return MOE_ZC_EINVAL;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(q)) & 15) return MOE_ZC_EALIGN;
  return moezc::launch_quant(src, dtype, nmat, rows, K, block_rows, q, scale_exp,
                             static_cast<hipStream_t>(stream)) == hipSuccess
             ? MOE_ZC_OK
             : MOE_ZC_EHIP;
}
