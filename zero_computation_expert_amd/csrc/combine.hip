// combine.hip -- steps 4-5 of the zero-computation-expert MoE forward:
//   out[t] = (sum of gates of zero-expert slots) * x[t] + sum_j gate_j * Y[rowmap[t, j]]
// A zero-computation expert returns its input and costs nothing (LongCat-Flash
// summary page, section 2 "architecture", item 1), so its whole contribution
// folds into one scale of x.  FFN terms are added in ascending slot order in
// fp32 and rounded once; no atomics, so the output is run-to-run identical
// (the same page, section 1, asks for deterministic computation).
#include "moe_zc_internal.h"

namespace moezc {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec16;  // 16 bytes of T
template <>
struct Vec16<bf16_t> {
  static constexpr int n = 8;
  static __device__ __forceinline__ void unpack(const uint4 &v, float *f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float *f) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <>
struct Vec16<float> {
  static constexpr int n = 4;
  static __device__ __forceinline__ void unpack(const uint4 &v, float *f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  static __device__ __forceinline__ uint4 pack(const float *f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};

// One block per token; each thread handles 16-byte column pieces.
constexpr int kRsrcFlags = 0x00020000;  // buffer descriptor word 3 for plain byte-addressed loads
constexpr int kNonTemporal = 2;         // buffer-load cache policy: non-temporal
// kBatch: Y loads in flight per thread (one batch of slots), the smallest
// of 4, 8, 12, 16 that holds k (16 beyond).  Loads for slots past k are
// empty ranges and cost issue slots only: kBatch = 12 at k = 12 (one batch
// instead of 8 + 4) made prod 2% and decode 10% faster than 8, while 12 at
// k = 6 was 10% slower than 8.
template <typename T, int kBatch>
__global__ void __launch_bounds__(256) combine_kernel(const T *__restrict__ x,
                                                      const T *__restrict__ y,
                                                      const int32_t *__restrict__ rowmap,
                                                      const float *__restrict__ gate, int d,
                                                      int k, T *__restrict__ out) {
  constexpr int VN = Vec16<T>::n;
  __shared__ int s_row[kMaxK];
  __shared__ float s_gate[kMaxK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) {
    s_row[threadIdx.x] = rowmap[t * k + threadIdx.x];
    s_gate[threadIdx.x] = gate[t * k + threadIdx.x];
  }
  __syncthreads();
  float zsum = 0.0f;
  for (int j = 0; j < k; ++j)
    if (s_row[j] < 0) zsum += s_gate[j];
  const int npieces = d / VN;
  for (int c = threadIdx.x; c < npieces; c += blockDim.x) {
    float acc[VN], v[VN];
    const uint4 xv = *reinterpret_cast<const uint4 *>(x + t * d + c * VN);
    // The slots' Y pieces are loaded kBatch at a time, all in flight
    // together, then added in ascending slot order.  Each load goes through
    // a buffer descriptor of its Y row; a zero-expert slot (or a slot past
    // k) gets an empty range, so its load returns zeros without touching
    // memory and no load waits behind a branch.  Y rows are read once: the
    // loads are non-temporal (combine -18% at prod).  The x term is formed
    // once the first batch is in flight (k >= 1).
    int j0 = 0;
    do {
      u32x4v yv[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int row = __builtin_amdgcn_readfirstlane(j0 + u < k ? s_row[j0 + u] : -1);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T *>(y) + static_cast<int64_t>(row < 0 ? 0 : row) * d, static_cast<short>(0),
            row < 0 ? 0 : d * static_cast<int>(sizeof(T)), kRsrcFlags);
        yv[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, c * 16, 0, kNonTemporal);
      }
      if (j0 == 0) {
        Vec16<T>::unpack(xv, v);
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] = zsum * v[i];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int row = j0 + u < k ? s_row[j0 + u] : -1;
        if (row < 0) continue;
        const float gj = s_gate[j0 + u];
        Vec16<T>::unpack(make_uint4(yv[u].x, yv[u].y, yv[u].z, yv[u].w), v);
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] += gj * v[i];
      }
      j0 += kBatch;
    } while (j0 < k);
    *reinterpret_cast<uint4 *>(out + t * d + c * VN) = Vec16<T>::pack(acc);
  }
}

template <typename T, int B>
static void launch_combine_t(const Plan &p, hipStream_t s) {
  hipLaunchKernelGGL((combine_kernel<T, B>), dim3(static_cast<unsigned>(p.T)), dim3(256), 0, s,
                     static_cast<const T *>(p.x), static_cast<const T *>(p.y), p.rowmap, p.gate,
                     p.d, p.k, static_cast<T *>(p.out));
}

template <typename T>
static void launch_combine_k(const Plan &p, hipStream_t s) {
  if (p.k <= 4) launch_combine_t<T, 4>(p, s);
  else if (p.k <= 8) launch_combine_t<T, 8>(p, s);
  else if (p.k <= 12) launch_combine_t<T, 12>(p, s);
  else launch_combine_t<T, 16>(p, s);
}

hipError_t launch_combine(const Plan &p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  if (p.dtype == MOE_ZC_BF16) launch_combine_k<bf16_t>(p, s);
  else launch_combine_k<float>(p, s);
  return hipGetLastError();
}

}  // namespace moezc
