// pad.hip -- zero-padded copies for forward widths that are not multiples of
// 8 elements.  The expert and router GEMMs move 16-byte row pieces, so they
// need d and I in whole pieces.  For other widths the forward copies x, the
// router weights and the expert matrices into workspace with rows padded by
// zeros (and W_gate / W_up / W_down with zero rows up to the padded width),
// runs on those, and copies the output's first d columns back.  The padded
// problem has the same result: every extra term of every dot product is a
// product with an exact zero, and the extra SwiGLU features are
// silu(0) * 0 = 0, which meet zero columns of W_down.
#include "moe_zc_internal.h"

namespace moezc {

// dst [nmat, rows_p, cols_p] <- src [nmat, rows, cols], zeros past rows and
// cols; one block per destination row (grid-stride).  T: the element's bits.
template <typename T>
__global__ void __launch_bounds__(256) pad_kernel(const T *__restrict__ src, int rows, int cols,
                                                  T *__restrict__ dst, int rows_p, int cols_p,
                                                  int64_t nrows_p) {
  for (int64_t row = blockIdx.x; row < nrows_p; row += gridDim.x) {
    const int64_t m = row / rows_p;
    const int r = static_cast<int>(row - m * rows_p);
    T *d = dst + row * cols_p;
    if (r < rows) {
      const T *s = src + (m * rows + r) * cols;
      for (int c = threadIdx.x; c < cols_p; c += 256) d[c] = c < cols ? s[c] : T(0);
    } else {
      for (int c = threadIdx.x; c < cols_p; c += 256) d[c] = T(0);
    }
  }
}

// dst [rows, cols] <- the first cols columns of src [rows, cols_p].
template <typename T>
__global__ void __launch_bounds__(256) unpad_kernel(const T *__restrict__ src, int cols_p,
                                                    T *__restrict__ dst, int cols, int64_t rows) {
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const T *s = src + row * cols_p;
    T *d = dst + row * cols;
    for (int c = threadIdx.x; c < cols; c += 256) d[c] = s[c];
  }
}

static unsigned grid_for(int64_t rows) {
  return static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(rows, 16384)));
}

hipError_t launch_pad(const void *src, int64_t nmat, int rows, int cols, void *dst, int rows_p,
                      int cols_p, int es, hipStream_t s) {
  const int64_t n = nmat * rows_p;
  if (n <= 0) return hipSuccess;
  if (es == 2)
    hipLaunchKernelGGL(pad_kernel<uint16_t>, dim3(grid_for(n)), dim3(256), 0, s,
                       static_cast<const uint16_t *>(src), rows, cols,
                       static_cast<uint16_t *>(dst), rows_p, cols_p, n);
  else
    hipLaunchKernelGGL(pad_kernel<uint32_t>, dim3(grid_for(n)), dim3(256), 0, s,
                       static_cast<const uint32_t *>(src), rows, cols,
                       static_cast<uint32_t *>(dst), rows_p, cols_p, n);
  return hipGetLastError();
}

hipError_t launch_unpad(const void *src, int64_t rows, int cols_p, void *dst, int cols, int es,
                        hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (es == 2)
    hipLaunchKernelGGL(unpad_kernel<uint16_t>, dim3(grid_for(rows)), dim3(256), 0, s,
                       static_cast<const uint16_t *>(src), cols_p, static_cast<uint16_t *>(dst),
                       cols, rows);
  else
    hipLaunchKernelGGL(unpad_kernel<uint32_t>, dim3(grid_for(rows)), dim3(256), 0, s,
                       static_cast<const uint32_t *>(src), cols_p, static_cast<uint32_t *>(dst),
                       cols, rows);
  return hipGetLastError();
}

}  // namespace moezc
