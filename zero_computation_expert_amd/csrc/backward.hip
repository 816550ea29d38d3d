// backward.hip -- the non-GEMM kernels of the block's backward: routing
// bookkeeping from the forward's top-k, the permuted operand rows, the
// router (softmax) backward and the deterministic gather of dx.
//
// LongCat-Flash summary page, section 5 "training infrastructure": the
// pages aggregate gradients with a deterministic scatter-add.  Here the
// aggregation is a gather instead: every token adds the rows of its own
// slots in slot order, so no two threads ever add into one element and the
// result does not depend on timing.
#include "moe_zc_internal.h"

namespace moezc {

// Per block of kTokPerBlk tokens (one wave, lanes = slots): validate the
// caller's routing -- an entry outside [0, E) or repeating an earlier slot
// of its token becomes -1 and is ignored by every later stage -- and count
// each expert's selections in this block.
__global__ void __launch_bounds__(kWave) bwd_hist_kernel(const int32_t *__restrict__ idx_in,
                                                         int64_t T, int k, int E,
                                                         int32_t *__restrict__ idx_s,
                                                         int32_t *__restrict__ blockhist) {
  __shared__ int s_hist[kMaxE];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += kWave) s_hist[e] = 0;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokPerBlk;
  const int nt = static_cast<int>(min<int64_t>(kTokPerBlk, T - t0));
  for (int tt = 0; tt < nt; ++tt) {
    const int64_t o = (t0 + tt) * k;
    const int e = lane < k ? idx_in[o + lane] : -1;
    bool ok = lane < k && e >= 0 && e < E;
    for (int j = 0; j < k; ++j) {
      const int ej = __shfl(e, j, kWave);
      if (j < lane && ej == e) ok = false;
    }
    if (lane < k) {
      idx_s[o + lane] = ok ? e : -1;
      if (ok) atomicAdd(&s_hist[e], 1);
    }
  }
  __syncthreads();
  int32_t *hrow = blockhist + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = lane; e < E; e += kWave) hrow[e] = s_hist[e];
}

// Rows of the wgrad operands in permuted order: xp[r] = x[tok[r]] and
// dyp[r] = gate_perm[r] * dout[tok[r]] (bf16), 8 elements per thread.
__global__ void __launch_bounds__(256) bwd_gather_kernel(const bf16_t *__restrict__ x,
                                                         const bf16_t *__restrict__ dout,
                                                         const int32_t *__restrict__ tok,
                                                         const float *__restrict__ gate_perm,
                                                         const int32_t *__restrict__ meta, int d,
                                                         bf16_t *__restrict__ xp,
                                                         bf16_t *__restrict__ dyp) {
  const int64_t r = blockIdx.x;
  if (r >= meta[1]) return;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= d) return;
  const int64_t src = static_cast<int64_t>(tok[r]) * d + c, dst = r * d + c;
  *reinterpret_cast<uint4 *>(xp + dst) = *reinterpret_cast<const uint4 *>(x + src);
  const uint4 g = *reinterpret_cast<const uint4 *>(dout + src);
  const float gt = gate_perm[r];
  const uint32_t w[4] = {g.x, g.y, g.z, g.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = gt * __uint_as_float(w[i] << 16);
    const float hi = gt * __uint_as_float(w[i] & 0xFFFF0000u);
    o[i] = pack_bf16x2(lo, hi);
  }
  *reinterpret_cast<uint4 *>(dyp + dst) = make_uint4(o[0], o[1], o[2], o[3]);
}

// Router backward, one wave per token (lane holds experts s*64 + lane):
// p = softmax(logits) (the K slices of a split router GEMM summed in slice
// order); the gate gradient of each slot -- FFN slot: the sum of the dgrad
// kernel's per-row-block partials, zero slot: <dout, x>; dl = p * (dp -
// <p, dp>) with dp the slots' gate gradients at their experts, written as
// bf16 with zeros in the row padding up to ldl.
template <int VPL>
__global__ void __launch_bounds__(kTokPerBlk * kWave) router_bwd_kernel(
    const float *__restrict__ logits, int split, int64_t part_stride, int64_t T, int E, int N,
    int k, const int32_t *__restrict__ idx_s, const int32_t *__restrict__ rowmap,
    const float *__restrict__ dpart, int nrbi, int64_t dpart_stride,
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ dout, int d, bf16_t *__restrict__ dl,
    int ldl, float routed_scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlk + threadIdx.x / kWave;
  if (t >= T) return;
  const float *lrow = logits + t * E;
  float p[VPL];
#pragma unroll
  for (int s = 0; s < VPL; ++s) {
    const int e = s * kWave + lane;
    p[s] = e < E ? lrow[e] : -INFINITY;
  }
  for (int sl = 1; sl < split; ++sl) {
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
      const int e = s * kWave + lane;
      if (e < E) p[s] += lrow[sl * part_stride + e];
    }
  }
  float m = p[0];
#pragma unroll
  for (int s = 1; s < VPL; ++s) m = fmaxf(m, p[s]);
  m = wave_max(m);
  float part = 0.0f;
#pragma unroll
  for (int s = 0; s < VPL; ++s) {
    const int e = s * kWave + lane;
    p[s] = e < E ? expf(p[s] - m) : 0.0f;
    part += p[s];
  }
  const float sum = wave_sum(part);
#pragma unroll
  for (int s = 0; s < VPL; ++s) p[s] = p[s] / sum;

  // <dout, x> for the zero-expert slots
  float xd = 0.0f;
  for (int c = lane * 8; c < d; c += kWave * 8) {
    const uint4 a = *reinterpret_cast<const uint4 *>(x + t * d + c);
    const uint4 b = *reinterpret_cast<const uint4 *>(dout + t * d + c);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xd += __uint_as_float(aw[i] << 16) * __uint_as_float(bw[i] << 16);
      xd += __uint_as_float(aw[i] & 0xFFFF0000u) * __uint_as_float(bw[i] & 0xFFFF0000u);
    }
  }
  xd = wave_sum(xd);

  // the slots' gate gradients (lane j < k holds slot j's)
  int e = -1;
  float dg = 0.0f;
  if (lane < k) {
    e = idx_s[t * k + lane];
    if (e >= N) {
      dg = xd;
    } else if (e >= 0) {
      const int64_t row = rowmap[t * k + lane];
      for (int b = 0; b < nrbi; ++b) dg += dpart[b * dpart_stride + row];
    }
  }
  float dp[VPL];
#pragma unroll
  for (int s = 0; s < VPL; ++s) dp[s] = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int ej = __shfl(e, j, kWave);
    const float gj = __shfl(dg, j, kWave);
    if (ej >= 0 && (ej & (kWave - 1)) == lane) {
#pragma unroll
      for (int s = 0; s < VPL; ++s)
        if (s == ej / kWave) dp[s] = routed_scale * gj;  // gate = routed_scale * p
    }
  }
  float pd = 0.0f;
#pragma unroll
  for (int s = 0; s < VPL; ++s) pd += p[s] * dp[s];
  pd = wave_sum(pd);
  bf16_t *drow = dl + t * ldl;
#pragma unroll
  for (int s = 0; s < VPL; ++s) {
    const int ee = s * kWave + lane;
    if (ee < ldl) drow[ee] = ee < E ? f32_to_bf16(p[s] * (dp[s] - pd)) : static_cast<bf16_t>(0);
  }
}

// dx[t] = zsum_t * dout[t] + sum_j (FFN slots, ascending j) dxp[row(t, j)]
// + dxr[t], summed in fp32 and rounded once; 8 elements per thread.
__global__ void __launch_bounds__(256) dx_gather_kernel(
    const bf16_t *__restrict__ dout, const int32_t *__restrict__ idx_s,
    const float *__restrict__ gate, const int32_t *__restrict__ rowmap,
    const bf16_t *__restrict__ dxp, const float *__restrict__ dxr, int k, int N, int E, int d,
    bf16_t *__restrict__ dx) {
  const int64_t t = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= d) return;
  float zs = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int e = idx_s[t * k + j];
    if (e >= N && e < E) zs += gate[t * k + j];
  }
  float acc[8];
  {
    const uint4 g = *reinterpret_cast<const uint4 *>(dout + t * d + c);
    const uint32_t w[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = zs * __uint_as_float(w[i] << 16);
      acc[2 * i + 1] = zs * __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  for (int j = 0; j < k; ++j) {
    const int row = rowmap[t * k + j];
    if (row < 0) continue;
    const uint4 g = *reinterpret_cast<const uint4 *>(dxp + static_cast<int64_t>(row) * d + c);
    const uint32_t w[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(w[i] << 16);
      acc[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  const float4 r0 = *reinterpret_cast<const float4 *>(dxr + t * d + c);
  const float4 r1 = *reinterpret_cast<const float4 *>(dxr + t * d + c + 4);
  const float rr[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack_bf16x2(acc[2 * i] + rr[2 * i], acc[2 * i + 1] + rr[2 * i + 1]);
  *reinterpret_cast<uint4 *>(dx + t * d + c) = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_bwd_route(const Plan &p, hipStream_t s) {
  hipLaunchKernelGGL(bwd_hist_kernel, dim3(p.nblk), dim3(kWave), 0, s, p.idx_in, p.T, p.k, p.E,
                     p.idx, p.blockhist);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = launch_scan(p, s);
  if (e == hipSuccess) e = launch_permute(p, s);
  return e;
}

hipError_t launch_bwd_gather(const Plan &p, hipStream_t s) {
  if (p.pmax == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.pmax), static_cast<unsigned>((p.d + 2047) / 2048));
  hipLaunchKernelGGL(bwd_gather_kernel, grid, dim3(256), 0, s,
                     static_cast<const bf16_t *>(p.x), static_cast<const bf16_t *>(p.dout), p.tok,
                     p.gate_perm, p.meta, p.d, static_cast<bf16_t *>(p.xp),
                     static_cast<bf16_t *>(p.dyp));
  return hipGetLastError();
}

hipError_t launch_router_bwd(const Plan &p, hipStream_t s) {
  const int vpl = (p.E + kWave - 1) / kWave;
  const int nrbi = p.N > 0 ? (p.I + 255) / 256 : 0;
#define MOEZC_RB_ARGS                                                                    \
  p.logits, p.rs.split, p.T * p.E, p.T, p.E, p.N, p.k, p.idx, p.rowmap, p.dpart, nrbi, \
      p.pmax, static_cast<const bf16_t *>(p.x), static_cast<const bf16_t *>(p.dout), p.d, \
      static_cast<bf16_t *>(p.dl), p.ldl, p.routed_scale
  const dim3 grid(p.nblk), block(kTokPerBlk * kWave);
  if (vpl <= 4)
    hipLaunchKernelGGL(router_bwd_kernel<4>, grid, block, 0, s, MOEZC_RB_ARGS);
  else if (vpl <= 16)
    hipLaunchKernelGGL(router_bwd_kernel<16>, grid, block, 0, s, MOEZC_RB_ARGS);
  else
    hipLaunchKernelGGL(router_bwd_kernel<32>, grid, block, 0, s, MOEZC_RB_ARGS);
#undef MOEZC_RB_ARGS
  return hipGetLastError();
}

hipError_t launch_dx_gather(const Plan &p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.T), static_cast<unsigned>((p.d + 2047) / 2048));
  hipLaunchKernelGGL(dx_gather_kernel, grid, dim3(256), 0, s,
                     static_cast<const bf16_t *>(p.dout), p.idx, p.gate, p.rowmap,
                     static_cast<const bf16_t *>(p.dxp), p.dxr, p.k, p.N, p.E, p.d,
                     static_cast<bf16_t *>(p.dx));
  return hipGetLastError();
}

}  // namespace moezc
