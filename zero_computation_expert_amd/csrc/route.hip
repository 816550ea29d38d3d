// route.hip -- steps 1-2 (softmax, selection bias, top-k, gates) and the
// dispatch bookkeeping (selection counts, expert offsets, stable token ->
// expert permutation) of the zero-computation-expert MoE forward.
//
// Method: LongCat-Flash technical-report summary page, section 2
// "architecture", item 1 "zero-computation experts": tokens choose among N
// FFN experts and Z zero experts; an expert-specific bias shifts the routing
// scores to hold the FFN / zero selection ratio; the per-expert selection
// counts are what the bias controller consumes.  Softmax over all experts,
// the bias used for selection only, unbiased gates and the tie-break towards
// the lower expert index are this library's readings of that passage.  The
// gates are scaled by the routed scale (LongCat-Flash-Lite article, part 02:
// the fused router kernel ends with a scaling step; the reading is that every
// selected slot's gate is multiplied by one constant).
#include "moe_zc_internal.h"

namespace moezc {

// Order-preserving map of an fp32 score to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The two largest keys below fl among a lane's slots (0 where there are none).
template <int VPL>
__device__ __forceinline__ void top2_below(const uint64_t (&key)[VPL], uint64_t fl, uint64_t &b1,
                                           uint64_t &b2) {
  b1 = 0ull;
  b2 = 0ull;
#pragma unroll
  for (int s = 0; s < VPL; ++s) {
    const uint64_t x = key[s] < fl ? key[s] : 0ull;
    const bool top = x > b1;
    b2 = top ? b1 : (x > b2 ? x : b2);
    b1 = top ? x : b1;
  }
}

// One wave per token.  Expert e lives in lane e % 64, register slot e / 64.
// Selection key = (ordered score << 32) | (0xffffffff - e): the wave maximum
// is the highest score and, among equal scores, the lowest index.  Key 0
// marks an absent expert (every real key is > 0).
// The block (kTokPerBlk waves) covers kTokPerBlk consecutive tokens and
// writes its per-expert selection histogram to blockhist[blockIdx.x].
// kSplit: the logits arrive as K-slice partials to add.  Without that sum's
// registers, and with at most 768 experts, a block fits twice per CU (the
// second launch bound asks for 8 waves per SIMD; wider keys would spill).
template <int VPL, bool kSplit>
__global__ void __launch_bounds__(kTokPerBlk * kWave, (kSplit || VPL > 12) ? 1 : 8)
    topk_kernel(const float *__restrict__ logits,
                                                   int split, int64_t part_stride,
                                                   const float *__restrict__ bias, int64_t T,
                                                   int E, int k, int32_t *__restrict__ idx_out,
                                                   float *__restrict__ gate_out,
                                                   int32_t *__restrict__ blockhist,
                                                   float routed_scale) {
  __shared__ float s_bias[kMaxE];
  __shared__ int s_hist[kMaxE];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    s_bias[e] = bias[e];
    s_hist[e] = 0;
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokPerBlk;

  const int64_t t = t0 + wave;
  if (t < T) {
    const float *lrow = logits + t * E;
    float l[VPL];
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
      int e = s * kWave + lane;
      l[s] = e < E ? lrow[e] : -INFINITY;
    }
    // A split router GEMM leaves one partial per K slice: add them in slice
    // order, loading U slices at a time so their loads overlap (U = 1 for the
    // widest expert counts, whose registers are already full).
    constexpr int U = VPL <= 16 ? 4 : 1;
    int sl = 1;
    if (!kSplit) sl = split;  // one slice (the launch guarantees split == 1)
    for (; kSplit && sl + U <= split; sl += U) {
      float a[U][VPL];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int s = 0; s < VPL; ++s) {
          int e = s * kWave + lane;
          a[u][s] = e < E ? lrow[(sl + u) * part_stride + e] : 0.0f;
        }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int s = 0; s < VPL; ++s) l[s] += a[u][s];
    }
    for (; kSplit && sl < split; ++sl) {
#pragma unroll
      for (int s = 0; s < VPL; ++s) {
        int e = s * kWave + lane;
        if (e < E) l[s] += lrow[sl * part_stride + e];
      }
    }
    // softmax: exp through the hardware exp2, one reciprocal of the sum
    float m = l[0];
#pragma unroll
    for (int s = 1; s < VPL; ++s) m = fmaxf(m, l[s]);
    m = wave_max_dpp(m);
    float p[VPL];
    float part = 0.0f;
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
      int e = s * kWave + lane;
      p[s] = e < E ? __builtin_amdgcn_exp2f((l[s] - m) * 1.44269504088896341f) : 0.0f;
      part += p[s];
    }
    const float inv = __builtin_amdgcn_rcpf(wave_sum_dpp(part));
    uint64_t key[VPL];
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
      int e = s * kWave + lane;
      p[s] *= inv;
      key[s] = e < E ? (static_cast<uint64_t>(ordered_bits(p[s] + s_bias[e])) << 32) |
                           (0xffffffffu - static_cast<uint32_t>(e))
                     : 0ull;
    }
    // Selection.  A lane's keys are taken in descending order, so the ones
    // it still holds are those below the last one it gave up (fl); it keeps
    // the largest two of them (b1 > b2, 0 = none).  A round takes the wave
    // maximum of b1: a 32-bit maximum of the score words, and only when
    // several lanes hold that score, a second one of their index words (the
    // lowest index wins).  The winning lane moves b2 up; when it has no b2,
    // every lane recomputes its pair (a uniform branch).
    uint64_t fl = ~0ull, b1, b2;
    top2_below<VPL>(key, fl, b1, b2);
    int my_idx = 0;
    float my_gate = 0.0f;
    for (int j = 0; j < k; ++j) {
      const uint32_t hi = static_cast<uint32_t>(b1 >> 32), lo = static_cast<uint32_t>(b1);
      const uint32_t mhi = wave_max_u32(hi);
      uint64_t win = __ballot(hi == mhi);
      if (__popcll(win) > 1) {
        const uint32_t mlo = wave_max_u32(hi == mhi ? lo : 0u);
        win = __ballot(hi == mhi && lo == mlo);
      }
      const int owner = __ffsll(static_cast<unsigned long long>(win)) - 1;
      const int e = static_cast<int>(
          0xffffffffu - static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), owner)));
      const int slot = e / kWave;
      float pe = p[0];
#pragma unroll
      for (int s = 1; s < VPL; ++s) pe = s == slot ? p[s] : pe;
      pe = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pe), owner));
      if (lane == owner) {
        fl = b1;
        b1 = b2;
        b2 = 0ull;
      }
      if (lane == j) {
        my_idx = e;
        my_gate = pe;
      }
      const uint32_t nhi = static_cast<uint32_t>(b1 >> 32), nlo = static_cast<uint32_t>(b1);
      if ((__builtin_amdgcn_readlane(static_cast<int>(nhi), owner) |
           __builtin_amdgcn_readlane(static_cast<int>(nlo), owner)) == 0 && j + 1 < k)
        top2_below<VPL>(key, fl, b1, b2);
    }
    if (lane < k) {
      idx_out[t * k + lane] = my_idx;
      gate_out[t * k + lane] = routed_scale * my_gate;
      atomicAdd(&s_hist[my_idx], 1);
    }
  }
  __syncthreads();
  int32_t *hrow = blockhist + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hrow[e] = s_hist[e];
}

// Column scan of blockhist: per expert, replace each block's count by the
// exclusive prefix over earlier blocks and write the total to counts[e].
// Block = 16 waves over 64 experts; wave w owns a contiguous run of blocks,
// read kScanRun rows at a time with all of a run's loads in flight (one row
// at a time, the two passes took 15 us at prod: 32 dependent round trips).
constexpr int kScanRun = 16;
__global__ void __launch_bounds__(1024) hist_scan_kernel(int32_t *__restrict__ blockhist,
                                                         int nblk, int E,
                                                         int32_t *__restrict__ counts) {
  __shared__ int s_part[16][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int e = blockIdx.x * kWave + lane;
  const int per = (nblk + 15) / 16;
  const int b0 = wave * per;
  const int b1 = min(nblk, b0 + per);
  const bool live = e < E;
  int sum = 0;
  for (int b = b0; b < b1; b += kScanRun) {
    int v[kScanRun];
#pragma unroll
    for (int i = 0; i < kScanRun; ++i)
      v[i] = live && b + i < b1 ? blockhist[static_cast<int64_t>(b + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < kScanRun; ++i) sum += v[i];
  }
  s_part[wave][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int w = 0; w < wave; ++w) run += s_part[w][lane];
  for (int b = b0; b < b1; b += kScanRun) {
    int v[kScanRun];
#pragma unroll
    for (int i = 0; i < kScanRun; ++i)
      v[i] = live && b + i < b1 ? blockhist[static_cast<int64_t>(b + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < kScanRun; ++i) {
      if (live && b + i < b1) blockhist[static_cast<int64_t>(b + i) * E + e] = run;
      run += v[i];
    }
  }
  if (live && wave == 15) counts[e] = run;
}

// Exclusive scan of a per-thread value over a 1024-thread block.
__device__ int block_exclusive_scan(int v, int *s_tmp /* [16] */, int *total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += n;
  }
  if (lane == kWave - 1) s_tmp[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    int x = s_tmp[w];
    if (w < wave) before += x;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Offsets of the FFN experts in permuted row order, and the prefix of GEMM
// chunks (ceil(M_e / chunk_rows) per expert).  Single block.
__global__ void __launch_bounds__(1024) expert_scan_kernel(const int32_t *__restrict__ counts,
                                                           int N, int chunk_rows, int hot_rows,
                                                           int32_t *__restrict__ offs,
                                                           int32_t *__restrict__ chunk_off,
                                                           int32_t *__restrict__ meta) {
  __shared__ int s_tmp[16];
  int base_rows = 0, base_chunks = 0;
  for (int e0 = 0; e0 < N; e0 += 1024) {
    int e = e0 + threadIdx.x;
    int c = e < N ? counts[e] : 0;
    const int rows = hot_rows > 0 && c >= hot_rows ? kHotMT : chunk_rows;
    int ch = (c + rows - 1) / rows;
    int tot_r, tot_c;
    int ex_r = block_exclusive_scan(c, s_tmp, &tot_r);
    int ex_c = block_exclusive_scan(ch, s_tmp, &tot_c);
    if (e < N) {
      offs[e] = base_rows + ex_r;
      chunk_off[e] = base_chunks + ex_c;
    }
    base_rows += tot_r;
    base_chunks += tot_c;
  }
  if (threadIdx.x == 0) {
    offs[N] = base_rows;
    chunk_off[N] = base_chunks;
    meta[0] = base_chunks;
    meta[1] = base_rows;
  }
}

// Stable permutation: FFN slot (t, j) -> row offs[e] + (number of earlier
// tokens routed to e).  One wave per block of kTokPerBlk tokens; tokens are
// walked in order, lanes are slots (the k experts of a token are distinct,
// so the lanes never touch the same counter at once).
// Negative entries (slots the backward's sanitizing dropped) map to no row.
// gate_perm (nullable) receives each permuted row's gate.
__global__ void __launch_bounds__(64) permute_kernel(const int32_t *__restrict__ idx, int64_t T,
                                                     int k, int N, int E,
                                                     const int32_t *__restrict__ offs,
                                                     const int32_t *__restrict__ blockhist,
                                                     int32_t *__restrict__ rowmap,
                                                     int32_t *__restrict__ tok,
                                                     const float *__restrict__ gate,
                                                     float *__restrict__ gate_perm) {
  __shared__ int s_next[kMaxE];
  __shared__ int s_idx[kTokPerBlk * kMaxK];
  const int lane = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokPerBlk;
  const int nt = static_cast<int>(min<int64_t>(kTokPerBlk, T - t0));
  const int32_t *hrow = blockhist + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = lane; e < N; e += kWave) s_next[e] = offs[e] + hrow[e];
  for (int i = lane; i < nt * k; i += kWave) s_idx[i] = idx[t0 * k + i];
  __syncthreads();
  for (int tt = 0; tt < nt; ++tt) {
    if (lane < k) {
      const int e = s_idx[tt * k + lane];
      int r = -1;
      if (e >= 0 && e < N) {
        r = s_next[e];
        s_next[e] = r + 1;
        tok[r] = static_cast<int32_t>(t0 + tt);
        if (gate_perm) gate_perm[r] = gate[(t0 + tt) * k + lane];
      }
      rowmap[(t0 + tt) * k + lane] = r;
    }
    __syncthreads();
  }
}

__global__ void zero_int_kernel(int32_t *p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Sum of a split router GEMM's K-slice partials, added in slice order (the
// order the top-k kernel adds them in, so the logits are bit-identical),
// written over slice 0.  V consecutive logits per thread.
template <int V>
__global__ void __launch_bounds__(256) slice_sum_kernel(float *__restrict__ logits, int split,
                                                        int64_t part_stride, int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * V;
  if (i >= n) return;
  float a[V];
#pragma unroll
  for (int v = 0; v < V; ++v) a[v] = logits[i + v];
  for (int sl = 1; sl < split; ++sl) {
    const float *src = logits + sl * part_stride + i;
    float b[V];
#pragma unroll
    for (int v = 0; v < V; ++v) b[v] = src[v];
#pragma unroll
    for (int v = 0; v < V; ++v) a[v] += b[v];
  }
#pragma unroll
  for (int v = 0; v < V; ++v) logits[i + v] = a[v];
}

// With few tokens the top-k kernel runs on few blocks (one per 16 tokens),
// and each of them would add up all K slices of its tokens: decode's 128
// tokens read 16 slices x 768 logits each on 8 CUs.  Then the slices are
// summed first by a kernel spread over the chip, and top-k reads one slice.
static bool sum_slices_first(const Plan &p) {
  const int64_t bytes = static_cast<int64_t>(p.rs.split) * p.T * p.E * 4;
  return p.rs.split > 1 && p.nblk < 128 && bytes >= (int64_t(1) << 19);
}

template <bool kSplit>
static void launch_topk_v(const Plan &p, int vpl, int split, int64_t n, hipStream_t s) {
  const dim3 grid(p.nblk), block(kTokPerBlk * kWave);
  if (vpl <= 4)
    hipLaunchKernelGGL((topk_kernel<4, kSplit>), grid, block, 0, s, p.logits, split, n, p.bias,
                       p.T, p.E, p.k, p.idx, p.gate, p.blockhist, p.routed_scale);
  else if (vpl <= 12)  // up to 768 experts
    hipLaunchKernelGGL((topk_kernel<12, kSplit>), grid, block, 0, s, p.logits, split, n, p.bias,
                       p.T, p.E, p.k, p.idx, p.gate, p.blockhist, p.routed_scale);
  else if (vpl <= 16)
    hipLaunchKernelGGL((topk_kernel<16, kSplit>), grid, block, 0, s, p.logits, split, n, p.bias,
                       p.T, p.E, p.k, p.idx, p.gate, p.blockhist, p.routed_scale);
  else
    hipLaunchKernelGGL((topk_kernel<32, kSplit>), grid, block, 0, s, p.logits, split, n, p.bias,
                       p.T, p.E, p.k, p.idx, p.gate, p.blockhist, p.routed_scale);
}

hipError_t launch_topk(const Plan &p, hipStream_t s) {
  int split = p.rs.split;
  const int64_t n = p.T * p.E;
  if (sum_slices_first(p)) {
    if (n % 4 == 0)
      hipLaunchKernelGGL(slice_sum_kernel<4>, dim3(static_cast<unsigned>((n / 4 + 255) / 256)),
                         dim3(256), 0, s, p.logits, split, n, n);
    else
      hipLaunchKernelGGL(slice_sum_kernel<1>, dim3(static_cast<unsigned>((n + 255) / 256)),
                         dim3(256), 0, s, p.logits, split, n, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    split = 1;
  }
  const int vpl = (p.E + kWave - 1) / kWave;
  if (split > 1) launch_topk_v<true>(p, vpl, split, n, s);
  else launch_topk_v<false>(p, vpl, split, n, s);
  return hipGetLastError();
}

hipError_t launch_scan(const Plan &p, hipStream_t s) {
  hipLaunchKernelGGL(hist_scan_kernel, dim3((p.E + kWave - 1) / kWave), dim3(1024), 0, s,
                     p.blockhist, p.nblk, p.E, p.counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.N == 0) return err;
  hipLaunchKernelGGL(expert_scan_kernel, dim3(1), dim3(1024), 0, s, p.counts, p.N, p.nbmax * 32,
                     p.hot_rows, p.offs, p.chunk_off, p.meta);
  return hipGetLastError();
}

hipError_t launch_permute(const Plan &p, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3(p.nblk), dim3(64), 0, s, p.idx, p.T, p.k, p.N, p.E,
                     p.offs, p.blockhist, p.rowmap, p.tok, p.gate, p.gate_perm);
  return hipGetLastError();
}

// The dense FFN as one expert that every token uses: identity permutation,
// one segment of T rows, ceil(T / rows) chunks (kHotMT rows from hot_rows
// tokens up, as for a hot expert).
__global__ void dense_route_kernel(int64_t T, int chunk_rows, int hot_rows,
                                   int32_t *__restrict__ tok, int32_t *__restrict__ offs,
                                   int32_t *__restrict__ chunk_off, int32_t *__restrict__ meta) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < T) tok[i] = static_cast<int32_t>(i);
  if (i == 0) {
    const int rows = hot_rows > 0 && T >= hot_rows ? kHotMT : chunk_rows;
    const int nch = static_cast<int>((T + rows - 1) / rows);
    offs[0] = 0;
    offs[1] = static_cast<int32_t>(T);
    chunk_off[0] = 0;
    chunk_off[1] = nch;
    meta[0] = nch;
    meta[1] = static_cast<int32_t>(T);
  }
}

hipError_t launch_dense_route(const Plan &p, hipStream_t s) {
  hipLaunchKernelGGL(dense_route_kernel, dim3(static_cast<unsigned>((p.T + 255) / 256)), dim3(256),
                     0, s, p.T, p.nbmax * 32, p.hot_rows, p.tok, p.offs, p.chunk_off, p.meta);
  return hipGetLastError();
}

hipError_t launch_zero_counts(const Plan &p, hipStream_t s) {
  hipLaunchKernelGGL(zero_int_kernel, dim3((p.E + 255) / 256), dim3(256), 0, s, p.counts, p.E);
  return hipGetLastError();
}

}  // namespace moezc
