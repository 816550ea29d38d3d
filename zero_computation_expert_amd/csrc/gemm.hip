// gemm.hip -- the contractions of the zero-computation-expert MoE forward on
// gfx950 MFMA:
//   ROUTER : logits[t, e] = <x[t], W_router[e]>                       (step 1)
//   GATE_UP: H[row, i]    = silu(<x[tok[row]], W_gate[e,i]>) * <x[tok[row]], W_up[e,i]>
//   DOWN   : Y[row, c]    = <H[row], W_down[e,c]>                     (step 3)
// for every FFN expert e over its permuted rows (LongCat-Flash summary page,
// section 2 "architecture": tokens routed to FFN experts run an expert FFN;
// the SwiGLU form with three matrices is this library's reading of it).
//
// Design (weight-stationary, one pass over every weight byte):
//   * A workgroup (4 waves) owns a block of weight rows of one expert and one
//     chunk of up to 32*NB of that expert's tokens.  Weight rows are the MFMA
//     "A" operand and are streamed from HBM straight into VGPRs, each lane
//     reading 64 contiguous bytes of its row per K-step; every weight byte is
//     used by exactly one wave, so weights never pass through LDS.
//   * Token rows (the MFMA "B" operand, shared by the 4 waves) are gathered
//     (GATE_UP: through the token index of each permuted row) into a
//     double-buffered LDS tile, 128 bytes of K per row per step.
//   * Within each 128-byte K-step the K order is permuted identically for A
//     and B (lane (r, h) supplies k = h*KC/2 + q*PIECE + [0, PIECE) for piece
//     q), which lets a lane load contiguous 64-byte runs.
//   * Weights are prefetched three K-steps ahead and token rows four (register
//     rings), issued in consumption order so that the in-order vector-memory
//     counter never makes a step wait for a later step's data; MFMAs cycle
//     over 2*NB independent accumulators.
//   * Tiles are enumerated expert-major, row-block next, chunk fastest, and
//     block ids are remapped so that consecutive tiles land on the same XCD
//     (workgroups are dealt round-robin over the 8 XCDs): the row blocks of
//     one expert share that expert's token rows in one L2, and the chunks of
//     one row block share its weight rows.
#include <algorithm>
#include <type_traits>

#include "moe_zc_internal.h"

namespace moezc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

enum { MODE_ROUTER = 0, MODE_GATE_UP = 1, MODE_DOWN = 2 };

struct GemmArgs {
  const void *wa;   // ROUTER: W_router; GATE_UP: W_gate; DOWN: W_down
  const void *wb;   // GATE_UP: W_up
  const void *src;  // token rows: x (ROUTER, GATE_UP) or H (DOWN)
  const int32_t *tok;        // GATE_UP: token of each permuted row
  const int32_t *offs;       // [N+1] permuted row offsets (GATE_UP, DOWN)
  const int32_t *chunk_off;  // [N+1] chunk prefix (GATE_UP, DOWN)
  const int32_t *meta;       // meta[0] = total chunks (GATE_UP, DOWN)
  void *out;                 // logits (f32) / H / Y
  int64_t w_expert_stride;   // elements between experts' matrices
  int64_t T;                 // ROUTER: tokens
  int K;                     // reduction length
  int nrows;                 // weight rows per expert (E, I or d)
  int out_ld;                // elements per output row
  int nrb;                   // row blocks per chunk
  int N;                     // FFN experts (GATE_UP, DOWN)
};

template <typename T>
struct MfmaOps;

template <>
struct MfmaOps<bf16_t> {
  // One 16-byte piece = 8 bf16 = one 32x32x16 MFMA.
  static __device__ __forceinline__ void piece(floatx16 &acc, const uint4 &a, const uint4 &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};

template <>
struct MfmaOps<float> {
  // One 16-byte piece = 4 fp32 = four 32x32x2 MFMAs (one k per half-wave each).
  static __device__ __forceinline__ void piece(floatx16 &acc, const uint4 &a, const uint4 &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc,
                                               0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc,
                                               0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc,
                                               0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc,
                                               0, 0, 0);
  }
};

template <typename T>
__device__ __forceinline__ void store4(T *dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float *dst, float a, float b, float c, float d) {
  *reinterpret_cast<float4 *>(dst) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t *dst, float a, float b, float c, float d) {
  uint2 v;
  v.x = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
  v.y = static_cast<uint32_t>(f32_to_bf16(c)) | (static_cast<uint32_t>(f32_to_bf16(d)) << 16);
  *reinterpret_cast<uint2 *>(dst) = v;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

constexpr int kPitch = 144;  // LDS bytes per token row: 128 data + 16 pad (conflict-free b128)
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past every range: the load reads zeros

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(off), 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Per-thread state of one tile.
template <int NB>
struct TileState {
  __amdgpu_buffer_rsrc_t ra[2];  // weight matrices (A operand)
  __amdgpu_buffer_rsrc_t rb;     // token rows (B operand)
  uint32_t voa[2];               // byte offset of this lane's weight row half-step
  uint32_t vob[NB];              // byte offset of this thread's token row piece (or kOOB)
  int kpos_a;                    // K element of this lane's first A piece within a step
  int kpos_b;                    // K element of this thread's B piece within a step
  int K;
};

// Weights of K-step ks: 4 pieces of 16 bytes per row block, straight to VGPRs.
// Pieces past K read zeros (out-of-range buffer offset).
template <typename T, int NB>
__device__ __forceinline__ void load_a(uint4 (&buf)[2][4], const TileState<NB> &st, int ks) {
  constexpr int KC = 128 / sizeof(T);
  constexpr int PIECE = 16 / sizeof(T);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool ok = ks * KC + st.kpos_a + q * PIECE < st.K;
#pragma unroll
    for (int a = 0; a < 2; ++a)
      buf[a][q] = bload(st.ra[a], ok ? st.voa[a] + ks * 128 + q * 16 : kOOB);
  }
}

// Token rows of K-step ks into registers (one 16-byte piece per 32 rows);
// rows past the chunk read zeros.
template <typename T, int NB>
__device__ __forceinline__ void load_b(uint4 (&xr)[NB], const TileState<NB> &st, int ks) {
  constexpr int KC = 128 / sizeof(T);
  const bool ok = ks * KC + st.kpos_b < st.K;
#pragma unroll
  for (int i = 0; i < NB; ++i)
    xr[i] = bload(st.rb, (ok && st.vob[i] != kOOB) ? st.vob[i] + ks * 128 : kOOB);
}

template <int NB>
__device__ __forceinline__ void store_b(char *tile, const uint4 (&xr)[NB], int brow, int bp) {
#pragma unroll
  for (int i = 0; i < NB; ++i)
    *reinterpret_cast<uint4 *>(tile + (brow + 32 * i) * kPitch + bp * 16) = xr[i];
}

// For each 16-byte piece: the NB token fragments from LDS, then 2 x NB
// independent MFMAs (consecutive MFMAs never share an accumulator).
template <typename T, int NB>
__device__ __forceinline__ void compute(floatx16 (&acc)[2][NB], const char *tile,
                                        const uint4 (&A)[2][4], int nb_rt, int r, int h) {
  const char *bp_lds = tile + r * kPitch + h * 64;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint4 B[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      if (nb < nb_rt) B[nb] = *reinterpret_cast<const uint4 *>(bp_lds + nb * 32 * kPitch + q * 16);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      if (nb < nb_rt)
#pragma unroll
        for (int a = 0; a < 2; ++a) MfmaOps<T>::piece(acc[a][nb], A[a][q], B[nb]);
  }
}

// One K-step with a ring of NST weight buffers and two token-row buffers.
// Issue order per step: token rows of step ks + 2, weights of step
// ks + NST - 1; then the MFMAs of step ks (weights in ring slot S, tokens in
// LDS tile ks & 1); then the token rows of step ks + 1 go to the other LDS
// tile.  Token rows are issued a step before the weights that follow them,
// so the in-order vector-memory counter lets each wait cover only data this
// step consumes, and NST - 1 steps of weights stay in flight.
template <typename T, int NB, int NST, int S>
__device__ __forceinline__ void kstep(int ks, int nks, floatx16 (&acc)[2][NB],
                                      uint4 (&abuf)[NST][2][4], uint4 (&xr)[2][NB],
                                      const TileState<NB> &st, char (*tile)[NB * 32 * kPitch],
                                      int nb_rt, int r, int h, int brow, int bp) {
  // Loads are unconditional: past the end of K they read zeros (their
  // buffer offsets are out of range), and a load on every path keeps the
  // compiler's in-order wait counts exact.
  load_b<T, NB>(xr[S & 1], st, ks + 2);
  load_a<T, NB>(abuf[(S + NST - 1) % NST], st, ks + NST - 1);
  compute<T, NB>(acc, tile[ks & 1], abuf[S], nb_rt, r, h);
  store_b<NB>(tile[(ks + 1) & 1], xr[(S + 1) & 1], brow, bp);
  __syncthreads();
}

template <typename T, int MODE, int NB, int NST>
__global__ void __launch_bounds__(256) gemm_kernel(GemmArgs g) {
  constexpr int KC = 128 / sizeof(T);     // K elements per step (128 bytes per row)
  constexpr int MT = NB * 32;             // tokens per chunk
  constexpr uint32_t ES = sizeof(T);
  __shared__ __attribute__((aligned(16))) char s_tile[2][MT * kPitch];
  __shared__ int s_co[kMaxE + 1];

  // ---- which tile -------------------------------------------------------
  int ntiles;
  if (MODE == MODE_ROUTER) {
    ntiles = static_cast<int>((g.T + MT - 1) / MT) * g.nrb;
  } else {
    ntiles = g.meta[0] * g.nrb;
  }
  const int quota = (ntiles + 7) / 8;
  const int loc = blockIdx.x / 8;
  if (loc >= quota) return;
  const int v = (blockIdx.x % 8) * quota + loc;
  if (v >= ntiles) return;

  int e = 0, rb, m0, mcount;
  if (MODE == MODE_ROUTER) {
    const int nch = static_cast<int>((g.T + MT - 1) / MT);
    rb = v / nch;
    const int ch = v % nch;
    m0 = ch * MT;
    mcount = static_cast<int>(min<int64_t>(MT, g.T - m0));
  } else {
    for (int i = threadIdx.x; i <= g.N; i += blockDim.x) s_co[i] = g.chunk_off[i];
    __syncthreads();
    const int c = v / g.nrb;
    int lo = 0, hi = g.N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_co[mid] <= c) lo = mid;
      else hi = mid - 1;
    }
    e = lo;
    const int local = v - g.nrb * s_co[e];
    const int nch = s_co[e + 1] - s_co[e];
    rb = local / nch;
    const int ch = local - rb * nch;
    m0 = g.offs[e] + ch * MT;
    mcount = min(MT, g.offs[e + 1] - m0);
  }
  const int nb_rt = (mcount + 31) / 32;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 31;
  const int h = lane >> 5;
  const int K = g.K;

  TileState<NB> st;
  st.K = K;
  st.kpos_a = h * (KC / 2);
  // ---- weight rows of this lane (MFMA A operand) -------------------------
  const uint32_t wbytes = static_cast<uint32_t>(g.nrows) * static_cast<uint32_t>(K) * ES;
  const char *w0 = static_cast<const char *>(g.wa) + e * g.w_expert_stride * ES;
  int rowbase;  // first weight row of this wave
  if (MODE == MODE_GATE_UP) {
    rowbase = rb * 128 + wave * 32;
    const int row = min(rowbase + r, g.nrows - 1);
    st.ra[0] = make_rsrc(w0, wbytes);
    st.ra[1] = make_rsrc(static_cast<const char *>(g.wb) + e * g.w_expert_stride * ES, wbytes);
    st.voa[0] = st.voa[1] = static_cast<uint32_t>(row) * K * ES + h * 64;
  } else {
    rowbase = rb * 256 + wave * 64;
    st.ra[0] = st.ra[1] = make_rsrc(w0, wbytes);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int row = min(rowbase + a * 32 + r, g.nrows - 1);
      st.voa[a] = static_cast<uint32_t>(row) * K * ES + h * 64;
    }
  }

  // ---- token rows this thread stages into LDS (B operand) ----------------
  const int bp = threadIdx.x & 7;     // 16-byte piece within the 128-byte step
  const int brow = threadIdx.x >> 3;  // 0..31
  st.kpos_b = bp * (16 / static_cast<int>(ES));
  if (MODE == MODE_GATE_UP) {
    st.rb = make_rsrc(g.src, static_cast<uint32_t>(g.T) * K * ES);  // all of x (gathered)
  } else {
    st.rb = make_rsrc(static_cast<const char *>(g.src) + static_cast<int64_t>(m0) * K * ES,
                      static_cast<uint32_t>(mcount) * K * ES);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int tr = brow + 32 * i;
    uint32_t row = 0;
    if (tr < mcount) row = MODE == MODE_GATE_UP ? static_cast<uint32_t>(g.tok[m0 + tr]) : tr;
    st.vob[i] = tr < mcount ? row * K * ES + bp * 16 : kOOB;
  }

  const int nks = (K + KC - 1) / KC;

  static_assert(NST % 2 == 0, "the token buffers alternate with the step parity");
  uint4 abuf[NST][2][4];
  uint4 xr[2][NB];
  floatx16 acc[2][NB];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][nb][i] = 0.0f;

  // ---- prologue: token tile 0 in LDS; then, in consumption order, token
  // rows of step 1 and weights of steps 0 .. NST-2 ------------------------
  load_b<T, NB>(xr[0], st, 0);
  store_b<NB>(s_tile[0], xr[0], brow, bp);
  load_b<T, NB>(xr[1], st, 1);
#pragma unroll
  for (int j = 0; j < NST - 1; ++j) load_a<T, NB>(abuf[j], st, j);
  __syncthreads();

  // ---- main loop, unrolled by the weight ring ----------------------------
  int ks = 0;
  for (; ks + NST <= nks; ks += NST) {
    kstep<T, NB, NST, 0>(ks, nks, acc, abuf, xr, st, s_tile, nb_rt, r, h, brow, bp);
    kstep<T, NB, NST, 1>(ks + 1, nks, acc, abuf, xr, st, s_tile, nb_rt, r, h, brow, bp);
    if constexpr (NST > 2) {
      kstep<T, NB, NST, 2>(ks + 2, nks, acc, abuf, xr, st, s_tile, nb_rt, r, h, brow, bp);
      kstep<T, NB, NST, 3>(ks + 3, nks, acc, abuf, xr, st, s_tile, nb_rt, r, h, brow, bp);
    }
  }
  if (ks < nks) kstep<T, NB, NST, 0>(ks, nks, acc, abuf, xr, st, s_tile, nb_rt, r, h, brow, bp);
  if constexpr (NST > 2) {
    if (ks + 1 < nks) kstep<T, NB, NST, 1>(ks + 1, nks, acc, abuf, xr, st, s_tile, nb_rt, r, h, brow, bp);
    if (ks + 2 < nks) kstep<T, NB, NST, 2>(ks + 2, nks, acc, abuf, xr, st, s_tile, nb_rt, r, h, brow, bp);
  }

  // ---- epilogue ----------------------------------------------------------
  // Lane (r, h) holds, for column r of each 32x32 tile, rows
  // gi*8 + h*4 + [0, 4) in acc elements gi*4 .. gi*4+3.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = nb * 32 + r;
    if (nb >= nb_rt || col >= mcount) continue;
    if (MODE == MODE_ROUTER) {
      float *orow = static_cast<float *>(g.out) + (static_cast<int64_t>(m0) + col) * g.out_ld;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = rowbase + a * 32 + gi * 8 + h * 4 + j;
            if (row < g.nrows) orow[row] = acc[a][nb][gi * 4 + j];
          }
    } else if (MODE == MODE_GATE_UP) {
      T *orow = static_cast<T *>(g.out) + (static_cast<int64_t>(m0) + col) * g.out_ld;
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int row = rowbase + gi * 8 + h * 4;
        if (row < g.nrows) {
          const floatx16 &ga = acc[0][nb];
          const floatx16 &ua = acc[1][nb];
          store4<T>(orow + row, silu_mul(ga[gi * 4 + 0], ua[gi * 4 + 0]),
                    silu_mul(ga[gi * 4 + 1], ua[gi * 4 + 1]),
                    silu_mul(ga[gi * 4 + 2], ua[gi * 4 + 2]),
                    silu_mul(ga[gi * 4 + 3], ua[gi * 4 + 3]));
        }
      }
    } else {
      T *orow = static_cast<T *>(g.out) + (static_cast<int64_t>(m0) + col) * g.out_ld;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const int row = rowbase + a * 32 + gi * 8 + h * 4;
          if (row < g.nrows)
            store4<T>(orow + row, acc[a][nb][gi * 4 + 0], acc[a][nb][gi * 4 + 1],
                      acc[a][nb][gi * 4 + 2], acc[a][nb][gi * 4 + 3]);
        }
    }
  }
}

#ifndef MOEZC_NST_BIG
#define MOEZC_NST_BIG 4
#endif
#ifndef MOEZC_NST_SMALL
#define MOEZC_NST_SMALL 4
#endif

template <typename T, int MODE>
static hipError_t launch_gemm_t(const GemmArgs &g, int nb, int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const int64_t grid = ((max_tiles + 7) / 8) * 8;
  const dim3 gd(static_cast<unsigned>(grid)), bd(256);
  switch (nb) {
    case 4: hipLaunchKernelGGL((gemm_kernel<T, MODE, 4, MOEZC_NST_BIG>), gd, bd, 0, s, g); break;
    case 2: hipLaunchKernelGGL((gemm_kernel<T, MODE, 2, MOEZC_NST_BIG>), gd, bd, 0, s, g); break;
    default: hipLaunchKernelGGL((gemm_kernel<T, MODE, 1, MOEZC_NST_SMALL>), gd, bd, 0, s, g); break;
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_gemm(const Plan &p, const GemmArgs &g, int nb, int64_t max_tiles,
                              hipStream_t s) {
  if (p.dtype == MOE_ZC_BF16) return launch_gemm_t<bf16_t, MODE>(g, nb, max_tiles, s);
  return launch_gemm_t<float, MODE>(g, nb, max_tiles, s);
}

// Upper bound of the GEMM chunks: sum_e ceil(M_e / MT) <= P / MT + min(N, P).
static int64_t max_chunks(const Plan &p) {
  const int64_t mt = 32 * p.nbmax;
  return p.pmax / mt + std::min<int64_t>(p.N, p.pmax) + 1;
}

hipError_t launch_router_gemm(const Plan &p, hipStream_t s) {
  GemmArgs g = {};
  g.wa = p.w_router;
  g.src = p.x;
  g.out = p.logits;
  g.T = p.T;
  g.K = p.d;
  g.nrows = p.E;
  g.out_ld = p.E;
  g.nrb = (p.E + 255) / 256;
  const int nb = 4;
  const int64_t tiles = ((p.T + 32 * nb - 1) / (32 * nb)) * g.nrb;
  return launch_gemm<MODE_ROUTER>(p, g, nb, tiles, s);
}

hipError_t launch_gate_up(const Plan &p, hipStream_t s) {
  GemmArgs g = {};
  g.wa = p.w_gate;
  g.wb = p.w_up;
  g.src = p.x;
  g.tok = p.tok;
  g.offs = p.offs;
  g.chunk_off = p.chunk_off;
  g.meta = p.meta;
  g.out = p.h;
  g.w_expert_stride = static_cast<int64_t>(p.I) * p.d;
  g.T = p.T;  // x rows are gathered from the whole of x
  g.K = p.d;
  g.nrows = p.I;
  g.out_ld = p.I;
  g.nrb = (p.I + 127) / 128;
  g.N = p.N;
  return launch_gemm<MODE_GATE_UP>(p, g, p.nbmax, max_chunks(p) * g.nrb, s);
}

hipError_t launch_down(const Plan &p, hipStream_t s) {
  GemmArgs g = {};
  g.wa = p.w_down;
  g.src = p.h;
  g.offs = p.offs;
  g.chunk_off = p.chunk_off;
  g.meta = p.meta;
  g.out = p.y;
  g.w_expert_stride = static_cast<int64_t>(p.I) * p.d;
  g.K = p.I;
  g.nrows = p.d;
  g.out_ld = p.d;
  g.nrb = (p.d + 255) / 256;
  g.N = p.N;
  return launch_gemm<MODE_DOWN>(p, g, p.nbmax, max_chunks(p) * g.nrb, s);
}

}  // namespace moezc
