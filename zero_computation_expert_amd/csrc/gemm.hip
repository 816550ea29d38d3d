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
//   * A workgroup of 4 waves owns 256 weight rows of one expert (GATE_UP: 128
//     rows of W_gate and the same 128 rows of W_up) and one chunk of up to
//     32*NB of that expert's tokens (NB = 5: 160 tokens).  Each wave owns two
//     32-row blocks (the MFMA "A" operand; in GATE_UP a gate block and the up
//     block of the same rows, so silu(g) * u is formed in registers) against
//     all the chunk's token blocks.
//   * Weights stream from HBM straight into LDS with direct-to-LDS buffer
//     loads: every instruction moves 8 whole rows x 128 bytes, fully
//     coalesced, into a three-slot ring private to the wave (two K-steps in
//     flight without holding registers).  An XOR swizzle of the 16-byte
//     chunks, applied on the global side, makes the MFMA-layout LDS reads
//     bank-conflict free.
//   * Token rows (the MFMA "B" operand, shared by the 4 waves) are gathered
//     the same way (GATE_UP: through the token index of each permuted row),
//     8 rows x 128 bytes per instruction, into a three-tile ring with the
//     same swizzle; no token byte passes through registers.  Three weight
//     slots and three 160-row tiles take 156 KB of the 160 KB of LDS.
//     Each K-step ends with one wait for the previous step's loads and one
//     workgroup barrier.
//   * Within each 128-byte K-step the K order is permuted identically for A
//     and B (lane (r, h) supplies k = h*KC/2 + q*PIECE + [0, PIECE) for piece
//     q), so both operands are read as contiguous 16-byte pieces.
//   * Loads are issued unconditionally (out-of-range buffer offsets read
//     zeros) and in consumption order, so the in-order vector-memory counter
//     never makes a step wait for data of a later step.
//   * Tiles are enumerated expert-major, row-block next, chunk fastest, and
//     block ids are remapped so that groups of consecutive tiles land on the
//     same XCD (xcd_tile_grouped; workgroups are dealt round-robin over the
//     8 XCDs): the row blocks of one expert share that expert's token rows
//     in one L2, and the chunks of one row block share its weight rows; the
//     groups are dealt over the XCDs so that their loads stay even.
//   * Expert weights and the outputs are touched once per launch and carry
//     the non-temporal cache hint, so they do not evict those token rows;
//     the router's weights, read by every token tile, do not.
//   * bf16 outputs leave through the idle ring: each wave stages its output
//     features of every token row in LDS and stores whole row segments
//     (stage_epilogue), instead of 16-byte pieces scattered over 32 rows.
//   * For 160-token chunks (bf16) the workgroup has 8 waves, two per SIMD
//     (gemm8w_kernel), and experts of more than 160 rows run 256 x 256
//     hot-expert tiles (gemm_hot_tile), which do more MFMA work per loaded
//     and per LDS-read byte (a last chunk of at most 128 rows as a narrow
//     tile: the waves split weight rows four ways and tokens two ways).
#include "gemm_common.h"

namespace moezc {

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

// Fragments of 16-byte piece q: the wave's two weight fragments (swizzled
// slot) and the NBR token fragments (swizzled tile); both operands hold
// logical chunk h*4 + q of a row whose bits 0-4 are r's (lds_swz reads bits
// 1-3 only).
template <int NBR>
__device__ __forceinline__ void load_frags(uint4 (&A)[2], uint4 (&B)[NBR], const char *slot_wave,
                                           const char *tb, int r, int h, int q) {
  const int chunk = ((h * 4 + q) ^ lds_swz(r)) * 16;
#pragma unroll
  for (int a = 0; a < 2; ++a)
    A[a] = *reinterpret_cast<const uint4 *>(slot_wave + (a * 32 + r) * 128 + chunk);
#pragma unroll
  for (int nb = 0; nb < NBR; ++nb)
    B[nb] = *reinterpret_cast<const uint4 *>(tb + nb * 32 * kPitch + chunk);
}

// MFMAs of one K-step: per 16-byte piece q, 2 x NBR independent MFMAs
// (consecutive MFMAs never share an accumulator) over the wave's two weight
// fragments and the NBR live token fragments.  NBR is a compile-time count
// (the tile is dispatched on it once), so the step is straight-line code.
// The reads of piece q + 1 are issued before the MFMAs of piece q, so the
// LDS latency hides behind 2 x NBR MFMAs; scheduling fences keep the
// compiler from regrouping them (it would otherwise read just in time).
template <typename T, int NBR>
__device__ __forceinline__ void compute(floatx16 (&acc)[2][NBR], const char *slot_wave,
                                        const char *tile, int r, int h) {
  const char *tb = tile + r * kPitch;
  uint4 A[2][2], B[2][NBR];
  load_frags<NBR>(A[0], B[0], slot_wave, tb, r, h, 0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < 3) load_frags<NBR>(A[(q + 1) & 1], B[(q + 1) & 1], slot_wave, tb, r, h, q + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb)
#pragma unroll
      for (int a = 0; a < 2; ++a) MfmaOps<T>::piece(acc[a][nb], A[q & 1][a], B[q & 1][nb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One K-step (S = ks mod 3 selects the weight slot and the token buffer at
// compile time): the token rows and then the weights of step ks + 2 go to
// the buffers read in step ks - 1, then the MFMAs of step ks, then the wait
// and the barrier that publish step ks + 1.
//
// Each direct-to-LDS load writes 64 lanes x 16 bytes, but the compiler's
// dependence tracking sees only the 16 bytes at its base address, so the
// wait is explicit: every step (and each of the two prologue groups) issues
// NBR token loads and 8 weight loads, in program order (compiler-level
// barriers keep the groups apart), so once only the NBR + 8 loads of step
// ks + 2 remain outstanding, this wave's loads of step ks + 1 have landed;
// the barrier then covers every wave's.
template <typename T, int NBR, int S, int WAUX>
__device__ __forceinline__ void kstep(int ks, floatx16 (&acc)[2][NBR], char *const (&w)[3],
                                      char *const (&tl)[3], const TileState<NBR> &st,
                                      const uint32_t (&tvo)[NBR], int r, int h, int wave) {
  load_t<T, NBR>(tl[(S + 2) % 3], tvo, st, ks + 2, wave);
  load_w<T, NBR, WAUX>(w[(S + 2) % 3], st, ks + 2);
  asm volatile("" ::: "memory");
  compute<T, NBR>(acc, w[S], tl[S], r, h);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(NBR + 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The whole K loop and epilogue of one tile with NBR live 32-token blocks
// (NBR <= NB; the LDS buffers are sized for NB).
template <typename T, int MODE, int NBR>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, const TileLoc &t,
                                          char *const (&s_w)[3], char *const (&tl)[3]) {
  constexpr int KC = 128 / sizeof(T);  // K elements per step (128 bytes per row)
  constexpr uint32_t ES = sizeof(T);
  // the router's weights are read by every token tile; expert weights once
  constexpr int kWAux = MODE == MODE_ROUTER ? kReuse : kStreamOnce;
  const int e = t.e, rb = t.rb, m0 = t.m0, mcount = t.mcount;
  const uint32_t kbyte0 = static_cast<uint32_t>(t.k0) * ES;  // first byte of the K range in a row

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 31;
  const int h = lane >> 5;
  const int K = g.K;  // row length (elements); this tile reduces over t.klen of them

  TileState<NBR> st;
  st.K = t.klen;
  // ---- the 64 weight rows of this wave (MFMA A operand) -------------------
  const uint32_t wbytes = static_cast<uint32_t>(g.nrows) * static_cast<uint32_t>(K) * ES;
  int rowbase[2];  // first weight row of each 32-row block
  constexpr bool kGateUp = MODE == MODE_GATE_UP || MODE == MODE_GATE_UP_RAW;
  if (kGateUp) {
    rowbase[0] = rowbase[1] = rb * 128 + wave * 32;  // block 0: W_gate, block 1: W_up
    st.ra[0] = make_rsrc(static_cast<const char *>(g.wa) + e * g.w_expert_stride * ES, wbytes);
    st.ra[1] = make_rsrc(static_cast<const char *>(g.wb) + e * g.w_expert_stride * ES, wbytes);
  } else {
    rowbase[0] = rb * 256 + wave * 64;
    rowbase[1] = rowbase[0] + 32;
    st.ra[0] = st.ra[1] =
        make_rsrc(static_cast<const char *>(g.wa) + e * g.w_expert_stride * ES, wbytes);
  }
  const int lr = lane >> 3;  // row within an 8-row group
  // logical 16-byte chunk this lane loads: weight rows of an 8-row group
  // with bit 3 clear (par 0) or set (par 1); token rows of this wave's groups
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int c = (lane & 7) ^ lds_swz(par * 8 + lr);
    st.wchunk[par] = c * 16;
    st.wkpos[par] = c * (16 / static_cast<int>(ES));
  }
  const int chunk = (lane & 7) ^ lds_swz((wave & 1) * 8 + lr);
  st.tkpos = chunk * (16 / static_cast<int>(ES));
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      st.wrow[a][j] =
          static_cast<uint32_t>(min(rowbase[a] + j * 8 + lr, g.nrows - 1)) * K * ES + kbyte0;

  // ---- token rows (B operand): lane (lr, chunk) of wave w loads row
  // (4i + w)*8 + lr of the chunk in instruction i ------------------------
  if (kGateUp) {
    st.rb = make_rsrc(g.src, static_cast<uint32_t>(g.T) * K * ES);  // all of x (gathered)
  } else {
    st.rb = make_rsrc(static_cast<const char *>(g.src) + static_cast<int64_t>(m0) * K * ES,
                      static_cast<uint32_t>(mcount) * K * ES);
  }
  uint32_t tvo[NBR];
#pragma unroll
  for (int i = 0; i < NBR; ++i) {
    const int tr = (i * 4 + wave) * 8 + lr;
    // The index load is clamped and its value always used (rows past the
    // chunk get kOOB added: an offset past every buffer's range), so the
    // compiler cannot sink it under a branch, and the NBR loads issue
    // together instead of one round trip each.
    const uint32_t row = kGateUp ? static_cast<uint32_t>(g.tok[m0 + min(tr, mcount - 1)])
                                 : static_cast<uint32_t>(tr);
    tvo[i] = row * K * ES + kbyte0 + chunk * 16 + (tr < mcount ? 0u : kOOB);
  }

  const int nks = (t.klen + KC - 1) / KC;
  char *const w[3] = {s_w[0] + wave * kWaveRowBytes, s_w[1] + wave * kWaveRowBytes,
                      s_w[2] + wave * kWaveRowBytes};

  floatx16 acc[2][NBR];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][nb][i] = 0.0f;

  // ---- prologue: steps 0 and 1 in the same per-step groups as the loop ----
  load_t<T, NBR>(tl[0], tvo, st, 0, wave);
  load_w<T, NBR, kWAux>(w[0], st, 0);
  asm volatile("" ::: "memory");
  load_t<T, NBR>(tl[1], tvo, st, 1, wave);
  load_w<T, NBR, kWAux>(w[1], st, 1);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(NBR + 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // ---- main loop, unrolled by the 3 buffers -----------------------------
  int ks = 0;
  for (; ks + 3 <= nks; ks += 3) {
    kstep<T, NBR, 0, kWAux>(ks, acc, w, tl, st, tvo, r, h, wave);
    kstep<T, NBR, 1, kWAux>(ks + 1, acc, w, tl, st, tvo, r, h, wave);
    kstep<T, NBR, 2, kWAux>(ks + 2, acc, w, tl, st, tvo, r, h, wave);
  }
  if (ks < nks) kstep<T, NBR, 0, kWAux>(ks, acc, w, tl, st, tvo, r, h, wave);
  if (ks + 1 < nks) kstep<T, NBR, 1, kWAux>(ks + 1, acc, w, tl, st, tvo, r, h, wave);

  // Drain the prefetches past the end of K (they read zeros into buffers
  // that are never read) so that no direct-to-LDS write is still in flight
  // when the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");

  // ---- epilogue ----------------------------------------------------------
  if constexpr (std::is_same<T, bf16_t>::value && MODE != MODE_ROUTER) {
    // The ring is reused as four wave-private staging areas: every wave's
    // prefetches past K have landed (each drained its own) before any wave
    // writes into it.
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    char *const st = wave == 0 ? tl[0] : (wave == 1 ? tl[1] : (wave == 2 ? tl[2] : s_w[0]));
    stage_epilogue<MODE, NBR>(g.out, g.out2, g.out_ld, g.nrows, t, acc, st, rowbase[0], r, h, lane);
    return;
  }
  // fp32 storage and the router's partial logits: straight from registers
  // (GATE_UP_RAW exists for bf16 only).
  // Lane (r, h) holds, for column r of each 32x32 tile, rows
  // gi*8 + h*4 + [0, 4) in acc elements gi*4 .. gi*4+3.
#pragma unroll
  for (int nb = 0; nb < NBR; ++nb) {
    const int col = nb * 32 + r;
    if (col >= mcount) continue;
    if (MODE == MODE_ROUTER) {
      float *orow = static_cast<float *>(g.out) + t.s * g.part_stride +
                    (static_cast<int64_t>(m0) + col) * g.out_ld;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = rowbase[a] + gi * 8 + h * 4 + j;
            if (row < g.nrows) orow[row] = acc[a][nb][gi * 4 + j];
          }
    } else if (MODE == MODE_GATE_UP) {
      T *orow = static_cast<T *>(g.out) + (static_cast<int64_t>(m0) + col) * g.out_ld;
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int row = rowbase[0] + gi * 8 + h * 4;
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
          const int row = rowbase[a] + gi * 8 + h * 4;
          if (row < g.nrows)
            store4<T>(orow + row, acc[a][nb][gi * 4 + 0], acc[a][nb][gi * 4 + 1],
                      acc[a][nb][gi * 4 + 2], acc[a][nb][gi * 4 + 3]);
        }
    }
  }
}

// Live token blocks of a tile -> the specialised tile body.  bf16 dispatches
// on every count up to NB; fp32 (a parity path, not a fast path) always runs
// NB blocks, the empty ones reading zeros.
template <typename T, int MODE, int NB>
__device__ __forceinline__ void dispatch_tile(const GemmArgs &g, const TileLoc &t, int nb_rt,
                                              char *const (&s_w)[3], char *const (&tl)[3]) {
  if constexpr (!std::is_same<T, bf16_t>::value || NB == 1) {
    (void)nb_rt;
    gemm_tile<T, MODE, NB>(g, t, s_w, tl);
  } else {
  switch (nb_rt) {
#define MOEZC_TILE_CASE(n)                                      \
  case n:                                                       \
    if constexpr (n <= NB) gemm_tile<T, MODE, n>(g, t, s_w, tl); \
    break;
    MOEZC_TILE_CASE(1)
    MOEZC_TILE_CASE(2)
    MOEZC_TILE_CASE(3)
    MOEZC_TILE_CASE(4)
    MOEZC_TILE_CASE(5)
#undef MOEZC_TILE_CASE
    default:
      break;
  }
  }
}

template <typename T, int MODE, int NB>
__global__ void __launch_bounds__(kThreads) gemm_kernel(GemmArgs g) {
  constexpr int MT = NB * 32;  // tokens per chunk
  // Three weight slots and three token tiles as distinct LDS objects: the
  // compiler tracks the direct-to-LDS loads of each separately.  At NB = 5
  // they take 156 KB of the 160 KB.
  __shared__ __attribute__((aligned(16))) char s_w0[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w1[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w2[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t0;
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t1;
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t2;

  // ---- which tile -------------------------------------------------------
  int ntiles;
  if (MODE == MODE_ROUTER) {
    ntiles = static_cast<int>((g.T + MT - 1) / MT) * g.nrb * g.split;
  } else {
    ntiles = g.meta[0] * g.nrb;
  }
  const int v = MODE == MODE_ROUTER ? xcd_tile(ntiles) : xcd_tile_grouped(ntiles, xcd_group(g.nrb));
  if (v < 0) return;

  TileLoc t;
  t.e = 0;
  t.k0 = 0;
  t.klen = g.K;
  t.s = 0;
  if (MODE == MODE_ROUTER) {
    // K slice outermost, then row block, then token chunk
    const int nch = static_cast<int>((g.T + MT - 1) / MT);
    t.s = v / (g.nrb * nch);
    const int rem = v - t.s * g.nrb * nch;
    t.rb = rem / nch;
    const int ch = rem % nch;
    t.m0 = ch * MT;
    t.mcount = static_cast<int>(min<int64_t>(MT, g.T - t.m0));
    t.k0 = t.s * g.kslice;
    t.klen = min(g.kslice, g.K - t.k0);
  } else {
    t = locate_expert_tile(g, v, MT);
  }
  const int nb_rt = (t.mcount + 31) / 32;
  char *const s_w[3] = {s_w0, s_w1, s_w2};
  char *const tl[3] = {s_t0, s_t1, s_t2};
  dispatch_tile<T, MODE, NB>(g, t, nb_rt, s_w, tl);
}

// Weight rows one workgroup covers (GATE_UP: per matrix).
static int rows_per_wg(int mode) {
  return mode == MODE_GATE_UP || mode == MODE_GATE_UP_RAW ? 128 : 256;
}

// ---- the 8-wave expert GEMM (bf16 expert modes, 160-token chunks) --------
// The same tile, LDS layout, ring and waits as gemm_kernel, with two waves
// per SIMD: waves w and w + 4 share SIMD w % 4 and its 64-row weight group
// and split the tile's token blocks (waves 0-3 the first ceil(NBR/2), waves
// 4-7 the rest).  With one wave per SIMD, a tile whose MFMA work is large
// (hot experts, the dense FFN) stalls on the dependencies inside its wave;
// the second wave fills them (skewed GATE_UP -7%, dense FFN -8%; prod, bound
// by the weight stream, unchanged).  Each output element is still produced
// by one wave with the same MFMA sequence, so results are bit-identical to
// the 4-wave kernel's.

constexpr int kThreads8 = 512;

// Weight rows: wave (row group rg, half th) loads block a = th (rows
// th*32 .. +31 of the group: W_gate or W_up for GATE_UP), 4 instructions of
// 8 rows, with the 4-wave kernel's swizzle (instruction j's rows have bit 3
// equal to j's bit 0: chunk offset wchunk[j & 1]).
template <int AUX>
__device__ __forceinline__ void load_w8(char *slot_rg, const __amdgpu_buffer_rsrc_t &ra,
                                        const uint32_t (&wrow)[4], const uint32_t (&wchunk)[2],
                                        const int (&wkpos)[2], int klen, int ks, int th) {
  constexpr int KC = 64;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool ok = ks * KC + wkpos[j & 1] < klen;
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(slot_rg + (th * 32 + j * 8) * 128), 16,
                                             ok ? wrow[j] + ks * 128 + wchunk[j & 1] : kOOB, 0, 0,
                                             AUX);
#else
    (void)slot_rg; (void)ra; (void)wrow; (void)ok; (void)th; (void)wchunk;
#endif
  }
}

// Token rows: instruction i of wave w fills tile rows (8i + w)*8 .. +7.
template <int NBT>
__device__ __forceinline__ void load_t8(char *tile, const __amdgpu_buffer_rsrc_t &rb,
                                        const uint32_t (&tvo)[NBT > 0 ? NBT : 1], int tkpos,
                                        int klen, int ks, int wave) {
  constexpr int KC = 64;
  const bool ok = ks * KC + tkpos < klen;
#pragma unroll
  for (int i = 0; i < NBT; ++i) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rb, (lds_void *)(tile + ((i * 8 + wave) * 8) * kPitch), 16,
        (ok && tvo[i] != kOOB) ? tvo[i] + ks * 128 : kOOB, 0, 0, 0);
#else
    (void)tile; (void)rb; (void)tvo; (void)ok; (void)wave;
#endif
  }
}

template <int NBW>
__device__ __forceinline__ void compute8w(floatx16 (&acc)[2][NBW > 0 ? NBW : 1],
                                          const char *slot_rg, const char *tile, int r, int h) {
  if constexpr (NBW == 0) {
    (void)acc; (void)slot_rg; (void)tile; (void)r; (void)h;
  } else {
    const char *tb = tile + r * kPitch;
    uint4 A[2][2], B[2][NBW];
    load_frags<NBW>(A[0], B[0], slot_rg, tb, r, h, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < 3) load_frags<NBW>(A[(q + 1) & 1], B[(q + 1) & 1], slot_rg, tb, r, h, q + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int a = 0; a < 2; ++a) MfmaOps<bf16_t>::piece(acc[a][nb], A[q & 1][a], B[q & 1][nb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int NBT, int NBW, int S, int AUX>
__device__ __forceinline__ void kstep8w(int ks, floatx16 (&acc)[2][NBW > 0 ? NBW : 1],
                                        char *const (&wrg)[3],
                                        char *const (&tl)[3], const __amdgpu_buffer_rsrc_t &ra,
                                        const uint32_t (&wrow)[4], const uint32_t (&wchunk)[2],
                                        const int (&wkpos)[2], const __amdgpu_buffer_rsrc_t &rb,
                                        const uint32_t (&tvo)[NBT > 0 ? NBT : 1], int tkpos,
                                        int klen, int nb0, int r, int h, int wave, int th) {
  load_t8<NBT>(tl[(S + 2) % 3], rb, tvo, tkpos, klen, ks + 2, wave);
  load_w8<AUX>(wrg[(S + 2) % 3], ra, wrow, wchunk, wkpos, klen, ks + 2, th);
  asm volatile("" ::: "memory");
  compute8w<NBW>(acc, wrg[S], tl[S] + nb0 * 32 * kPitch, r, h);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(NBT + 4));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// one wave's part of a tile: NBR live blocks in the tile, NBW of them this
// wave's (starting at block nb0)
template <int MODE, int NBR, int NBW>
__device__ __forceinline__ void gemm_tile8w(const GemmArgs &g, const TileLoc &t,
                                            char *const (&s_w)[3], char *const (&tl)[3], int nb0) {
  // token loads per wave per step: the tile's 4*NBR groups of 8 rows go to
  // waves g % 8, so waves 0-3 take ceil(NBR/2) and waves 4-7 floor(NBR/2),
  // the same counts as their token blocks; the highest row is NBR*32 - 1
  constexpr int NBT = NBW;
  constexpr uint32_t ES = 2;
  constexpr int AUX = kStreamOnce;
  const int e = t.e, rb = t.rb, m0 = t.m0, mcount = t.mcount;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = wave & 3, th = wave >> 2;
  const int r = lane & 31, h = lane >> 5;
  const int K = g.K;
  const int klen = t.klen;
  constexpr bool kGateUp = MODE == MODE_GATE_UP || MODE == MODE_GATE_UP_RAW;
  const uint32_t wbytes = static_cast<uint32_t>(g.nrows) * static_cast<uint32_t>(K) * ES;
  int rowbase0;
  __amdgpu_buffer_rsrc_t ra;
  int myrow0;  // first weight row this wave loads (block a = th)
  if (kGateUp) {
    rowbase0 = rb * 128 + rg * 32;
    ra = make_rsrc(static_cast<const char *>(th == 0 ? g.wa : g.wb) + e * g.w_expert_stride * ES,
                   wbytes);
    myrow0 = rowbase0;
  } else {
    rowbase0 = rb * 256 + rg * 64;
    ra = make_rsrc(static_cast<const char *>(g.wa) + e * g.w_expert_stride * ES, wbytes);
    myrow0 = rowbase0 + th * 32;
  }
  const int lr = lane >> 3;
  uint32_t wchunk[2];
  int wkpos[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int c = (lane & 7) ^ lds_swz(par * 8 + lr);
    wchunk[par] = c * 16;
    wkpos[par] = c * 8;
  }
  // token rows (i*8 + wave)*8 + lr: bit 3 is wave's bit 0
  const int chunk = (lane & 7) ^ lds_swz((wave & 1) * 8 + lr);
  const int tkpos = chunk * 8;
  uint32_t wrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wrow[j] = static_cast<uint32_t>(min(myrow0 + j * 8 + lr, g.nrows - 1)) * K * ES;
  __amdgpu_buffer_rsrc_t rbuf;
  if (kGateUp)
    rbuf = make_rsrc(g.src, static_cast<uint32_t>(g.T) * K * ES);
  else
    rbuf = make_rsrc(static_cast<const char *>(g.src) + static_cast<int64_t>(m0) * K * ES,
                     static_cast<uint32_t>(mcount) * K * ES);
  uint32_t tvo[NBT > 0 ? NBT : 1];
  tvo[0] = kOOB;
#pragma unroll
  for (int i = 0; i < NBT; ++i) {
    const int tr = (i * 8 + wave) * 8 + lr;
    const uint32_t row = kGateUp ? static_cast<uint32_t>(g.tok[m0 + min(tr, mcount - 1)])
                                 : static_cast<uint32_t>(tr);
    tvo[i] = row * K * ES + chunk * 16 + (tr < mcount ? 0u : kOOB);
  }
  const int nks = (klen + 63) / 64;
  char *const wrg[3] = {s_w[0] + rg * kWaveRowBytes, s_w[1] + rg * kWaveRowBytes,
                        s_w[2] + rg * kWaveRowBytes};
  constexpr int NBX = NBW > 0 ? NBW : 1;
  floatx16 acc[2][NBX];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nb = 0; nb < NBX; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][nb][i] = 0.0f;

  // prologue: steps 0 and 1
  load_t8<NBT>(tl[0], rbuf, tvo, tkpos, klen, 0, wave);
  load_w8<AUX>(wrg[0], ra, wrow, wchunk, wkpos, klen, 0, th);
  asm volatile("" ::: "memory");
  load_t8<NBT>(tl[1], rbuf, tvo, tkpos, klen, 1, wave);
  load_w8<AUX>(wrg[1], ra, wrow, wchunk, wkpos, klen, 1, th);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(NBT + 4));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  int ks = 0;
  for (; ks + 3 <= nks; ks += 3) {
    kstep8w<NBT, NBW, 0, AUX>(ks, acc, wrg, tl, ra, wrow, wchunk, wkpos, rbuf, tvo, tkpos, klen, nb0, r, h, wave, th);
    kstep8w<NBT, NBW, 1, AUX>(ks + 1, acc, wrg, tl, ra, wrow, wchunk, wkpos, rbuf, tvo, tkpos, klen, nb0, r, h, wave, th);
    kstep8w<NBT, NBW, 2, AUX>(ks + 2, acc, wrg, tl, ra, wrow, wchunk, wkpos, rbuf, tvo, tkpos, klen, nb0, r, h, wave, th);
  }
  if (ks < nks)
    kstep8w<NBT, NBW, 0, AUX>(ks, acc, wrg, tl, ra, wrow, wchunk, wkpos, rbuf, tvo, tkpos, klen, nb0, r, h, wave, th);
  if (ks + 1 < nks)
    kstep8w<NBT, NBW, 1, AUX>(ks + 1, acc, wrg, tl, ra, wrow, wchunk, wkpos, rbuf, tvo, tkpos, klen, nb0, r, h, wave, th);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
  // the ring becomes 8 wave-private staging areas of 12 KB (96 rows)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if constexpr (NBW > 0) {
    char *st;
    if (wave < 6) st = (wave < 2 ? s_w[0] : (wave < 4 ? s_w[1] : s_w[2])) + (wave & 1) * 12288;
    else st = wave == 6 ? tl[0] : tl[1];
    TileLoc ts = t;
    ts.m0 = t.m0 + nb0 * 32;
    ts.mcount = max(0, min(t.mcount - nb0 * 32, NBW * 32));
    stage_epilogue<MODE, NBW>(g.out, g.out2, g.out_ld, g.nrows, ts, acc, st, rowbase0, r, h,
                              lane);
  }
}

template <int MODE, int NBR>
__device__ __forceinline__ void gemm_tile8(const GemmArgs &g, const TileLoc &t,
                                           char *const (&s_w)[3], char *const (&tl)[3]) {
  constexpr int NBW0 = (NBR + 1) / 2, NBW1 = NBR / 2;
  if ((threadIdx.x >> 6) < 4) gemm_tile8w<MODE, NBR, NBW0>(g, t, s_w, tl, 0);
  else gemm_tile8w<MODE, NBR, NBW1>(g, t, s_w, tl, NBW0);
}

// ---- hot-expert tiles (bf16 GATE_UP / DOWN on the 8-wave kernel) ----------
// An expert with at least kHotRows permuted rows is chunked kHotMT = 256
// rows at a time (scan kernel), and each of its tiles multiplies the
// workgroup's 256 weight rows (GATE_UP: the same 128 rows of W_gate and of
// W_up) by up to 256 token rows, in K-steps of 32 elements (64-byte row
// segments) through a three-stage direct-to-LDS ring held in the three
// weight slots (per stage 16 KB of weight rows, then 16 KB of token rows).
// Wave w computes 128 weight rows x 64 tokens (w / 4: row half, for GATE_UP
// the gate and up rows of its 64 features; w % 4: token quarter): 8 MFMAs
// per 16-element piece from 6 fragments, where the 160-row tile's waves do
// 4 or 6 from 4 or 5, and each SIMD runs 16 MFMAs per piece between
// barriers instead of 10.  On a compute-bound dense GEMM this structure ran
// at 0.51 of the bf16 MFMA peak against 0.40 for the 160-row one.  The hot
// experts' weights are read by many chunks, so they keep the default cache
// policy.  A chunk of at most 128 rows (an expert's last, partial chunk) is
// a narrow tile (kNarrow): wave w computes 64 weight rows (w % 4: row
// quarter; for GATE_UP the gate and up rows of its 32 features) x 64 tokens
// (w / 4: token half), so every SIMD does half the full tile's MFMAs instead
// of two SIMDs idling on empty token quarters.  Loads, LDS layout and each
// output element's MFMA sequence are the full tile's: bit-identical results.
constexpr int kHotKS = 32;         // bf16 elements per K-step
constexpr int kHotOpB = 256 * 64;  // one operand's stage: 256 rows x 64 bytes

// 16-byte chunk swizzle of the 64-byte LDS rows: logical chunk c of row `row`
// sits at c ^ hot_swz(row).  A fragment read hands 16 consecutive rows to 16
// lanes at one logical chunk; with the swizzle from row bits 2-3 their
// granules (row * 4 + chunk) mod 16 are all distinct: no bank conflicts.
__device__ __forceinline__ int hot_swz(int row) { return (row >> 2) & 3; }

template <int MODE, bool kNarrow>
__device__ __forceinline__ void gemm_hot_tile(const GemmArgs &g, const TileLoc &t,
                                              char *const (&s_w)[3], char *const (&tl)[3]) {
  constexpr uint32_t ES = 2;
  constexpr bool kGateUp = MODE == MODE_GATE_UP;
  constexpr int NA = kNarrow ? 2 : 4;  // 32-row weight blocks per wave
  const int e = t.e, rb = t.rb, m0 = t.m0, mcount = t.mcount;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  // full: row half wr, token quarter wc; narrow: row quarter wr, token half wc
  const int wr = kNarrow ? wave & 3 : wave >> 2, wc = kNarrow ? wave >> 2 : wave & 3;
  const int r = lane & 31, h = lane >> 5;
  const int K = g.K;
  const uint32_t rowb = static_cast<uint32_t>(K) * ES;
  const uint32_t wbytes = static_cast<uint32_t>(g.nrows) * rowb;
  const char *const wa = static_cast<const char *>(g.wa) + e * g.w_expert_stride * ES;

  // Loads: instruction i of wave w fills LDS row group 8i + w of the stage
  // (16 rows x 64 bytes; groups 0-15 weight rows, 16-31 token rows); lane l
  // loads row 16 (8i + w) + l/4 of its operand into physical chunk l % 4,
  // i.e. logical chunk (l % 4) ^ hot_swz(row), which depends on l only.
  const int lr = lane >> 2;
  const int chunk = (lane & 3) ^ ((lr >> 2) & 3);
  const int kpos = chunk * 8;  // K element of this lane's chunk within a step
  __amdgpu_buffer_rsrc_t ra0, ra1;
  uint32_t wrow0, wrow1;
  if (kGateUp) {  // groups 0-7: W_gate rows rb*128 + 16w + lr; groups 8-15: W_up's
    ra0 = make_rsrc(wa, wbytes);
    ra1 = make_rsrc(static_cast<const char *>(g.wb) + e * g.w_expert_stride * ES, wbytes);
    wrow0 = wrow1 = static_cast<uint32_t>(min(rb * 128 + wave * 16 + lr, g.nrows - 1)) * rowb;
  } else {  // W_down rows rb*256 + 16 (8i + w) + lr
    ra0 = ra1 = make_rsrc(wa, wbytes);
    wrow0 = static_cast<uint32_t>(min(rb * 256 + wave * 16 + lr, g.nrows - 1)) * rowb;
    wrow1 = static_cast<uint32_t>(min(rb * 256 + 128 + wave * 16 + lr, g.nrows - 1)) * rowb;
  }
  // token rows of instructions 2 and 3 (kOOB past the chunk)
  const int tr0 = wave * 16 + lr, tr1 = 128 + wave * 16 + lr;
  __amdgpu_buffer_rsrc_t rbuf;
  uint32_t tvo0, tvo1;
  if (kGateUp) {
    rbuf = make_rsrc(g.src, static_cast<uint32_t>(g.T) * rowb);
    // clamped index loads whose values are always used, so both issue at once
    const uint32_t i0 = static_cast<uint32_t>(g.tok[m0 + min(tr0, mcount - 1)]);
    const uint32_t i1 = static_cast<uint32_t>(g.tok[m0 + min(tr1, mcount - 1)]);
    tvo0 = tr0 < mcount ? i0 * rowb : kOOB;
    tvo1 = tr1 < mcount ? i1 * rowb : kOOB;
  } else {
    rbuf = make_rsrc(static_cast<const char *>(g.src) + static_cast<int64_t>(m0) * rowb,
                     static_cast<uint32_t>(mcount) * rowb);
    tvo0 = tr0 < mcount ? static_cast<uint32_t>(tr0) * rowb : kOOB;
    tvo1 = tr1 < mcount ? static_cast<uint32_t>(tr1) * rowb : kOOB;
  }
  // Four loads per wave per stage, issued unconditionally (past K or past
  // the chunk they read zeros), so every step's wait count is the same.
  auto load_stage = [&](char *stage, int ks) {
    const bool ok = ks * kHotKS + kpos < K;
    const uint32_t ko = static_cast<uint32_t>(ks) * 64 + chunk * 16;
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra0, (lds_void *)(stage + wave * 1024), 16,
                                             ok ? wrow0 + ko : kOOB, 0, 0, kReuse);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra1, (lds_void *)(stage + (8 + wave) * 1024), 16,
                                             ok ? wrow1 + ko : kOOB, 0, 0, kReuse);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rbuf, (lds_void *)(stage + kHotOpB + wave * 1024),
                                             16, (ok && tvo0 != kOOB) ? tvo0 + ko : kOOB, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rbuf,
                                             (lds_void *)(stage + kHotOpB + (8 + wave) * 1024),
                                             16, (ok && tvo1 != kOOB) ? tvo1 + ko : kOOB, 0, 0, 0);
#else
    (void)stage; (void)ok; (void)ko;
#endif
  };

  // Fragment byte offsets within a stage, per 16-element piece q: lane
  // (r, h) reads logical chunk 2q + h of its rows.
  int aoff[2][NA], boff[2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      int row;
      if (kNarrow)  // GATE_UP: block 0 gate rows, block 1 up rows of features wr*32 + [0, 32)
        row = kGateUp ? i * 128 + wr * 32 + r : wr * 64 + i * 32 + r;
      else
        row = kGateUp ? (i < 2 ? wr * 64 + i * 32 + r : 128 + wr * 64 + (i - 2) * 32 + r)
                      : wr * 128 + i * 32 + r;
      aoff[q][i] = row * 64 + (((2 * q + h) ^ hot_swz(row)) << 4);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = wc * 64 + j * 32 + r;
      boff[q][j] = kHotOpB + row * 64 + (((2 * q + h) ^ hot_swz(row)) << 4);
    }
  }
  floatx16 acc[NA][2];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  auto compute = [&](const char *stage) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint4 fa[NA], fb[2];
#pragma unroll
      for (int i = 0; i < NA; ++i) fa[i] = *reinterpret_cast<const uint4 *>(stage + aoff[q][i]);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = *reinterpret_cast<const uint4 *>(stage + boff[q][j]);
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) MfmaOps<bf16_t>::piece(acc[i][j], fa[i], fb[j]);
    }
  };
  // One step (S = ks mod 3): the loads of step ks + 2, the MFMAs of step ks,
  // the wait that leaves only step ks + 2's four loads in flight, and the
  // barrier that publishes step ks + 1.
  auto step = [&](char *ld_stage, const char *cmp_stage, int ks) {
    load_stage(ld_stage, ks + 2);
    asm volatile("" ::: "memory");
    compute(cmp_stage);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  const int nks = (K + kHotKS - 1) / kHotKS;
  load_stage(s_w[0], 0);
  asm volatile("" ::: "memory");
  load_stage(s_w[1], 1);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  int ks = 0;
  for (; ks + 3 <= nks; ks += 3) {
    step(s_w[2], s_w[0], ks);
    step(s_w[0], s_w[1], ks + 1);
    step(s_w[1], s_w[2], ks + 2);
  }
  if (ks < nks) step(s_w[2], s_w[0], ks);
  if (ks + 1 < nks) step(s_w[0], s_w[1], ks + 1);
  // drain the loads past the end of K; after the barrier all LDS is free
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // Epilogue: each wave's 64 tokens x its features through an 8 KB staging
  // area of its own (waves 0-3 in slot 0, 4-7 in slot 1), 32 (GATE_UP) or
  // 64 (DOWN) features per pass, with the 160-row tile's staging code.
  char *const st = (wave < 4 ? s_w[0] : s_w[1]) + (wave & 3) * 8192;
  TileLoc ts = t;
  ts.m0 = m0 + wc * 64;
  ts.mcount = max(0, min(mcount - wc * 64, 64));
  (void)tl;
  if constexpr (kNarrow) {  // features rb*128 + wr*32 (GATE_UP) / rows rb*256 + wr*64 (DOWN)
    const floatx16 pr[2][2] = {{acc[0][0], acc[0][1]}, {acc[1][0], acc[1][1]}};
    stage_epilogue<MODE, 2>(g.out, nullptr, g.out_ld, g.nrows, ts, pr, st,
                            kGateUp ? rb * 128 + wr * 32 : rb * 256 + wr * 64, r, h, lane);
  } else if (kGateUp) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {  // features rb*128 + wr*64 + 32p + [0, 32): gate block p, up p + 2
      const floatx16 pr[2][2] = {{acc[p][0], acc[p][1]}, {acc[p + 2][0], acc[p + 2][1]}};
      stage_epilogue<MODE_GATE_UP, 2>(g.out, nullptr, g.out_ld, g.nrows, ts, pr, st,
                                      rb * 128 + wr * 64 + 32 * p, r, h, lane);
    }
  } else {
#pragma unroll
    for (int p = 0; p < 2; ++p) {  // features rb*256 + wr*128 + 64p + [0, 64): blocks 2p, 2p + 1
      const floatx16 pr[2][2] = {{acc[2 * p][0], acc[2 * p][1]}, {acc[2 * p + 1][0], acc[2 * p + 1][1]}};
      stage_epilogue<MODE_DOWN, 2>(g.out, nullptr, g.out_ld, g.nrows, ts, pr, st,
                                   rb * 256 + wr * 128 + 64 * p, r, h, lane);
    }
  }
}

template <int MODE, int NB>
__global__ void __launch_bounds__(kThreads8) gemm8w_kernel(GemmArgs g) {
  constexpr int MT = NB * 32;
  __shared__ __attribute__((aligned(16))) char s_w0[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w1[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w2[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t0;
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t1;
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t2;
  const int ntiles = g.meta[0] * g.nrb;
  const int v = xcd_tile_grouped(ntiles, xcd_group(g.nrb));
  if (v < 0) return;
  TileLoc t = locate_expert_tile(g, v, MT);
  const int nb_rt = (t.mcount + 31) / 32;
  char *const s_w[3] = {s_w0, s_w1, s_w2};
  char *const tl[3] = {s_t0, s_t1, s_t2};
  if constexpr (MODE == MODE_GATE_UP || MODE == MODE_DOWN) {
    if (t.mt == kHotMT) {
      if (t.mcount <= 128) gemm_hot_tile<MODE, true>(g, t, s_w, tl);
      else gemm_hot_tile<MODE, false>(g, t, s_w, tl);
      return;
    }
  }
  switch (nb_rt) {
    case 1: gemm_tile8<MODE, 1>(g, t, s_w, tl); break;
    case 2: gemm_tile8<MODE, 2>(g, t, s_w, tl); break;
    case 3: gemm_tile8<MODE, 3>(g, t, s_w, tl); break;
    case 4: gemm_tile8<MODE, 4>(g, t, s_w, tl); break;
    case 5: if constexpr (NB >= 5) gemm_tile8<MODE, 5>(g, t, s_w, tl); break;
    default: break;
  }
}

template <typename T, int MODE>
static hipError_t launch_gemm_t(const GemmArgs &g, int nb, int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const int64_t grid = MODE == MODE_ROUTER ? ((max_tiles + 7) / 8) * 8 : grouped_grid(max_tiles, xcd_group(g.nrb));
  const dim3 gd(static_cast<unsigned>(grid)), bd(kThreads);
  if constexpr (std::is_same<T, bf16_t>::value && MODE != MODE_ROUTER) {
    if (nb == 5)  // 160-token chunks: two waves per SIMD
      hipLaunchKernelGGL((gemm8w_kernel<MODE, 5>), gd, dim3(kThreads8), 0, s, g);
    else if (nb == 4)
      hipLaunchKernelGGL((gemm_kernel<T, MODE, 4>), gd, bd, 0, s, g);
    else
      hipLaunchKernelGGL((gemm_kernel<T, MODE, 1>), gd, bd, 0, s, g);
    return hipGetLastError();
  }
  if (nb == 5)
    hipLaunchKernelGGL((gemm_kernel<T, MODE, 5>), gd, bd, 0, s, g);
  else if (nb == 4)
    hipLaunchKernelGGL((gemm_kernel<T, MODE, 4>), gd, bd, 0, s, g);
  else
    hipLaunchKernelGGL((gemm_kernel<T, MODE, 1>), gd, bd, 0, s, g);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_gemm(const Plan &p, const GemmArgs &g, int nb, int64_t max_tiles,
                              hipStream_t s) {
  if (p.dtype == MOE_ZC_BF16) return launch_gemm_t<bf16_t, MODE>(g, nb, max_tiles, s);
  if constexpr (MODE == MODE_GATE_UP_RAW) return hipErrorInvalidValue;  // bf16 only
  else return launch_gemm_t<float, MODE>(g, nb, max_tiles, s);
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
  g.nrb = (p.E + rows_per_wg(MODE_ROUTER) - 1) / rows_per_wg(MODE_ROUTER);
  g.split = p.rs.split;
  g.kslice = p.rs.kslice;
  g.part_stride = p.T * p.E;
  const int nb = p.rs.nb;
  const int64_t tiles = ((p.T + 32 * nb - 1) / (32 * nb)) * g.nrb * g.split;
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
  g.nrb = (p.I + rows_per_wg(MODE_GATE_UP) - 1) / rows_per_wg(MODE_GATE_UP);
  g.N = p.N;
  g.split = 1;
  g.hot_rows = p.hot_rows;
  return launch_gemm<MODE_GATE_UP>(p, g, p.nbmax, max_chunks(p) * g.nrb, s);
}

// The backward's recomputation of both projections: G = X W_gate^T and
// U = X W_up^T per expert ([P, I] each, the dims' dtype).
hipError_t launch_gate_up_raw(const Plan &p, hipStream_t s) {
  GemmArgs g = {};
  g.wa = p.w_gate;
  g.wb = p.w_up;
  g.src = p.x;
  g.tok = p.tok;
  g.offs = p.offs;
  g.chunk_off = p.chunk_off;
  g.meta = p.meta;
  g.out = p.bG;
  g.out2 = p.bU;
  g.w_expert_stride = static_cast<int64_t>(p.I) * p.d;
  g.T = p.T;
  g.K = p.d;
  g.nrows = p.I;
  g.out_ld = p.I;
  g.nrb = (p.I + rows_per_wg(MODE_GATE_UP_RAW) - 1) / rows_per_wg(MODE_GATE_UP_RAW);
  g.N = p.N;
  g.split = 1;
  return launch_gemm<MODE_GATE_UP_RAW>(p, g, p.nbmax, max_chunks(p) * g.nrb, s);
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
  g.nrb = (p.d + rows_per_wg(MODE_DOWN) - 1) / rows_per_wg(MODE_DOWN);
  g.N = p.N;
  g.split = 1;
  g.hot_rows = p.hot_rows;
  return launch_gemm<MODE_DOWN>(p, g, p.nbmax, max_chunks(p) * g.nrb, s);
}

}  // namespace moezc
