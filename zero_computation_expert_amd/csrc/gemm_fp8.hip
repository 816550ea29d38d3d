// gemm_fp8.hip -- the expert GEMMs with block-scaled FP8 operands (gfx950).
//
// LongCat-Flash technical-report summary page, section 6 "inference and
// deployment", custom kernels, quantization item: DeepSeek-V3-style
// fine-grained quantization, activations per [1,128] block and weights per
// [128,128] block.  This library's reading: E4M3 values with one power-of-two
// scale per block, stored as an E8M0 exponent byte (2^(byte - 127)).
//   GATE_UP8: H = silu(X W_gate^T) * (X W_up^T), then H quantized per [1,128]
//             (its 128-row I block is exactly one workgroup's rows)
//   DOWN8   : Y = H W_down^T in bf16
// Each 128-byte K-step of a row is one 128-wide scale block, so a step is two
// 32x32x64 FP8 MFMAs per (row block, token block) that apply both operands'
// exponents in hardware (the scaled MFMA takes one exponent per row of A and
// per column of B and per 32-wide K half; every lane of a row or token passes
// the same byte, which scales the whole step) and accumulate in fp32.
//
// Everything else is the bf16 design of gemm.hip (direct-to-LDS weight ring
// and token-tile ring, the same LDS swizzle, explicit waits, XCD-aware tile
// order, per-count tile bodies, two waves per SIMD for 160-token chunks):
// per step the bytes moved and read from LDS are the same as bf16's, for
// twice the K.  The weight blocks' exponents (two
// rows of K/128 bytes) are copied into LDS once per tile.  The token rows'
// exponents are stored K-block-major ([K/128, rows]), so the exponents of one
// step's tile rows are contiguous: each lane loads its column tokens' bytes
// for step ks + 2 with the step's other loads (one byte load per token
// block), into a three-deep register ring.
#include "gemm_common.h"

namespace moezc {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef uint8_t fp8_t;

enum { MODE8_GATE_UP = 1, MODE8_DOWN = 2 };

// 32 bytes of one operand row for one 32x32x64 MFMA.
struct Frag8 {
  uint4 lo, hi;
};

__device__ __forceinline__ void mfma8(floatx16 &acc, const Frag8 &a, const Frag8 &b, int sa, int sb) {
  const v8i av = {static_cast<int>(a.lo.x), static_cast<int>(a.lo.y), static_cast<int>(a.lo.z),
                  static_cast<int>(a.lo.w), static_cast<int>(a.hi.x), static_cast<int>(a.hi.y),
                  static_cast<int>(a.hi.z), static_cast<int>(a.hi.w)};
  const v8i bv = {static_cast<int>(b.lo.x), static_cast<int>(b.lo.y), static_cast<int>(b.lo.z),
                  static_cast<int>(b.lo.w), static_cast<int>(b.hi.x), static_cast<int>(b.hi.y),
                  static_cast<int>(b.hi.z), static_cast<int>(b.hi.w)};
  // formats 0/0: E4M3 for both operands; exponent bytes in bits 0..7 of sa/sb
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, sa, 0, sb);
}

// Fragments of MFMA m of a step (m = 0, 1): lane (r, h) holds the logical
// 16-byte chunks 4m + 2h and 4m + 2h + 1 of its row (the same K elements for
// A and B, so the dot products pair the right bytes), read from the weight
// slot and token tile, both swizzled by lds_swz (conflict-free reads).
template <int NBR>
__device__ __forceinline__ void load_frags8(Frag8 (&A)[2], Frag8 (&B)[NBR], const char *slot_wave,
                                            const char *tb, int r, int h, int m) {
  const int c0 = 4 * m + 2 * h;
  const int p0 = (c0 ^ lds_swz(r)) * 16, p1 = ((c0 + 1) ^ lds_swz(r)) * 16;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    A[a].lo = *reinterpret_cast<const uint4 *>(slot_wave + (a * 32 + r) * 128 + p0);
    A[a].hi = *reinterpret_cast<const uint4 *>(slot_wave + (a * 32 + r) * 128 + p1);
  }
#pragma unroll
  for (int nb = 0; nb < NBR; ++nb) {
    B[nb].lo = *reinterpret_cast<const uint4 *>(tb + nb * 32 * kPitch + p0);
    B[nb].hi = *reinterpret_cast<const uint4 *>(tb + nb * 32 * kPitch + p1);
  }
}

// The MFMAs of one step (its weights, tokens and token exponents landed at
// the end of the previous step).  The weight blocks' exponents come from the
// tile's LDS copy (one byte per 32-row block, the same for every lane), the
// column tokens' from registers.
template <int NBR>
__device__ __forceinline__ void compute8(floatx16 (&acc)[2][NBR], const char *slot_wave,
                                         const char *tile, const uint8_t *sa_row0,
                                         const uint8_t *sa_row1, const int (&sb)[NBR], int ks,
                                         int r, int h) {
  const int sa[2] = {sa_row0[ks], sa_row1[ks]};
  const char *tb = tile + r * kPitch;
  Frag8 A[2][2], B[2][NBR];
  load_frags8<NBR>(A[0], B[0], slot_wave, tb, r, h, 0);
  load_frags8<NBR>(A[1], B[1], slot_wave, tb, r, h, 1);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb)
#pragma unroll
      for (int a = 0; a < 2; ++a) mfma8(acc[a][nb], A[m][a], B[m][nb], sa[a], sb[nb]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Exponent bytes of K block ks of this lane's column tokens, one per live
// token block: eo[nb] is the token's row offset in the K-block-major
// exponent matrix (kOOB past the chunk); blocks past K read zeros.
template <int NBR>
__device__ __forceinline__ void load_e(int (&eb)[NBR], const __amdgpu_buffer_rsrc_t &re,
                                       const uint32_t (&eo)[NBR], uint32_t ldt, int ks, int nks) {
#pragma unroll
  for (int nb = 0; nb < NBR; ++nb)
    eb[nb] = __builtin_amdgcn_raw_buffer_load_b8(
        re, static_cast<int>((ks < nks && eo[nb] != kOOB) ? eo[nb] + static_cast<uint32_t>(ks) * ldt
                                                          : kOOB),
        0, 0);
}

// One K-step (S = ks mod 3 picks the ring slots at compile time): the token
// exponents, token rows and weights of step ks + 2, the MFMAs of step ks,
// then the wait that leaves only step ks + 2's 2 NBR + 8 loads in flight and
// the barrier that publishes step ks + 1.
template <int NBR, int S>
__device__ __forceinline__ void kstep8(int ks, int nks, floatx16 (&acc)[2][NBR],
                                       char *const (&w)[3], char *const (&tl)[3],
                                       int (&eb)[3][NBR], const TileState<NBR> &st,
                                       const uint32_t (&tvo)[NBR],
                                       const __amdgpu_buffer_rsrc_t &re, const uint32_t (&eo)[NBR],
                                       uint32_t ldt, const uint8_t *sa0, const uint8_t *sa1, int r,
                                       int h, int wave) {
  load_e<NBR>(eb[(S + 2) % 3], re, eo, ldt, ks + 2, nks);
  load_t<fp8_t, NBR>(tl[(S + 2) % 3], tvo, st, ks + 2, wave);
  load_w<fp8_t, NBR, kStreamOnce>(w[(S + 2) % 3], st, ks + 2);
  asm volatile("" ::: "memory");
  compute8<NBR>(acc, w[S], tl[S], sa0, sa1, eb[S], ks, r, h);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NBR + 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Smallest power of two >= amax / 448 as an exponent (clamped to E8M0's
// -127); 0 (a scale of 1) for amax = 0.
__device__ __forceinline__ int block_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  const float r = amax / 448.0f;
  const uint32_t b = __float_as_uint(r);
  const int ex = static_cast<int>((b >> 23) & 0xFF);
  const uint32_t man = b & 0x7FFFFFu;
  int e;
  if (ex == 0) {  // subnormal ratio: man * 2^-149
    const int lg = 31 - __clz(man);
    e = (man == (1u << lg) ? lg : lg + 1) - 149;
  } else {
    e = ex - 127 + (man != 0u ? 1 : 0);
  }
  return e < -127 ? -127 : e;
}

// 2^-e for e in [-127, 127], exactly.
__device__ __forceinline__ float pow2_neg(int e) {
  return e <= 126 ? __uint_as_float(static_cast<uint32_t>(127 - e) << 23)
                  : __uint_as_float(1u << 22);  // 2^-127, subnormal
}

// Four fp32 values -> four E4M3 bytes (round to nearest even) in one word.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

template <int MODE, int NB, int NBR>
__device__ __forceinline__ void gemm8_tile(const GemmArgs &g, const TileLoc &t, char *s_w0,
                                           char *s_w1, char *s_w2, char *s_t0, char *s_t1,
                                           char *s_t2, uint8_t *s_sa) {
  constexpr int KC = 128;  // FP8 elements per 128-byte step (= one scale block)
  const int e = t.e, rb = t.rb, m0 = t.m0, mcount = t.mcount;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 31;
  const int h = lane >> 5;
  const int K = g.K;
  const int nkb = K / 128;  // scale blocks per row

  TileState<NBR> st;
  st.K = K;
  const uint32_t wbytes = static_cast<uint32_t>(g.nrows) * static_cast<uint32_t>(K);
  const uint32_t sbytes = static_cast<uint32_t>(g.nrows / 128) * static_cast<uint32_t>(nkb);
  int rowbase[2];
  if (MODE == MODE8_GATE_UP) {
    rowbase[0] = rowbase[1] = rb * 128 + wave * 32;  // block 0: W_gate, block 1: W_up
    st.ra[0] = make_rsrc(static_cast<const char *>(g.wa) + e * g.w_expert_stride, wbytes);
    st.ra[1] = make_rsrc(static_cast<const char *>(g.wb) + e * g.w_expert_stride, wbytes);
  } else {
    rowbase[0] = rb * 256 + wave * 64;
    rowbase[1] = rowbase[0] + 32;
    st.ra[0] = st.ra[1] =
        make_rsrc(static_cast<const char *>(g.wa) + e * g.w_expert_stride, wbytes);
  }
  const int lr = lane >> 3;
#pragma unroll
  for (int par = 0; par < 2; ++par) {  // 8-row groups with row bit 3 clear / set
    const int c = (lane & 7) ^ lds_swz(par * 8 + lr);
    st.wchunk[par] = c * 16;
    st.wkpos[par] = c * 16;
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      st.wrow[a][j] = static_cast<uint32_t>(min(rowbase[a] + j * 8 + lr, g.nrows - 1)) * K;

  // token rows, direct to LDS: instruction i of wave w fills tile rows
  // (4i + w)*8 .. +7 (bit 3 of those rows is w's bit 0)
  const int tchunk = (lane & 7) ^ lds_swz((wave & 1) * 8 + lr);
  st.tkpos = tchunk * 16;
  if (MODE == MODE8_GATE_UP) {
    st.rb = make_rsrc(g.src, static_cast<uint32_t>(g.T) * K);
  } else {
    st.rb = make_rsrc(static_cast<const char *>(g.src) + static_cast<int64_t>(m0) * K,
                      static_cast<uint32_t>(mcount) * K);
  }
  uint32_t tvo[NBR];
#pragma unroll
  for (int i = 0; i < NBR; ++i) {
    const int tr = (i * 4 + wave) * 8 + lr;
    // clamped index load whose value is always used (kOOB added for rows
    // past the chunk), so the NBR loads issue together
    const uint32_t row = MODE == MODE8_GATE_UP ? static_cast<uint32_t>(g.tok[m0 + min(tr, mcount - 1)])
                                               : static_cast<uint32_t>(tr);
    tvo[i] = row * K + tchunk * 16 + (tr < mcount ? 0u : kOOB);
  }
  // this lane's column tokens' exponents: row m0 + nb*32 + r of each K block
  const uint32_t ldt = static_cast<uint32_t>(g.ldt);
  const __amdgpu_buffer_rsrc_t re = make_rsrc(g.sb, static_cast<uint32_t>(nkb) * ldt);
  uint32_t eo[NBR];
#pragma unroll
  for (int nb = 0; nb < NBR; ++nb)
    eo[nb] = nb * 32 + r < mcount ? static_cast<uint32_t>(m0 + nb * 32 + r) : kOOB;

  // The weight blocks' exponents into LDS, once per tile: two rows of nkb
  // bytes (GATE_UP: W_gate's and W_up's block rb; DOWN: W_down's blocks 2 rb
  // and 2 rb + 1, waves 0-1 and 2-3).  Done before the first tile loads, so
  // the waits these loads need do not hold up the load pipeline.
  for (int i = threadIdx.x; i < 2 * nkb; i += kThreads) {
    const int which = i / nkb, kb = i - which * nkb;
    const uint8_t *src_e = MODE == MODE8_GATE_UP
                               ? (which == 0 ? g.sa : g.sa2) + static_cast<int64_t>(e) * sbytes +
                                     static_cast<int64_t>(rb) * nkb
                               : g.sa + static_cast<int64_t>(e) * sbytes +
                                     static_cast<int64_t>(2 * rb + which) * nkb;
    const bool ok = MODE == MODE8_GATE_UP || (2 * rb + which) * 128 < g.nrows;
    s_sa[i] = ok ? src_e[kb] : 0;
  }
  const uint8_t *sa0 = MODE == MODE8_GATE_UP ? s_sa : s_sa + (wave >> 1) * nkb;
  const uint8_t *sa1 = MODE == MODE8_GATE_UP ? s_sa + nkb : sa0;

  const int nks = (K + KC - 1) / KC;
  char *const w[3] = {s_w0 + wave * kWaveRowBytes, s_w1 + wave * kWaveRowBytes,
                      s_w2 + wave * kWaveRowBytes};
  char *const tl[3] = {s_t0, s_t1, s_t2};

  int eb[3][NBR];
  floatx16 acc[2][NBR];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][nb][i] = 0.0f;

  // prologue: steps 0 and 1 in the loop's per-step load order
  load_e<NBR>(eb[0], re, eo, ldt, 0, nks);
  load_t<fp8_t, NBR>(tl[0], tvo, st, 0, wave);
  load_w<fp8_t, NBR, kStreamOnce>(w[0], st, 0);
  asm volatile("" ::: "memory");
  load_e<NBR>(eb[1], re, eo, ldt, 1, nks);
  load_t<fp8_t, NBR>(tl[1], tvo, st, 1, wave);
  load_w<fp8_t, NBR, kStreamOnce>(w[1], st, 1);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NBR + 8));
  asm volatile("" ::: "memory");
  tile_barrier();  // also publishes the weight exponents

  int ks = 0;
  for (; ks + 3 <= nks; ks += 3) {
    kstep8<NBR, 0>(ks, nks, acc, w, tl, eb, st, tvo, re, eo, ldt, sa0, sa1, r, h, wave);
    kstep8<NBR, 1>(ks + 1, nks, acc, w, tl, eb, st, tvo, re, eo, ldt, sa0, sa1, r, h, wave);
    kstep8<NBR, 2>(ks + 2, nks, acc, w, tl, eb, st, tvo, re, eo, ldt, sa0, sa1, r, h, wave);
  }
  if (ks < nks) kstep8<NBR, 0>(ks, nks, acc, w, tl, eb, st, tvo, re, eo, ldt, sa0, sa1, r, h, wave);
  if (ks + 1 < nks)
    kstep8<NBR, 1>(ks + 1, nks, acc, w, tl, eb, st, tvo, re, eo, ldt, sa0, sa1, r, h, wave);

  // drain the prefetches past the end of K before LDS is reused or released
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");

  // Lane (r, h) holds, for column r of each 32x32 tile, rows
  // gi*8 + h*4 + [0, 4) in acc elements gi*4 .. gi*4+3.
  if (MODE == MODE8_DOWN) {
    // bf16 Y staged through wave-private LDS rows, as in the bf16 kernel; the
    // barrier follows every wave's drain of its own direct-to-LDS loads
    tile_barrier();
    char *const stg = wave == 0 ? s_t0 : (wave == 1 ? s_t1 : (wave == 2 ? s_t2 : s_w0));
    stage_epilogue<MODE_DOWN, NBR>(g.out, nullptr, g.out_ld, g.nrows, t, acc, stg, rowbase[0], r,
                                   h, lane);
    return;
  }

  // GATE_UP8: H = silu(g) * u, quantized per token over the workgroup's 128
  // I rows (one [1,128] block): per-wave column maxima, a barrier, then
  // every wave forms the block maximum.
  // Wave w's maxima live in its own part of slot 0, which only its own
  // (now drained) direct-to-LDS loads ever wrote; H is recomputed in the
  // second pass rather than held (registers are scarce here)
  float *s_amax_mine = reinterpret_cast<float *>(s_w0 + wave * kWaveRowBytes);
#pragma unroll
  for (int nb = 0; nb < NBR; ++nb) {
    float m = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) m = fmaxf(m, fabsf(silu_mul(acc[0][nb][v], acc[1][nb][v])));
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    if (h == 0) s_amax_mine[nb * 32 + r] = m;
  }
  tile_barrier();
  // The workgroup's 128 quantized features of a token row are one 128-byte
  // line: the four waves write their 32 bytes of every row into one shared
  // LDS tile (16-byte chunks XOR-swizzled by row), then store whole lines.
  char *const hs = s_t0;
#pragma unroll
  for (int nb = 0; nb < NBR; ++nb) {
    const int col = nb * 32 + r;
    float amax = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      amax = fmaxf(amax, reinterpret_cast<const float *>(s_w0 + w * kWaveRowBytes)[nb * 32 + r]);
    const int ex = block_exponent(amax);
    const float inv = pow2_neg(ex);
    char *hrow = hs + col * 128;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const floatx16 &ga = acc[0][nb];
      const floatx16 &ua = acc[1][nb];
      const int q = wave * 2 + (gi >> 1);  // 16-byte chunk of features wave*32 + gi*8 + h*4
      *reinterpret_cast<uint32_t *>(hrow + ((q ^ (col & 7)) << 4) + (gi & 1) * 8 + h * 4) =
          pack4_e4m3(silu_mul(ga[gi * 4 + 0], ua[gi * 4 + 0]) * inv,
                     silu_mul(ga[gi * 4 + 1], ua[gi * 4 + 1]) * inv,
                     silu_mul(ga[gi * 4 + 2], ua[gi * 4 + 2]) * inv,
                     silu_mul(ga[gi * 4 + 3], ua[gi * 4 + 3]) * inv);
    }
    if (wave == 0 && h == 0 && col < mcount)  // K-block-major: [I/128, ldt]
      g.out_s[static_cast<int64_t>(rb) * g.ldt + m0 + col] = static_cast<uint8_t>(ex + 127);
  }
  tile_barrier();
  // rows (4i + wave)*8 + lane/8, 16-byte chunk lane%8; rows past the chunk
  // fall outside the tile's buffer range and are dropped
  const uint32_t tbytes = static_cast<uint32_t>(mcount) * static_cast<uint32_t>(g.out_ld);
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(static_cast<fp8_t *>(g.out) + static_cast<int64_t>(m0) * g.out_ld, tbytes);
  const int c = lane & 7;
#pragma unroll
  for (int i = 0; i < NBR; ++i) {
    const int row = (i * 4 + wave) * 8 + (lane >> 3);
    const uint4 v = *reinterpret_cast<const uint4 *>(hs + row * 128 + ((c ^ (row & 7)) << 4));
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{v.x, v.y, v.z, v.w}, ro,
        static_cast<int>(static_cast<uint32_t>(row) * static_cast<uint32_t>(g.out_ld) +
                         static_cast<uint32_t>(rb) * 128 + c * 16),
        0, kStreamOnce);
  }
}

template <int MODE, int NB>
__device__ __forceinline__ void dispatch_tile8(const GemmArgs &g, const TileLoc &t, int nb_rt,
                                               char *s_w0, char *s_w1, char *s_w2, char *s_t0,
                                               char *s_t1, char *s_t2, uint8_t *s_sa) {
  if constexpr (NB == 1) {
    (void)nb_rt;
    gemm8_tile<MODE, NB, 1>(g, t, s_w0, s_w1, s_w2, s_t0, s_t1, s_t2, s_sa);
  } else {
    switch (nb_rt) {
#define MOEZC_TILE8_CASE(n)                                                                \
  case n:                                                                                  \
    if constexpr (n <= NB) gemm8_tile<MODE, NB, n>(g, t, s_w0, s_w1, s_w2, s_t0, s_t1, s_t2, s_sa); \
    break;
      MOEZC_TILE8_CASE(1)
      MOEZC_TILE8_CASE(2)
      MOEZC_TILE8_CASE(3)
      MOEZC_TILE8_CASE(4)
      MOEZC_TILE8_CASE(5)
#undef MOEZC_TILE8_CASE
      default:
        break;
    }
  }
}

template <int MODE, int NB>
__global__ void __launch_bounds__(kThreads) gemm8_kernel(GemmArgs g) {
  constexpr int MT = NB * 32;
  // three weight slots and three token tiles as distinct LDS objects (the
  // compiler tracks each one's direct-to-LDS loads separately): 156 KB at
  // NB = 5, plus the weight blocks' exponents
  __shared__ __attribute__((aligned(16))) char s_w0[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w1[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w2[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t0;
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t1;
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t2;
  __shared__ __attribute__((aligned(16))) uint8_t s_sa[2 * kMaxKb8];
  const int v = xcd_tile_grouped(g.meta[0] * g.nrb, xcd_group(g.nrb));
  if (v < 0) return;
  const TileLoc t = locate_expert_tile(g, v, MT);
  dispatch_tile8<MODE, NB>(g, t, (t.mcount + 31) / 32, s_w0, s_w1, s_w2, s_t0, s_t1, s_t2, s_sa);
}

// ---- the 8-wave FP8 expert GEMM (160-token chunks) ------------------------
// The bf16 8-wave kernel's arrangement on the FP8 tile: waves w and w + 4
// share SIMD w % 4 and its 64-row weight group (w loads the group's first
// 32-row block, w + 4 the second) and split the tile's token blocks (waves
// 0-3 the first ceil(NBR/2), waves 4-7 the rest); each wave loads the
// exponents of its own token columns.  The second wave per SIMD hides the
// dependency stalls of the first, as in bf16.  Every output element comes
// from the same MFMA sequence as in the 4-wave kernel, so the results are
// bit-identical to it.  Measured against the 4-wave kernel on the same box:
// prod GATE_UP / DOWN -2%, skewed -8% / -7%, small -13% / -10%.
constexpr int kThreadsF8 = 512;

// Weight rows of one wave: block th of its group, 4 instructions of 8 rows
// (instruction j's rows have bit 3 equal to j's bit 0: chunk wchunk[j & 1]).
__device__ __forceinline__ void load_w8f(char *slot_rg, const __amdgpu_buffer_rsrc_t &ra,
                                         const uint32_t (&wrow)[4], const uint32_t (&wchunk)[2],
                                         const int (&wkpos)[2], int klen, int ks, int th) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool ok = ks * 128 + wkpos[j & 1] < klen;
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(slot_rg + (th * 32 + j * 8) * 128), 16,
                                             ok ? wrow[j] + ks * 128 + wchunk[j & 1] : kOOB, 0, 0,
                                             kStreamOnce);
#else
    (void)slot_rg; (void)ra; (void)wrow; (void)ok; (void)th; (void)wchunk;
#endif
  }
}

// Token rows: instruction i of wave w fills tile rows (8i + w)*8 .. +7.
template <int NBT>
__device__ __forceinline__ void load_t8f(char *tile, const __amdgpu_buffer_rsrc_t &rb,
                                         const uint32_t (&tvo)[NBT > 0 ? NBT : 1], int tkpos,
                                         int klen, int ks, int wave) {
  const bool ok = ks * 128 + tkpos < klen;
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

// The MFMAs of one step for one wave of the 8-wave kernel: the fragments of
// one MFMA half at a time (40 VGPRs instead of 80, which two waves per SIMD
// could not hold beside their accumulators without spilling).
template <int NBW>
__device__ __forceinline__ void compute8w(floatx16 (&acc)[2][NBW], const char *slot_rg,
                                          const char *tile, const uint8_t *sa_row0,
                                          const uint8_t *sa_row1, const int (&sb)[NBW], int ks,
                                          int r, int h) {
  const int sa[2] = {sa_row0[ks], sa_row1[ks]};
  const char *tb = tile + r * kPitch;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    Frag8 A[2], B[NBW];
    load_frags8<NBW>(A, B, slot_rg, tb, r, h, m);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int a = 0; a < 2; ++a) mfma8(acc[a][nb], A[a], B[nb], sa[a], sb[nb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One K-step of one wave: exponents, token rows and weights of step ks + 2,
// the MFMAs of step ks over this wave's NBW token blocks (from block nb0),
// then the wait that leaves only step ks + 2's 2 NBW + 4 loads in flight and
// the barrier that publishes step ks + 1.
template <int NBW, int S>
__device__ __forceinline__ void kstep8fw(int ks, int nks, int klen,
                                         floatx16 (&acc)[2][NBW > 0 ? NBW : 1],
                                         char *const (&wrg)[3], char *const (&tl)[3],
                                         int (&eb)[3][NBW > 0 ? NBW : 1],
                                         const __amdgpu_buffer_rsrc_t &ra,
                                         const uint32_t (&wrow)[4], const uint32_t (&wchunk)[2],
                                         const int (&wkpos)[2], const __amdgpu_buffer_rsrc_t &rbuf,
                                         const uint32_t (&tvo)[NBW > 0 ? NBW : 1], int tkpos,
                                         const __amdgpu_buffer_rsrc_t &re,
                                         const uint32_t (&eo)[NBW > 0 ? NBW : 1], uint32_t ldt,
                                         const uint8_t *sa0, const uint8_t *sa1, int nb0, int r,
                                         int h, int wave, int th) {
  if constexpr (NBW > 0) load_e<NBW>(eb[(S + 2) % 3], re, eo, ldt, ks + 2, nks);
  load_t8f<NBW>(tl[(S + 2) % 3], rbuf, tvo, tkpos, klen, ks + 2, wave);
  load_w8f(wrg[(S + 2) % 3], ra, wrow, wchunk, wkpos, klen, ks + 2, th);
  asm volatile("" ::: "memory");
  if constexpr (NBW > 0)
    compute8w<NBW>(acc, wrg[S], tl[S] + nb0 * 32 * kPitch, sa0, sa1, eb[S], ks, r, h);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NBW + 4));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One wave's part of a tile: NBR live blocks, NBW of them this wave's
// (starting at block nb0).
template <int MODE, int NBR, int NBW>
__device__ __forceinline__ void gemm8_tile8w(const GemmArgs &g, const TileLoc &t,
                                             char *const (&s_w)[3], char *const (&tl)[3],
                                             uint8_t *s_sa, int nb0) {
  constexpr int NBX = NBW > 0 ? NBW : 1;
  const int e = t.e, rb = t.rb, m0 = t.m0, mcount = t.mcount;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = wave & 3, th = wave >> 2;
  const int r = lane & 31, h = lane >> 5;
  const int K = g.K;
  const int klen = K;
  const int nkb = K / 128;
  const uint32_t wbytes = static_cast<uint32_t>(g.nrows) * static_cast<uint32_t>(K);
  const uint32_t sbytes = static_cast<uint32_t>(g.nrows / 128) * static_cast<uint32_t>(nkb);
  int rowbase0, myrow0;
  __amdgpu_buffer_rsrc_t ra;
  if (MODE == MODE8_GATE_UP) {
    rowbase0 = rb * 128 + rg * 32;  // block 0: W_gate, block 1: W_up
    ra = make_rsrc(static_cast<const char *>(th == 0 ? g.wa : g.wb) + e * g.w_expert_stride,
                   wbytes);
    myrow0 = rowbase0;
  } else {
    rowbase0 = rb * 256 + rg * 64;
    ra = make_rsrc(static_cast<const char *>(g.wa) + e * g.w_expert_stride, wbytes);
    myrow0 = rowbase0 + th * 32;
  }
  const int lr = lane >> 3;
  uint32_t wchunk[2];
  int wkpos[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {  // 8-row groups with row bit 3 clear / set
    const int c = (lane & 7) ^ lds_swz(par * 8 + lr);
    wchunk[par] = c * 16;
    wkpos[par] = c * 16;
  }
  uint32_t wrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wrow[j] = static_cast<uint32_t>(min(myrow0 + j * 8 + lr, g.nrows - 1)) * K;

  // token rows (i*8 + wave)*8 + lr: bit 3 is wave's bit 0
  const int chunk = (lane & 7) ^ lds_swz((wave & 1) * 8 + lr);
  const int tkpos = chunk * 16;
  __amdgpu_buffer_rsrc_t rbuf;
  if (MODE == MODE8_GATE_UP)
    rbuf = make_rsrc(g.src, static_cast<uint32_t>(g.T) * K);
  else
    rbuf = make_rsrc(static_cast<const char *>(g.src) + static_cast<int64_t>(m0) * K,
                     static_cast<uint32_t>(mcount) * K);
  uint32_t tvo[NBX];
  tvo[0] = kOOB;
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int tr = (i * 8 + wave) * 8 + lr;
    const uint32_t row = MODE == MODE8_GATE_UP
                             ? static_cast<uint32_t>(g.tok[m0 + min(tr, mcount - 1)])
                             : static_cast<uint32_t>(tr);
    tvo[i] = row * K + chunk * 16 + (tr < mcount ? 0u : kOOB);
  }
  // this lane's column tokens' exponents: row m0 + (nb0 + nb)*32 + r of each K block
  const uint32_t ldt = static_cast<uint32_t>(g.ldt);
  const __amdgpu_buffer_rsrc_t re = make_rsrc(g.sb, static_cast<uint32_t>(nkb) * ldt);
  uint32_t eo[NBX];
  eo[0] = kOOB;
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int col = (nb0 + nb) * 32 + r;
    eo[nb] = col < mcount ? static_cast<uint32_t>(m0 + col) : kOOB;
  }

  // the weight blocks' exponents into LDS, once per tile (as in the 4-wave kernel)
  for (int i = threadIdx.x; i < 2 * nkb; i += kThreadsF8) {
    const int which = i / nkb, kb = i - which * nkb;
    const uint8_t *src_e = MODE == MODE8_GATE_UP
                               ? (which == 0 ? g.sa : g.sa2) + static_cast<int64_t>(e) * sbytes +
                                     static_cast<int64_t>(rb) * nkb
                               : g.sa + static_cast<int64_t>(e) * sbytes +
                                     static_cast<int64_t>(2 * rb + which) * nkb;
    const bool ok = MODE == MODE8_GATE_UP || (2 * rb + which) * 128 < g.nrows;
    s_sa[i] = ok ? src_e[kb] : 0;
  }
  const uint8_t *sa0 = MODE == MODE8_GATE_UP ? s_sa : s_sa + (rg >> 1) * nkb;
  const uint8_t *sa1 = MODE == MODE8_GATE_UP ? s_sa + nkb : sa0;

  const int nks = (K + 127) / 128;
  char *const wrg[3] = {s_w[0] + rg * kWaveRowBytes, s_w[1] + rg * kWaveRowBytes,
                        s_w[2] + rg * kWaveRowBytes};
  int eb[3][NBX];
  floatx16 acc[2][NBX];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nb = 0; nb < NBX; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][nb][i] = 0.0f;

  // prologue: steps 0 and 1 in the loop's per-step load order
  if constexpr (NBW > 0) load_e<NBW>(eb[0], re, eo, ldt, 0, nks);
  load_t8f<NBW>(tl[0], rbuf, tvo, tkpos, klen, 0, wave);
  load_w8f(wrg[0], ra, wrow, wchunk, wkpos, klen, 0, th);
  asm volatile("" ::: "memory");
  if constexpr (NBW > 0) load_e<NBW>(eb[1], re, eo, ldt, 1, nks);
  load_t8f<NBW>(tl[1], rbuf, tvo, tkpos, klen, 1, wave);
  load_w8f(wrg[1], ra, wrow, wchunk, wkpos, klen, 1, th);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NBW + 4));
  asm volatile("" ::: "memory");
  tile_barrier();  // also publishes the weight exponents

  int ks = 0;
  for (; ks + 3 <= nks; ks += 3) {
    kstep8fw<NBW, 0>(ks, nks, klen, acc, wrg, tl, eb, ra, wrow, wchunk, wkpos, rbuf, tvo, tkpos, re, eo, ldt, sa0, sa1, nb0, r, h, wave, th);
    kstep8fw<NBW, 1>(ks + 1, nks, klen, acc, wrg, tl, eb, ra, wrow, wchunk, wkpos, rbuf, tvo, tkpos, re, eo, ldt, sa0, sa1, nb0, r, h, wave, th);
    kstep8fw<NBW, 2>(ks + 2, nks, klen, acc, wrg, tl, eb, ra, wrow, wchunk, wkpos, rbuf, tvo, tkpos, re, eo, ldt, sa0, sa1, nb0, r, h, wave, th);
  }
  if (ks < nks)
    kstep8fw<NBW, 0>(ks, nks, klen, acc, wrg, tl, eb, ra, wrow, wchunk, wkpos, rbuf, tvo, tkpos, re, eo, ldt, sa0, sa1, nb0, r, h, wave, th);
  if (ks + 1 < nks)
    kstep8fw<NBW, 1>(ks + 1, nks, klen, acc, wrg, tl, eb, ra, wrow, wchunk, wkpos, rbuf, tvo, tkpos, re, eo, ldt, sa0, sa1, nb0, r, h, wave, th);

  // drain the prefetches past the end of K; after the barrier the whole ring
  // is free
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  if constexpr (MODE == MODE8_DOWN) {
    // bf16 Y through 8 wave-private staging areas of 12 KB (96 rows)
    if constexpr (NBW > 0) {
      char *st;
      if (wave < 6) st = (wave < 2 ? s_w[0] : (wave < 4 ? s_w[1] : s_w[2])) + (wave & 1) * 12288;
      else st = wave == 6 ? tl[0] : tl[1];
      TileLoc ts = t;
      ts.m0 = m0 + nb0 * 32;
      ts.mcount = max(0, min(mcount - nb0 * 32, NBW * 32));
      stage_epilogue<MODE_DOWN, NBW>(g.out, nullptr, g.out_ld, g.nrows, ts, acc, st, rowbase0, r,
                                     h, lane);
    }
    return;
  } else {
    // GATE_UP8: H = silu(g) * u, quantized per token over the workgroup's
    // 128 I rows: the per-group column maxima go to s_amax[rg][column] (in
    // slot 0), a barrier, then each wave forms its columns' block maximum
    float *const s_amax = reinterpret_cast<float *>(s_w[0]);
    constexpr int kCols = 5 * 32;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      float m = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) m = fmaxf(m, fabsf(silu_mul(acc[0][nb][v], acc[1][nb][v])));
      m = fmaxf(m, __shfl_xor(m, 32, kWave));
      if (h == 0) s_amax[rg * kCols + (nb0 + nb) * 32 + r] = m;
    }
    tile_barrier();
    // the 128 quantized features of a token row are one 128-byte line: the
    // waves write their 32 bytes of each of their rows into one shared LDS
    // tile (16-byte chunks XOR-swizzled by row), then store whole lines
    char *const hs = tl[0];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int col = (nb0 + nb) * 32 + r;
      float amax = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) amax = fmaxf(amax, s_amax[w * kCols + col]);
      const int ex = block_exponent(amax);
      const float inv = pow2_neg(ex);
      char *hrow = hs + col * 128;
      const floatx16 &ga = acc[0][nb];
      const floatx16 &ua = acc[1][nb];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int q = rg * 2 + (gi >> 1);  // 16-byte chunk of features rg*32 + gi*8 + h*4
        *reinterpret_cast<uint32_t *>(hrow + ((q ^ (col & 7)) << 4) + (gi & 1) * 8 + h * 4) =
            pack4_e4m3(silu_mul(ga[gi * 4 + 0], ua[gi * 4 + 0]) * inv,
                       silu_mul(ga[gi * 4 + 1], ua[gi * 4 + 1]) * inv,
                       silu_mul(ga[gi * 4 + 2], ua[gi * 4 + 2]) * inv,
                       silu_mul(ga[gi * 4 + 3], ua[gi * 4 + 3]) * inv);
      }
      if (rg == 0 && h == 0 && col < mcount)  // K-block-major: [I/128, ldt]
        g.out_s[static_cast<int64_t>(rb) * g.ldt + m0 + col] = static_cast<uint8_t>(ex + 127);
    }
    tile_barrier();
    // rows (8i + wave)*8 + lane/8, 16-byte chunk lane%8; rows past the chunk
    // fall outside the tile's buffer range and are dropped
    const uint32_t tbytes = static_cast<uint32_t>(mcount) * static_cast<uint32_t>(g.out_ld);
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(static_cast<fp8_t *>(g.out) + static_cast<int64_t>(m0) * g.out_ld, tbytes);
    const int c = lane & 7;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int row = (i * 8 + wave) * 8 + (lane >> 3);
      const uint4 v = *reinterpret_cast<const uint4 *>(hs + row * 128 + ((c ^ (row & 7)) << 4));
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{v.x, v.y, v.z, v.w}, ro,
          static_cast<int>(static_cast<uint32_t>(row) * static_cast<uint32_t>(g.out_ld) +
                           static_cast<uint32_t>(rb) * 128 + c * 16),
          0, kStreamOnce);
    }
  }
}

template <int MODE, int NBR>
__device__ __forceinline__ void gemm8_tile8(const GemmArgs &g, const TileLoc &t,
                                            char *const (&s_w)[3], char *const (&tl)[3],
                                            uint8_t *s_sa) {
  constexpr int NBW0 = (NBR + 1) / 2, NBW1 = NBR / 2;
  if ((threadIdx.x >> 6) < 4) gemm8_tile8w<MODE, NBR, NBW0>(g, t, s_w, tl, s_sa, 0);
  else gemm8_tile8w<MODE, NBR, NBW1>(g, t, s_w, tl, s_sa, NBW0);
}

template <int MODE>
__global__ void __launch_bounds__(kThreadsF8) gemm8f_w8_kernel(GemmArgs g) {
  constexpr int NB = 5;
  constexpr int MT = NB * 32;
  __shared__ __attribute__((aligned(16))) char s_w0[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w1[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w2[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t0;
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t1;
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t2;
  __shared__ __attribute__((aligned(16))) uint8_t s_sa[2 * kMaxKb8];
  const int v = xcd_tile_grouped(g.meta[0] * g.nrb, xcd_group(g.nrb));
  if (v < 0) return;
  const TileLoc t = locate_expert_tile(g, v, MT);
  char *const s_w[3] = {s_w0, s_w1, s_w2};
  char *const tl[3] = {s_t0, s_t1, s_t2};
  switch ((t.mcount + 31) / 32) {
    case 1: gemm8_tile8<MODE, 1>(g, t, s_w, tl, s_sa); break;
    case 2: gemm8_tile8<MODE, 2>(g, t, s_w, tl, s_sa); break;
    case 3: gemm8_tile8<MODE, 3>(g, t, s_w, tl, s_sa); break;
    case 4: gemm8_tile8<MODE, 4>(g, t, s_w, tl, s_sa); break;
    case 5: gemm8_tile8<MODE, 5>(g, t, s_w, tl, s_sa); break;
    default: break;
  }
}

template <int MODE>
static hipError_t launch_gemm8(const GemmArgs &g, int nb, int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const dim3 gd(static_cast<unsigned>(grouped_grid(max_tiles, xcd_group(g.nrb)))), bd(kThreads);
  if (nb == 5)  // 160-token chunks: two waves per SIMD
    hipLaunchKernelGGL((gemm8f_w8_kernel<MODE>), gd, dim3(kThreadsF8), 0, s, g);
  else if (nb == 4)
    hipLaunchKernelGGL((gemm8_kernel<MODE, 4>), gd, bd, 0, s, g);
  else
    hipLaunchKernelGGL((gemm8_kernel<MODE, 1>), gd, bd, 0, s, g);
  return hipGetLastError();
}

static int64_t max_chunks8(const Plan &p) {
  const int64_t mt = 32 * p.nbmax;
  return p.pmax / mt + std::min<int64_t>(p.N, p.pmax) + 1;
}

hipError_t launch_gate_up8(const Plan &p, hipStream_t s) {
  GemmArgs g = {};
  g.wa = p.w_gate;
  g.wb = p.w_up;
  g.sa = p.s_gate;
  g.sa2 = p.s_up;
  g.src = p.qx;
  g.sb = p.sxp;
  g.ldt = static_cast<int>(p.pmax);
  g.tok = p.tok;
  g.offs = p.offs;
  g.chunk_off = p.chunk_off;
  g.meta = p.meta;
  g.out = p.h;
  g.out_s = p.sh;
  g.w_expert_stride = static_cast<int64_t>(p.I) * p.d;
  g.T = p.T;
  g.K = p.d;
  g.nrows = p.I;
  g.out_ld = p.I;
  g.nrb = p.I / 128;
  g.N = p.N;
  g.split = 1;
  return launch_gemm8<MODE8_GATE_UP>(g, p.nbmax, max_chunks8(p) * g.nrb, s);
}

hipError_t launch_down8(const Plan &p, hipStream_t s) {
  GemmArgs g = {};
  g.wa = p.w_down;
  g.sa = p.s_down;
  g.src = p.h;
  g.sb = p.sh;
  g.ldt = static_cast<int>(p.pmax);
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
  g.split = 1;
  return launch_gemm8<MODE8_DOWN>(g, p.nbmax, max_chunks8(p) * g.nrb, s);
}

}  // namespace moezc
