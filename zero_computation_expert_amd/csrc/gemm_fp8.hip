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
// Everything else is the bf16 design of gemm.hip (direct-to-LDS weight ring,
// register-staged token tile, the same LDS swizzle, explicit waits, XCD-aware tile order,
// per-count tile bodies): per step the bytes moved and read from LDS are the
// same as bf16's, for twice the K.  A tile's exponents (its token rows' and
// its weight blocks' rows, K/128 bytes each) are copied into LDS once, in
// the prologue, token-major per K block so that the per-step byte reads of
// a wave's 32 tokens hit consecutive bytes.
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

// The MFMAs of one step.  The explicit wait covers the weight slot (filled
// by direct-to-LDS loads, which the compiler tracks only in part): two
// groups of NBR + 8 loads are younger than the weights of step ks.  The
// step's exponents come from the tile's LDS copy: the weight blocks' (one
// byte per 32-row block, the same for every lane) and this lane's column
// tokens'.
template <int NBR>
__device__ __forceinline__ void compute8(floatx16 (&acc)[2][NBR], const char *slot_wave,
                                         const char *tile, const uint8_t *sa_row0,
                                         const uint8_t *sa_row1, const uint8_t *sb_col, int nkb,
                                         int ks, int r, int h) {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (NBR + 8)));
  asm volatile("" ::: "memory");
  const int sa[2] = {sa_row0[ks], sa_row1[ks]};
  int sb[NBR];
#pragma unroll
  for (int nb = 0; nb < NBR; ++nb) sb[nb] = sb_col[nb * 32 * nkb + ks];
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

template <int NB, int NBR, int S>
__device__ __forceinline__ void kstep8(int ks, floatx16 (&acc)[2][NBR], char *w0, char *w1,
                                       char *w2, uint4 (&xr)[2][NBR], const TileState<NBR> &st,
                                       TileBuf<NB> *tile, const uint8_t *sa0, const uint8_t *sa1,
                                       const uint8_t *sbc, int nkb, int r, int h, int brow,
                                       int bp) {
  char *const slot_now = S % 3 == 0 ? w0 : (S % 3 == 1 ? w1 : w2);
  char *const slot_next = (S + 2) % 3 == 0 ? w0 : ((S + 2) % 3 == 1 ? w1 : w2);
  load_b<fp8_t, NBR>(xr[S & 1], st, ks + 2);
  load_w<fp8_t, NBR, kStreamOnce>(slot_next, st, ks + 2);
  compute8<NBR>(acc, slot_now, tile[ks & 1], sa0, sa1, sbc, nkb, ks, r, h);
  store_b<NBR>(tile[(ks + 1) & 1], xr[(S + 1) & 1], brow, bp);
  tile_barrier();
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
                                           char *s_w1, char *s_w2, TileBuf<NB> *s_tile,
                                           uint8_t *s_sa, uint8_t *s_sb) {
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
  {
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
  }

  // token rows (staged into LDS) and this lane's column tokens (exponents)
  const int bp = threadIdx.x & 7;
  const int brow = threadIdx.x >> 3;
  st.kpos_b = bp * 16;
  if (MODE == MODE8_GATE_UP) {
    st.rb = make_rsrc(g.src, static_cast<uint32_t>(g.T) * K);
  } else {
    st.rb = make_rsrc(static_cast<const char *>(g.src) + static_cast<int64_t>(m0) * K,
                      static_cast<uint32_t>(mcount) * K);
  }
#pragma unroll
  for (int i = 0; i < NBR; ++i) {
    const int tr = brow + 32 * i;
    // clamped index load whose value is always used (kOOB added for rows
    // past the chunk), so the NBR loads issue together
    const uint32_t row = MODE == MODE8_GATE_UP ? static_cast<uint32_t>(g.tok[m0 + min(tr, mcount - 1)])
                                               : static_cast<uint32_t>(tr);
    st.vob[i] = row * K + bp * 16 + (tr < mcount ? 0u : kOOB);
  }

  // Exponents into LDS, once per tile.  s_sa: two rows of nkb bytes, the
  // weight blocks this workgroup reads (GATE_UP: W_gate's and W_up's block
  // rb; DOWN: W_down's blocks 2 rb and 2 rb + 1, waves 0-1 and 2-3).  s_sb:
  // [mcount][nkb], the exponent rows of the tile's token rows (x's rows
  // gathered into permuted order, or H's rows), then 127 for padding.
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
  {
    // the tile's token exponent rows are contiguous (permuted row order):
    // copy mcount * nkb bytes, all loads issued before the stores
    const uint8_t *src_e = g.sb + static_cast<int64_t>(m0) * nkb;
    const int nbytes = mcount * nkb;
    constexpr int kMaxDw = (kMaxKb8 * NB * 32 / 4 + kThreads - 1) / kThreads;
    if (((reinterpret_cast<uintptr_t>(src_e) | static_cast<uintptr_t>(nbytes)) & 3) == 0) {
      const uint32_t *s32 = reinterpret_cast<const uint32_t *>(src_e);
      uint32_t *d32 = reinterpret_cast<uint32_t *>(s_sb);
      const int nd = nbytes / 4;
      uint32_t v[kMaxDw];
#pragma unroll
      for (int u = 0; u < kMaxDw; ++u) {
        const int i = threadIdx.x + u * kThreads;
        v[u] = i < nd ? s32[i] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kMaxDw; ++u) {
        const int i = threadIdx.x + u * kThreads;
        if (i < nd) d32[i] = v[u];
      }
    } else {
      for (int i = threadIdx.x; i < nbytes; i += kThreads) s_sb[i] = src_e[i];
    }
    // padding columns: exponent 127 (a scale of 1) on their zero data
    for (int i = nbytes + threadIdx.x; i < NBR * 32 * nkb; i += kThreads) s_sb[i] = 127;
  }
  const uint8_t *sa0 = MODE == MODE8_GATE_UP ? s_sa : s_sa + (wave >> 1) * nkb;
  const uint8_t *sa1 = MODE == MODE8_GATE_UP ? s_sa + nkb : sa0;
  const uint8_t *sbc = s_sb + r * nkb;  // this lane's column token in token block 0

  const int nks = (K + KC - 1) / KC;
  char *const w0 = s_w0 + wave * kWaveRowBytes;
  char *const w1 = s_w1 + wave * kWaveRowBytes;
  char *const w2 = s_w2 + wave * kWaveRowBytes;

  uint4 xr[2][NBR];
  floatx16 acc[2][NBR];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][nb][i] = 0.0f;

  // prologue: the loads of steps 0 and 1 in the main loop's group order
  load_b<fp8_t, NBR>(xr[0], st, 0);
  load_w<fp8_t, NBR, kStreamOnce>(w0, st, 0);
  asm volatile("" ::: "memory");
  store_b<NBR>(s_tile[0], xr[0], brow, bp);
  load_b<fp8_t, NBR>(xr[1], st, 1);
  load_w<fp8_t, NBR, kStreamOnce>(w1, st, 1);
  tile_barrier();  // also publishes the exponent copies

  int ks = 0;
  for (; ks + 6 <= nks; ks += 6) {
    kstep8<NB, NBR, 0>(ks, acc, w0, w1, w2, xr, st, s_tile, sa0, sa1, sbc, nkb, r, h, brow, bp);
    kstep8<NB, NBR, 1>(ks + 1, acc, w0, w1, w2, xr, st, s_tile, sa0, sa1, sbc, nkb, r, h, brow, bp);
    kstep8<NB, NBR, 2>(ks + 2, acc, w0, w1, w2, xr, st, s_tile, sa0, sa1, sbc, nkb, r, h, brow, bp);
    kstep8<NB, NBR, 3>(ks + 3, acc, w0, w1, w2, xr, st, s_tile, sa0, sa1, sbc, nkb, r, h, brow, bp);
    kstep8<NB, NBR, 4>(ks + 4, acc, w0, w1, w2, xr, st, s_tile, sa0, sa1, sbc, nkb, r, h, brow, bp);
    kstep8<NB, NBR, 5>(ks + 5, acc, w0, w1, w2, xr, st, s_tile, sa0, sa1, sbc, nkb, r, h, brow, bp);
  }
  if (ks < nks) kstep8<NB, NBR, 0>(ks, acc, w0, w1, w2, xr, st, s_tile, sa0, sa1, sbc, nkb, r, h, brow, bp);
  if (ks + 1 < nks) kstep8<NB, NBR, 1>(ks + 1, acc, w0, w1, w2, xr, st, s_tile, sa0, sa1, sbc, nkb, r, h, brow, bp);
  if (ks + 2 < nks) kstep8<NB, NBR, 2>(ks + 2, acc, w0, w1, w2, xr, st, s_tile, sa0, sa1, sbc, nkb, r, h, brow, bp);
  if (ks + 3 < nks) kstep8<NB, NBR, 3>(ks + 3, acc, w0, w1, w2, xr, st, s_tile, sa0, sa1, sbc, nkb, r, h, brow, bp);
  if (ks + 4 < nks) kstep8<NB, NBR, 4>(ks + 4, acc, w0, w1, w2, xr, st, s_tile, sa0, sa1, sbc, nkb, r, h, brow, bp);

  // drain the prefetches past the end of K before LDS is reused or released
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");

  // Lane (r, h) holds, for column r of each 32x32 tile, rows
  // gi*8 + h*4 + [0, 4) in acc elements gi*4 .. gi*4+3.
  if (MODE == MODE8_DOWN) {
    // bf16 Y staged through wave-private LDS rows, as in the bf16 kernel; the
    // barrier covers every wave's last loads and token-tile writes
    tile_barrier();
    char *const stg = wave == 0 ? s_tile[0] : (wave == 1 ? s_tile[1] : (wave == 2 ? s_w0 : s_w1));
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
  const int nkb_i = g.nrows / 128;  // H exponent row length (I / 128)
  // The workgroup's 128 quantized features of a token row are one 128-byte
  // line: the four waves write their 32 bytes of every row into one shared
  // LDS tile (16-byte chunks XOR-swizzled by row), then store whole lines.
  char *const hs = s_tile[0];
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
    if (wave == 0 && h == 0 && col < mcount)
      g.out_s[(static_cast<int64_t>(m0) + col) * nkb_i + rb] = static_cast<uint8_t>(ex + 127);
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
                                               char *s_w0, char *s_w1, char *s_w2,
                                               TileBuf<NB> *s_tile, uint8_t *s_sa, uint8_t *s_sb) {
  if constexpr (NB == 1) {
    (void)nb_rt;
    gemm8_tile<MODE, NB, 1>(g, t, s_w0, s_w1, s_w2, s_tile, s_sa, s_sb);
  } else {
    switch (nb_rt) {
#define MOEZC_TILE8_CASE(n)                                                    \
  case n:                                                              \
    if constexpr (n <= NB) gemm8_tile<MODE, NB, n>(g, t, s_w0, s_w1, s_w2, s_tile, s_sa, s_sb); \
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
  __shared__ __attribute__((aligned(16))) char s_w0[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w1[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w2[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_tile[2];
  __shared__ __attribute__((aligned(16))) uint8_t s_sa[2 * kMaxKb8];
  __shared__ __attribute__((aligned(16))) uint8_t s_sb[kMaxKb8 * NB * 32];
  const int v = xcd_tile(g.meta[0] * g.nrb);
  if (v < 0) return;
  const TileLoc t = locate_expert_tile(g, v, MT);
  dispatch_tile8<MODE, NB>(g, t, (t.mcount + 31) / 32, s_w0, s_w1, s_w2, s_tile, s_sa, s_sb);
}

template <int MODE>
static hipError_t launch_gemm8(const GemmArgs &g, int nb, int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const dim3 gd(static_cast<unsigned>(((max_tiles + 7) / 8) * 8)), bd(kThreads);
  if (nb == 5)
    hipLaunchKernelGGL((gemm8_kernel<MODE, 5>), gd, bd, 0, s, g);
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
