// gemm_bwd.hip -- the contractions of the block's backward on gfx950 MFMA
// (bfloat16 operands, fp32 accumulation).  The chain rule through the
// forward with the routing fixed (LongCat-Flash summary page, section 5
// "training infrastructure": grouped GEMMs for the backward, fp32 weight
// gradient accumulation fused into the GEMM epilogue):
//
//   dgrad, per FFN expert e over its permuted rows r (output rows m):
//     V   : v[r, i]  = sum_c dout[tok[r], c] W_down[e][c, i]     (m = i)
//           epilogue: h = silu(g) u from the recomputed G, U;
//           dgate partial = sum_i v h; dh = gate v;
//           dG = dh u s (1 + g (1 - s)), dU = dh g s  (s = sigmoid(g));  H = h
//     DX  : dx_e[r, c] = sum_i dG[r, i] W_gate[e][i, c] + dU[r, i] W_up[e][i, c]
//   dgrad, dense over tokens t:
//     DXR : dx_r[t, c] = sum_e dl[t, e] W_router[e, c]           (fp32 out)
//   wgrad (C += P^T Q over the rows of a segment, fp32 read-modify-write):
//     dW_down[e]  += dY_e^T H_e   (dY = gate * dout, gathered)
//     dW_gate[e]  += dG_e^T X_e,  dW_up[e] += dU_e^T X_e   (X gathered)
//     dW_router   += dl^T x
//
// Every one of these reduces over a dimension that is not contiguous in
// memory for at least one operand: the weights are stored [K-rows][M] for
// dgrad (W_down[e] is [d, I] and dgrad reduces over d), and wgrad reduces
// over rows.  Such an operand is streamed into LDS in its memory layout and
// its MFMA fragments are read with the gfx950 transposing LDS read
// (ds_read_b64_tr_b16), which gives each lane four consecutive K-rows of
// one column per instruction.  A wave's own 64 columns (the MN operand) are
// kept as 64 K-rows x 128 bytes with swizzled 16-byte chunks, so every load
// is whole lines; the workgroup-shared column operand of wgrad as 4 KB
// sub-tiles of 64 K-rows x 32 columns (64 bytes per row).  The K-contiguous
// operands of dgrad (dout, dG/dU, dl rows) use the forward's swizzled
// 128-byte token tile.
//
// Tile structure, streaming and waits follow the forward GEMM: 4 waves, 256
// output rows per workgroup (two 32-row blocks per wave) x up to 160
// columns; every operand moves HBM -> LDS with direct-to-LDS buffer loads
// into three-buffer rings, two K-steps ahead; each K-step issues exactly
// NBR + 8 loads per wave, ends with s_waitcnt vmcnt(NBR + 8) and one
// workgroup barrier.
#include "gemm_common.h"

namespace moezc {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr int kSub = 64 * 64;  // one K-step (64 rows) of a 32-column sub-tile, 64 B per row

// MFMA operand of 8 K-rows of one column from a sub-tile: lane (r, h)
// receives column r at K-rows s*16 + h*8 + [0, 8).  The transposing read
// works on groups of 16 lanes: group lane l (4b + a) supplies the address
// of row `base + b`, columns 4a .. 4a + 3, and receives column l at rows
// base + [0, 4).  Groups 0..3 are (h, column half) = (0,0), (0,1), (1,0),
// (1,1); the second read covers rows + 4.
__device__ __forceinline__ bf16x8_t tr_frag(const char *sub, int s, int lane) {
  const int grp = lane >> 4, l = lane & 15;
  const int off = (s * 16 + (grp >> 1) * 8 + (l >> 2)) * 64 + (grp & 1) * 32 + (l & 3) * 8;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(sub + off));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(sub + off + 4 * 64));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The MN operand's K-step in LDS: 64 K-rows of the wave's 64 columns, 128
// bytes per row, 16-byte chunk c of row r stored at position c ^ mn_swz(r).
// Besides the usual row & 7, rows with bit 1 set also flip chunk bit 2: the
// 32 lanes of one pass of a transposing read cover rows r0 + [0, 4) of two
// 4-chunk groups, and rows r0 and r0 + 2 share a bank half, so they must sit
// in different chunk groups to keep the read free of bank conflicts.
__device__ __forceinline__ int mn_swz(int row) { return (row & 7) ^ (((row >> 1) & 1) << 2); }

// tr_frag for that layout: the same operand as tr_frag on a 32-column
// sub-tile (columns a*32 ..), each lane's 4 columns located in the swizzled
// 128-byte row (the second read is 4 rows further, with its own swizzle).
__device__ __forceinline__ bf16x8_t tr_frag_mn(const char *region, int a, int s, int lane) {
  const int grp = lane >> 4, l = lane & 15;
  const int row = s * 16 + (grp >> 1) * 8 + (l >> 2);
  const int col = a * 32 + (grp & 1) * 16 + (l & 3) * 4;
  const int chunk = col >> 3, within = (col & 7) * 2;
  const int o0 = row * 128 + ((chunk ^ mn_swz(row)) << 4) + within;
  const int o1 = (row + 4) * 128 + ((chunk ^ mn_swz(row + 4)) << 4) + within;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(region + o0));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(region + o1));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// MFMA operand from the swizzled 128-byte-per-row token tile: row r, K
// elements s*16 + h*8 + [0, 8) (chunk 2s + h, XOR-swizzled by r & 7).
__device__ __forceinline__ bf16x8_t k_frag(const char *tb, int s, int r, int h) {
  return __builtin_bit_cast(
      bf16x8_t, *reinterpret_cast<const uint4 *>(tb + (((2 * s + h) ^ (r & 7)) * 16)));
}

__device__ __forceinline__ void mfma(floatx16 &acc, const bf16x8_t &a, const bf16x8_t &b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

template <int AUX = kReuse>
__device__ __forceinline__ void dma16(const __amdgpu_buffer_rsrc_t &rs, char *lds_base,
                                      uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)lds_base, 16, off, 0, 0, AUX);
#else
  (void)rs; (void)lds_base; (void)off;
#endif
}

// ---- operand streams ------------------------------------------------------
// An MN-contiguous operand, one wave's 64 columns per K-step: instruction i
// moves K-rows i*8 + lane/8 whole (128 bytes: 8 lanes of 16 bytes, lane
// position p loading chunk p ^ mn_swz(row)), so every read is full lines.  Up to two K halves (dx: W_gate then W_up),
// each of `K` rows and its own buffer; a step past the half's rows, or
// columns past the matrix, read zeros.
struct MnStream {
  __amdgpu_buffer_rsrc_t rs[2];
  uint32_t off[8];   // byte offset of this lane's row/column in step 0 (kOOB: no column)
  int row[8];        // K-row within a step
  uint32_t step;     // bytes per K-step (64 rows)
  int K, nks1;       // rows per half, K-steps of the first half
};

// AUX: the cache policy (the expert weights of dgrad are read once).
template <int AUX>
__device__ __forceinline__ void mn_load(char *region, const MnStream &a, int ks) {
  const int half = ks >= a.nks1 ? 1 : 0;
  const int kk = ks - half * a.nks1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool ok = a.off[i] != kOOB && kk * 64 + a.row[i] < a.K;
    dma16<AUX>(a.rs[half], region + i * 1024,
          ok ? a.off[i] + static_cast<uint32_t>(kk) * a.step : kOOB);
  }
}

// The K-contiguous token operand (dgrad): instruction i of wave w fills tile
// rows (4i + w)*8 .. +7, lane (row lr, position p) loading logical chunk
// p ^ lr, as in the forward.  Two halves as above.
template <int NBR>
struct KStream {
  __amdgpu_buffer_rsrc_t rs[2];
  uint32_t off[NBR];  // byte offset of this lane's row + chunk in step 0 (kOOB: no row)
  int kpos;           // first K element of this lane's chunk within a step
  int K, nks1;
};

template <int NBR>
__device__ __forceinline__ void k_load(char *tile, const KStream<NBR> &b, int ks, int wave) {
  const int half = ks >= b.nks1 ? 1 : 0;
  const int kk = ks - half * b.nks1;
  const bool ok = kk * 64 + b.kpos < b.K;
#pragma unroll
  for (int i = 0; i < NBR; ++i)
    dma16(b.rs[half], tile + ((i * 4 + wave) * 8) * kPitch,
          (ok && b.off[i] != kOOB) ? b.off[i] + static_cast<uint32_t>(kk) * 128 : kOOB);
}

// The MN-contiguous column operand of wgrad, shared by the workgroup:
// sub-tile i (columns i*32 ..) gets its K-rows w*16 + lane/4 from wave w.
template <int NBR>
struct NStream {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off[NBR];  // kOOB: columns past the matrix
  int row;            // K-row within a step
  uint32_t step;
  int K;
};

template <int NBR>
__device__ __forceinline__ void n_load(char *tile, const NStream<NBR> &b, int ks, int wave) {
  const bool ok = ks * 64 + b.row < b.K;
#pragma unroll
  for (int i = 0; i < NBR; ++i)
    dma16(b.rs, tile + i * kSub + wave * 1024,
          (ok && b.off[i] != kOOB) ? b.off[i] + static_cast<uint32_t>(ks) * b.step : kOOB);
}

// MFMAs of one K-step (four 16-row MFMA steps), fragments of step s + 1
// read before the MFMAs of step s.
template <bool B_TR, int NBR>
__device__ __forceinline__ void compute(floatx16 (&acc)[2][NBR], const char *wa, const char *tile,
                                        int lane) {
  const int r = lane & 31, h = lane >> 5;
  const char *tb = tile + r * kPitch;
  bf16x8_t A[2][2], B[2][NBR];
  auto frags = [&](int s, int buf) {
#pragma unroll
    for (int a = 0; a < 2; ++a) A[buf][a] = tr_frag_mn(wa, a, s, lane);
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb)
      B[buf][nb] = B_TR ? tr_frag(tile + nb * kSub, s, lane) : k_frag(tb + nb * 32 * kPitch, s, r, h);
  };
  frags(0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < 3) frags(s + 1, (s + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb)
#pragma unroll
      for (int a = 0; a < 2; ++a) mfma(acc[a][nb], A[s & 1][a], B[s & 1][nb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int N>
__device__ __forceinline__ void end_step() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The K loop shared by both kernels: LOAD(buf, ks) issues step ks's NBR + 8
// loads into ring position buf.
template <bool B_TR, int NBR, typename Load>
__device__ __forceinline__ void k_loop(floatx16 (&acc)[2][NBR], int nks, char *const (&w)[3],
                                       char *const (&tl)[3], int lane, Load load) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][nb][i] = 0.0f;
  load(0, 0);
  asm volatile("" ::: "memory");
  load(1, 1);
  asm volatile("" ::: "memory");
  end_step<NBR + 8>();
  int ks = 0;
  auto step = [&](int pos, int k) {
    load((pos + 2) % 3, k + 2);
    asm volatile("" ::: "memory");
    compute<B_TR, NBR>(acc, w[pos], tl[pos], lane);
    end_step<NBR + 8>();
  };
  for (; ks + 3 <= nks; ks += 3) {
    step(0, ks);
    step(1, ks + 1);
    step(2, ks + 2);
  }
  if (ks < nks) step(0, ks);
  if (ks + 1 < nks) step(1, ks + 1);
  // drain the zero-filled prefetches past the end of K
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
}

// ---- dgrad -----------------------------------------------------------------
enum { BW_V = 0, BW_DX = 1, BW_DXR = 2 };

struct DgradArgs {
  const void *a0, *a1;      // [K][lda] per expert (a1: second K half, DX)
  int64_t a_stride;         // elements between experts' matrices (0: one matrix)
  int lda, K, M, nrb;       // A row length (= M), K rows per half, output rows, M blocks of 256
  const void *b0, *b1;      // K-contiguous rows [.., ldb] (b1: second half, DX)
  int ldb;
  const int32_t *tok;       // V: B row of permuted row r is tok[r]
  int64_t brows;            // V: rows of b0
  const int32_t *offs, *chunk_off, *meta;  // expert segments (V, DX)
  int N;
  int64_t ndense;           // DXR: rows
  void *out;                // DX: bf16 [rows, ldo]; DXR: fp32 [rows, ldo]
  int ldo;
  const float *gate_perm;   // V: gate of each permuted row
  bf16_t *gbuf, *ubuf;      // V: G, U in; dG, dU out (in place)
  bf16_t *hbuf;             // V: H out
  float *dpart;             // V: [nrb, dpart_stride] partial dgate sums
  int64_t dpart_stride;
};

template <int MODE, int NBR>
__device__ __forceinline__ void dgrad_tile(const DgradArgs &g, const TileLoc &t,
                                           char *const (&s_w)[3], char *const (&tl)[3]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int m_base = t.rb * 256 + wave * 64;
  // A: this wave's 64 output rows are columns of the [K][lda] matrix
  MnStream a;
  const int64_t aoff = static_cast<int64_t>(t.e) * g.a_stride;
  const uint32_t abytes = static_cast<uint32_t>(g.K) * g.lda * 2;
  a.rs[0] = make_rsrc(static_cast<const bf16_t *>(g.a0) + aoff, abytes);
  a.rs[1] = make_rsrc(static_cast<const bf16_t *>(g.a1 ? g.a1 : g.a0) + aoff, abytes);
  a.step = 64u * g.lda * 2;
  a.K = g.K;
  a.nks1 = (g.K + 63) / 64;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a.row[i] = i * 8 + (lane >> 3);
    const int col = m_base + ((lane & 7) ^ mn_swz(lane >> 3)) * 8;
    a.off[i] = col < g.M ? static_cast<uint32_t>(a.row[i]) * g.lda * 2 + col * 2 : kOOB;
  }
  // B: the tile's rows, K-contiguous
  KStream<NBR> b;
  const int lr = lane >> 3, chunk = (lane & 7) ^ lr;
  b.kpos = chunk * 8;
  b.K = g.K;
  b.nks1 = a.nks1;
  if (MODE == BW_V) {
    b.rs[0] = b.rs[1] = make_rsrc(g.b0, static_cast<uint32_t>(g.brows) * g.ldb * 2);
  } else {
    const int64_t o = static_cast<int64_t>(t.m0) * g.ldb;
    const uint32_t bb = static_cast<uint32_t>(t.mcount) * g.ldb * 2;
    b.rs[0] = make_rsrc(static_cast<const bf16_t *>(g.b0) + o, bb);
    b.rs[1] = make_rsrc(static_cast<const bf16_t *>(g.b1 ? g.b1 : g.b0) + o, bb);
  }
#pragma unroll
  for (int i = 0; i < NBR; ++i) {
    const int tr = (i * 4 + wave) * 8 + lr;
    // clamped index load whose value is always used (kOOB added for rows
    // past the tile), so the NBR loads issue together
    const uint32_t row = MODE == BW_V ? static_cast<uint32_t>(g.tok[t.m0 + min(tr, t.mcount - 1)])
                                      : static_cast<uint32_t>(tr);
    b.off[i] = row * g.ldb * 2 + chunk * 16 + (tr < t.mcount ? 0u : kOOB);
  }
  char *const w[3] = {s_w[0] + wave * kWaveRowBytes, s_w[1] + wave * kWaveRowBytes,
                      s_w[2] + wave * kWaveRowBytes};
  const int nks = a.nks1 * (MODE == BW_DX ? 2 : 1);
  floatx16 acc[2][NBR];
  k_loop<false, NBR>(acc, nks, w, tl, lane, [&](int pos, int ks) {
    k_load<NBR>(tl[pos], b, ks, wave);
    mn_load<MODE == BW_DXR ? kReuse : kStreamOnce>(w[pos], a, ks);
  });

  // ---- epilogue: lane (r, h) holds column r, rows gi*8 + h*4 + [0, 4) ----
  if (MODE == BW_V) {
    float *s_part = reinterpret_cast<float *>(w[0]);  // this wave's own slot region
    // G, U (read, then overwritten by dG, dU) and H: this tile's rows through
    // buffer descriptors, edges by out-of-range offsets, every load of the
    // epilogue issued before the first use
    const int64_t rb0 = static_cast<int64_t>(t.m0) * g.M;
    const uint32_t rbytes = static_cast<uint32_t>(t.mcount) * g.M * 2;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(g.gbuf + rb0, rbytes);
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(g.ubuf + rb0, rbytes);
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(g.hbuf + rb0, rbytes);
    auto eoff = [&](int nb, int a2, int gi) -> uint32_t {
      const int col = nb * 32 + r;
      const int i0 = m_base + a2 * 32 + gi * 8 + h * 4;
      return (col < t.mcount && i0 < g.M) ? static_cast<uint32_t>(col * g.M + i0) * 2u : kOOB;
    };
    // two-deep pipeline over the 32-column blocks: the loads of block nb + 1
    // are issued before block nb is processed
    uint2 gv[2][8], uv[2][8];
    float gt[2];
    auto issue = [&](int nb, int buf) {
      gt[buf] = g.gate_perm[t.m0 + min(nb * 32 + r, t.mcount - 1)];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int o = static_cast<int>(eoff(nb, q >> 2, q & 3));
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(rg, o, 0, 0);
        const auto y = __builtin_amdgcn_raw_buffer_load_b64(ru, o, 0, 0);
        gv[buf][q] = make_uint2(x[0], x[1]);
        uv[buf][q] = make_uint2(y[0], y[1]);
      }
    };
    issue(0, 0);
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb) {
      const int cur = nb & 1;
      if (nb + 1 < NBR) issue(nb + 1, cur ^ 1);
      float dsum = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int a2 = q >> 2, gi = q & 3;
        const uint32_t gw[2] = {gv[cur][q].x, gv[cur][q].y}, uw[2] = {uv[cur][q].x, uv[cur][q].y};
        float dg[4], du[4], hh[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t gb = (j & 1) ? (gw[j >> 1] & 0xFFFF0000u) : (gw[j >> 1] << 16);
          const uint32_t ub = (j & 1) ? (uw[j >> 1] & 0xFFFF0000u) : (uw[j >> 1] << 16);
          const float gg = __uint_as_float(gb), uu = __uint_as_float(ub);
          const float sg = sigmoid_hw(gg);
          const float v = acc[a2][nb][gi * 4 + j];
          hh[j] = gg * sg * uu;
          dsum += v * hh[j];  // zero for rows past the tile (G, U read as zeros)
          const float dh = gt[cur] * v;
          dg[j] = dh * uu * sg * (1.0f + gg * (1.0f - sg));
          du[j] = dh * gg * sg;
        }
        auto pack = [](const float (&f)[4]) {
          return make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
        };
        const int o = static_cast<int>(eoff(nb, a2, gi));
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const uint2 pg = pack(dg), pu = pack(du), ph = pack(hh);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pg.x, pg.y}, rg, o, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pu.x, pu.y}, ru, o, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{ph.x, ph.y}, rh, o, 0, 0);
      }
      dsum += __shfl_xor(dsum, 32, kWave);
      if (h == 0) s_part[nb * 32 + r] = dsum;
    }
    __syncthreads();
    // fixed-order sum over the 4 waves' 64-row slices of this row block
    const int c = threadIdx.x;
    if (c < NBR * 32 && c < t.mcount) {
      float sum = 0.0f;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv)
        sum += reinterpret_cast<const float *>(s_w[0] + wv * kWaveRowBytes)[c];
      g.dpart[static_cast<int64_t>(t.rb) * g.dpart_stride + t.m0 + c] = sum;
    }
  } else if (MODE == BW_DX) {
    // bf16 dx rows of the tile (the wave's 64 contiguous columns from
    // m_base) staged through wave-private LDS rows in the idle ring, as in
    // the forward expert GEMMs
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    char *const st = wave == 0 ? tl[0] : (wave == 1 ? tl[1] : (wave == 2 ? tl[2] : s_w[0]));
    stage_epilogue<MODE_DOWN, NBR>(g.out, nullptr, g.ldo, g.M, t, acc, st, m_base, r, h, lane);
  } else {
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb) {
      const int col = nb * 32 + r;
      if (col >= t.mcount) continue;
      const int64_t orow = (static_cast<int64_t>(t.m0) + col) * g.ldo;
#pragma unroll
      for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const int m = m_base + a2 * 32 + gi * 8 + h * 4;
          if (m >= g.M) continue;
          const floatx16 &v = acc[a2][nb];
          store4<float>(static_cast<float *>(g.out) + orow + m, v[gi * 4], v[gi * 4 + 1],
                        v[gi * 4 + 2], v[gi * 4 + 3]);
        }
    }
  }
}

template <int MODE, int NB>
__global__ void __launch_bounds__(kThreads) dgrad_kernel(DgradArgs g) {
  constexpr int MT = NB * 32;
  __shared__ __attribute__((aligned(16))) char s_w0[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w1[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w2[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t0;
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t1;
  __shared__ __attribute__((aligned(16))) TileBuf<NB> s_t2;
  TileLoc t;
  if (MODE == BW_DXR) {
    const int nch = static_cast<int>((g.ndense + MT - 1) / MT);
    const int v = xcd_tile(nch * g.nrb);
    if (v < 0) return;
    t.e = 0;
    t.rb = v / nch;
    t.m0 = (v % nch) * MT;
    t.mcount = static_cast<int>(min<int64_t>(MT, g.ndense - t.m0));
  } else {
    const int v = xcd_tile(g.meta[0] * g.nrb);
    if (v < 0) return;
    t = locate_segment_tile(g.offs, g.chunk_off, g.N, g.nrb, v, MT);
  }
  char *const s_w[3] = {s_w0, s_w1, s_w2};
  char *const tl[3] = {s_t0, s_t1, s_t2};
  switch ((t.mcount + 31) / 32) {
#define MOEZC_DG_CASE(n)                                   \
  case n:                                                  \
    if constexpr (n <= NB) dgrad_tile<MODE, n>(g, t, s_w, tl); \
    break;
    MOEZC_DG_CASE(1)
    MOEZC_DG_CASE(2)
    MOEZC_DG_CASE(3)
    MOEZC_DG_CASE(4)
    MOEZC_DG_CASE(5)
#undef MOEZC_DG_CASE
    default:
      break;
  }
}

// ---- wgrad -----------------------------------------------------------------
struct WgradArgs {
  const void *p, *q;        // [rows, ldp] (columns = output rows m), [rows, ldq] (columns n)
  int ldp, ldq;
  int M, Ncols;             // output [M, Ncols] per segment, fp32
  float *c;
  int64_t c_stride;         // elements between segments' outputs
  const int32_t *offs;      // [nseg + 1] row ranges; null: one segment of `rows` rows
  int nseg;
  int64_t rows;
  int nmb, nnb;             // M blocks of 256, N blocks of 32*NB
};

template <int NB, int NBR>
__device__ __forceinline__ void wgrad_tile(const WgradArgs &g, int e, int r0, int nrows, int mb,
                                           int n0, char *const (&s_w)[3], char *const (&tl)[3]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int m_base = mb * 256 + wave * 64;
  MnStream a;
  a.rs[0] = a.rs[1] = make_rsrc(static_cast<const bf16_t *>(g.p) + static_cast<int64_t>(r0) * g.ldp,
                                static_cast<uint32_t>(nrows) * g.ldp * 2);
  a.step = 64u * g.ldp * 2;
  a.K = nrows;
  a.nks1 = (nrows + 63) / 64;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a.row[i] = i * 8 + (lane >> 3);
    const int col = m_base + ((lane & 7) ^ mn_swz(lane >> 3)) * 8;
    a.off[i] = col < g.M ? static_cast<uint32_t>(a.row[i]) * g.ldp * 2 + col * 2 : kOOB;
  }
  NStream<NBR> b;
  b.rs = make_rsrc(static_cast<const bf16_t *>(g.q) + static_cast<int64_t>(r0) * g.ldq,
                   static_cast<uint32_t>(nrows) * g.ldq * 2);
  b.row = wave * 16 + (lane >> 2);
  b.step = 64u * g.ldq * 2;
  b.K = nrows;
#pragma unroll
  for (int i = 0; i < NBR; ++i) {
    const int col = n0 + i * 32 + (lane & 3) * 8;
    b.off[i] = col < g.Ncols ? static_cast<uint32_t>(b.row) * g.ldq * 2 + col * 2 : kOOB;
  }
  // The fp32 read-modify-write of C[m, n] += acc (every element has one
  // owner per launch): the tile's old values are loaded before the K loop,
  // so their HBM latency overlaps the operand stream (the loop's explicit
  // waits count them: they complete in order before the first step's
  // loads), and no branch splits the batch.
  // Buffer loads and stores with out-of-range offsets for the tile's edges:
  // no branches, so nothing splits the batch.
  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(g.c + static_cast<int64_t>(e) * g.c_stride, static_cast<uint32_t>(g.M) * g.Ncols * 4);
  auto coff = [&](int nb, int a2, int i) -> uint32_t {
    const int n = n0 + nb * 32 + r;
    const int m = m_base + a2 * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
    return (m < g.M && n < g.Ncols) ? static_cast<uint32_t>(m * g.Ncols + n) * 4u : kOOB;
  };
  // the first kPre 32-column blocks' old values are loaded before the K
  // loop (what the register file holds beside the loop), the rest after it
  constexpr int kPre = NBR < 2 ? NBR : 2;
  float old[NBR][32];
  auto load_old = [&](int nb) {
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        old[nb][a2 * 16 + i] = __uint_as_float(static_cast<uint32_t>(
            __builtin_amdgcn_raw_buffer_load_b32(rc, static_cast<int>(coff(nb, a2, i)), 0,
                                                 kStreamOnce)));
  };
#pragma unroll
  for (int nb = 0; nb < kPre; ++nb) load_old(nb);
  asm volatile("" ::: "memory");
  char *const w[3] = {s_w[0] + wave * kWaveRowBytes, s_w[1] + wave * kWaveRowBytes,
                      s_w[2] + wave * kWaveRowBytes};
  floatx16 acc[2][NBR];
  k_loop<true, NBR>(acc, a.nks1, w, tl, lane, [&](int pos, int ks) {
    n_load<NBR>(tl[pos], b, ks, wave);
    mn_load<kReuse>(w[pos], a, ks);
  });
  // ---- epilogue: C[m, n] += acc ----
#pragma unroll
  for (int nb = kPre; nb < NBR; ++nb) load_old(nb);
#pragma unroll
  for (int nb = 0; nb < NBR; ++nb)
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __builtin_amdgcn_raw_buffer_store_b32(
            __float_as_uint(old[nb][a2 * 16 + i] + acc[a2][nb][i]), rc,
            static_cast<int>(coff(nb, a2, i)), 0, kStreamOnce);
}

template <int NB>
__global__ void __launch_bounds__(kThreads) wgrad_kernel(WgradArgs g) {
  __shared__ __attribute__((aligned(16))) char s_w0[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w1[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_w2[kWSlotBytes];
  __shared__ __attribute__((aligned(16))) char s_b0[NB * kSub];
  __shared__ __attribute__((aligned(16))) char s_b1[NB * kSub];
  __shared__ __attribute__((aligned(16))) char s_b2[NB * kSub];
  const int per = g.nmb * g.nnb;
  const int v = xcd_tile(g.nseg * per);
  if (v < 0) return;
  const int e = v / per, rem = v - e * per;
  const int mb = rem / g.nnb, nbk = rem - mb * g.nnb;
  const int r0 = g.offs ? g.offs[e] : 0;
  const int nrows = g.offs ? g.offs[e + 1] - r0 : static_cast<int>(g.rows);
  if (nrows <= 0) return;
  const int n0 = nbk * NB * 32;
  char *const s_w[3] = {s_w0, s_w1, s_w2};
  char *const tl[3] = {s_b0, s_b1, s_b2};
  switch ((min(NB * 32, g.Ncols - n0) + 31) / 32) {
#define MOEZC_WG_CASE(n)                                                  \
  case n:                                                                 \
    if constexpr (n <= NB) wgrad_tile<NB, n>(g, e, r0, nrows, mb, n0, s_w, tl); \
    break;
    MOEZC_WG_CASE(1)
    MOEZC_WG_CASE(2)
    MOEZC_WG_CASE(3)
    MOEZC_WG_CASE(4)
    MOEZC_WG_CASE(5)
#undef MOEZC_WG_CASE
    default:
      break;
  }
}

// ---- launchers ------------------------------------------------------------
static int64_t bwd_max_chunks(const Plan &p) {
  const int64_t mt = 32 * p.nbmax;
  return p.pmax / mt + std::min<int64_t>(p.N, p.pmax) + 1;
}

template <int MODE>
static hipError_t launch_dgrad(const DgradArgs &g, int nb, int64_t tiles, hipStream_t s) {
  if (tiles <= 0) return hipSuccess;
  const dim3 gd(static_cast<unsigned>(((tiles + 7) / 8) * 8)), bd(kThreads);
  if (nb == 5)
    hipLaunchKernelGGL((dgrad_kernel<MODE, 5>), gd, bd, 0, s, g);
  else if (nb == 4)
    hipLaunchKernelGGL((dgrad_kernel<MODE, 4>), gd, bd, 0, s, g);
  else
    hipLaunchKernelGGL((dgrad_kernel<MODE, 1>), gd, bd, 0, s, g);
  return hipGetLastError();
}

hipError_t launch_dgrad_v(const Plan &p, hipStream_t s) {
  DgradArgs g = {};
  g.a0 = p.w_down;
  g.a_stride = static_cast<int64_t>(p.d) * p.I;
  g.lda = p.I;
  g.K = p.d;
  g.M = p.I;
  g.nrb = (p.I + 255) / 256;
  g.b0 = p.dout;
  g.ldb = p.d;
  g.tok = p.tok;
  g.brows = p.T;
  g.offs = p.offs;
  g.chunk_off = p.chunk_off;
  g.meta = p.meta;
  g.N = p.N;
  g.gate_perm = p.gate_perm;
  g.gbuf = static_cast<bf16_t *>(p.bG);
  g.ubuf = static_cast<bf16_t *>(p.bU);
  g.hbuf = static_cast<bf16_t *>(p.bH);
  g.dpart = p.dpart;
  g.dpart_stride = p.pmax;
  return launch_dgrad<BW_V>(g, p.nbmax, bwd_max_chunks(p) * g.nrb, s);
}

hipError_t launch_dgrad_x(const Plan &p, hipStream_t s) {
  DgradArgs g = {};
  g.a0 = p.w_gate;
  g.a1 = p.w_up;
  g.a_stride = static_cast<int64_t>(p.I) * p.d;
  g.lda = p.d;
  g.K = p.I;
  g.M = p.d;
  g.nrb = (p.d + 255) / 256;
  g.b0 = p.bG;  // dG
  g.b1 = p.bU;  // dU
  g.ldb = p.I;
  g.offs = p.offs;
  g.chunk_off = p.chunk_off;
  g.meta = p.meta;
  g.N = p.N;
  g.out = p.dxp;
  g.ldo = p.d;
  return launch_dgrad<BW_DX>(g, p.nbmax, bwd_max_chunks(p) * g.nrb, s);
}

hipError_t launch_dgrad_router(const Plan &p, hipStream_t s) {
  DgradArgs g = {};
  g.a0 = p.w_router;
  g.lda = p.d;
  g.K = p.E;
  g.M = p.d;
  g.nrb = (p.d + 255) / 256;
  g.b0 = p.dl;
  g.ldb = p.ldl;
  g.ndense = p.T;
  g.out = p.dxr;
  g.ldo = p.d;
  const int nb = p.T >= 128 ? 4 : 1;
  const int64_t tiles = ((p.T + 32 * nb - 1) / (32 * nb)) * g.nrb;
  return launch_dgrad<BW_DXR>(g, nb, tiles, s);
}

static hipError_t launch_wgrad(const WgradArgs &g0, hipStream_t s) {
  WgradArgs g = g0;
  constexpr int NB = 5;
  g.nmb = (g.M + 255) / 256;
  g.nnb = (g.Ncols + NB * 32 - 1) / (NB * 32);
  const int64_t tiles = static_cast<int64_t>(g.nseg) * g.nmb * g.nnb;
  if (tiles <= 0) return hipSuccess;
  if (tiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((wgrad_kernel<NB>), dim3(static_cast<unsigned>(((tiles + 7) / 8) * 8)),
                     dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_wgrad_down(const Plan &p, hipStream_t s) {
  WgradArgs g = {};
  g.p = p.dyp;  // gate * dout, gathered: columns c = rows of dW_down
  g.q = p.bH;   // H: columns i
  g.ldp = p.d;
  g.ldq = p.I;
  g.M = p.d;
  g.Ncols = p.I;
  g.c = p.dw_down;
  g.c_stride = static_cast<int64_t>(p.d) * p.I;
  g.offs = p.offs;
  g.nseg = p.N;
  return launch_wgrad(g, s);
}

hipError_t launch_wgrad_gate_up(const Plan &p, hipStream_t s) {
  WgradArgs g = {};
  g.p = p.bG;  // dG: columns i = rows of dW_gate
  g.q = p.xp;  // x, gathered: columns c
  g.ldp = p.I;
  g.ldq = p.d;
  g.M = p.I;
  g.Ncols = p.d;
  g.c = p.dw_gate;
  g.c_stride = static_cast<int64_t>(p.I) * p.d;
  g.offs = p.offs;
  g.nseg = p.N;
  hipError_t e = launch_wgrad(g, s);
  if (e != hipSuccess) return e;
  g.p = p.bU;
  g.c = p.dw_up;
  return launch_wgrad(g, s);
}

hipError_t launch_wgrad_router(const Plan &p, hipStream_t s) {
  WgradArgs g = {};
  g.p = p.dl;  // columns e
  g.q = p.x;   // columns c
  g.ldp = p.ldl;
  g.ldq = p.d;
  g.M = p.E;
  g.Ncols = p.d;
  g.c = p.dw_router;
  g.nseg = 1;
  g.rows = p.T;
  return launch_wgrad(g, s);
}

}  // namespace moezc
