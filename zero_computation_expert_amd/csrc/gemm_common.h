// gemm_common.h -- device building blocks shared by the expert GEMM kernels
// (bf16 / fp32 in gemm.hip, FP8 in gemm_fp8.hip): buffer descriptors, the
// per-tile load state, the direct-to-LDS weight stream, the token-row
// staging, the LDS tile barrier and the tile geometry.  The design they
// serve is described at the top of gemm.hip.
#pragma once

#include <algorithm>
#include <type_traits>

#include "moe_zc_internal.h"

namespace moezc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// GATE_UP_RAW: the gate/up GEMM writing both projections (G to out, U to
// out2) instead of their SwiGLU, for the backward.
enum { MODE_ROUTER = 0, MODE_GATE_UP = 1, MODE_DOWN = 2, MODE_GATE_UP_RAW = 3 };

struct GemmArgs {
  const void *wa;   // ROUTER: W_router; GATE_UP: W_gate; DOWN: W_down
  const void *wb;   // GATE_UP: W_up
  const void *src;  // token rows: x (ROUTER, GATE_UP) or H (DOWN)
  const int32_t *tok;        // GATE_UP: token of each permuted row
  const int32_t *offs;       // [N+1] permuted row offsets (GATE_UP, DOWN)
  const int32_t *chunk_off;  // [N+1] chunk prefix (GATE_UP, DOWN)
  const int32_t *meta;       // meta[0] = total chunks (GATE_UP, DOWN)
  void *out;                 // logits (f32) / H / Y / G (GATE_UP_RAW)
  void *out2;                // GATE_UP_RAW: U
  int64_t w_expert_stride;   // elements between experts' matrices
  int64_t T;                 // tokens (ROUTER: chunking; GATE_UP: rows of x)
  int K;                     // reduction length
  int nrows;                 // weight rows per expert (E, I or d)
  int out_ld;                // elements per output row
  int nrb;                   // row blocks per chunk
  int N;                     // FFN experts (GATE_UP, DOWN)
  int split;                 // ROUTER: K slices (1 = no split)
  int kslice;                // ROUTER: K elements per slice
  int64_t part_stride;       // ROUTER: elements between slices' partial logits
  // FP8 experts: E8M0 exponents (2^(byte - 127)) of the 128-wide K blocks
  const uint8_t *sa;   // weights [N, nrows/128, K/128] (GATE_UP: W_gate)
  const uint8_t *sa2;  // GATE_UP: W_up, same layout
  const uint8_t *sb;   // token rows' exponents, K-block-major [K/128, ldt] (x's rows in
                       // permuted order, or H's rows)
  uint8_t *out_s;      // GATE_UP: exponents of the quantized H, [I/128, ldt]
  int ldt;             // row length of those exponent matrices (>= the permuted rows)
  int hot_rows;        // bf16 GATE_UP / DOWN: experts with at least this many rows are
                       // chunked kHotMT rows at a time (hot-expert tiles); 0: none
};

template <typename T>
__device__ __forceinline__ void store4(T *dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float *dst, float a, float b, float c, float d) {
  *reinterpret_cast<float4 *>(dst) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t *dst, float a, float b, float c, float d) {
  *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

// Logistic sigmoid 1 / (1 + e^-x) from the hardware base-2 exponential and
// reciprocal (about 1 ulp each; e^-x = 2^(-x log2 e)).  Large negative x
// gives 2^(+big) = inf and a reciprocal of 0, large positive x gives 1.
// Every caller rounds the result's products to bfloat16 or FP8.
__device__ __forceinline__ float sigmoid_hw(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}

// SwiGLU of one gate/up pair: silu(g) * u = g * sigmoid(g) * u.
__device__ __forceinline__ float silu_mul(float g, float u) { return g * sigmoid_hw(g) * u; }

constexpr int kThreads = 256;                  // 4 waves, each with two 32-row weight blocks
constexpr int kWaveRowBytes = 64 * 128;        // one K-step of a wave's 64 weight rows
constexpr int kWSlotBytes = 4 * kWaveRowBytes; // one K-step of the workgroup's weights
constexpr int kPitch = 128;  // LDS bytes per token row (16-byte chunks XOR-swizzled by row)
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past every range: the load reads zeros
// Cache policy of buffer accesses to data a launch touches once (the expert
// weight streams, the GEMM outputs, the weight gradients' read-modify-write):
// non-temporal, so it does not evict the rows that are reused (token tiles,
// operands shared by several tiles).  Measured: prod GATE_UP -3 to -10%,
// decode -11%; the outputs' stores another -1% (GATE_UP) and -5% (DOWN).
constexpr int kStreamOnce = 2;  // NT
constexpr int kReuse = 0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(off), 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// XOR swizzle of the 16-byte chunks of a 128-byte LDS row (the expert
// GEMMs' weight slots and token tiles): logical chunk c of row `row` sits at
// chunk c ^ lds_swz(row).
// The LDS serves a 16-byte read to 16 lanes per clock over 64 four-byte
// banks; a 128-byte row covers half of them, so the bank group of a chunk is
// (row & 1) * 8 + physical chunk.  The MFMA fragment reads hand lanes 0-15
// rows 0-15 (and so on), all at one logical chunk: with the swizzle taken
// from row bits 1-3, the even rows and the odd rows of any 16 consecutive
// rows each land on 8 distinct chunks, so the 16 lanes hit 16 distinct bank
// groups.  (Swizzling by row bits 0-2 put rows r and r + 8 on the same
// banks: half of all LDS cycles of the expert GEMMs were bank conflicts.)
__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & 7; }

// Per-thread state of one tile.
template <int NB>
struct TileState {
  __amdgpu_buffer_rsrc_t ra[2];  // weight matrix of each 32-row block (A operand)
  __amdgpu_buffer_rsrc_t rb;     // token rows (B operand)
  uint32_t wrow[2][4];           // byte offset of the weight row this lane loads in each
                                 // direct-to-LDS instruction (block, 8-row group)
  uint32_t wchunk[2];            // byte offset of the 16-byte chunk this lane loads, for
                                 // 8-row groups with row bit 3 clear / set
  int wkpos[2];                  // K element of that chunk within a step
  int tkpos;                     // K element of this lane's token chunk (direct-to-LDS)
  uint32_t vob[NB];              // byte offset of this thread's token row piece (or kOOB)
  int kpos_b;                    // K element of this thread's token piece within a step
  int K;
};

// Weights of K-step ks from HBM into this wave's LDS slot: 8 fully
// coalesced instructions of 8 rows x 128 bytes.  Lane l of instruction i
// loads row (i%4)*8 + l/8 of block i/4 and lands in LDS chunk l%8, which
// therefore holds the row's 16-byte chunk (l%8) ^ lds_swz(row) (wchunk).
// Chunks past K read zeros.
template <typename T, int NB, int AUX>
__device__ __forceinline__ void load_w(char *slot_wave, const TileState<NB> &st, int ks) {
  constexpr int KC = 128 / sizeof(T);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int a = i >> 2;
    const bool ok = ks * KC + st.wkpos[i & 1] < st.K;  // rows of instruction i: bit 3 = i & 1
    const uint32_t o = ks * 128 + st.wchunk[i & 1];
#if defined(__HIP_DEVICE_COMPILE__)  // the direct-to-LDS load exists only for the device
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        st.ra[a], (lds_void *)(slot_wave + (a * 32 + (i & 3) * 8) * 128), 16,
        ok ? st.wrow[a][i & 3] + o : kOOB, 0, 0, AUX);
#else
    (void)a;
    (void)o;
    (void)ok;
#endif
  }
}

// Token rows of one K-step, gathered straight into LDS: instruction i of
// wave w fills tile rows (4i + w)*8 .. +7, lane (row lr, position p) loading
// logical chunk p ^ lds_swz(row) of its row (the swizzle the fragment reads
// expect; bit 3 of those rows is w's bit 0, so the chunk is fixed per lane).
// Rows past the chunk's end and steps past K read zeros (kOOB offset); the
// instruction is issued regardless, so every step issues exactly NBR token
// loads.
template <typename T, int NBR>
__device__ __forceinline__ void load_t(char *tile, const uint32_t (&tvo)[NBR],
                                       const TileState<NBR> &st, int ks, int wave) {
  constexpr int KC = 128 / sizeof(T);
  const bool ok = ks * KC + st.tkpos < st.K;
#pragma unroll
  for (int i = 0; i < NBR; ++i) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        st.rb, (lds_void *)(tile + ((i * 4 + wave) * 8) * kPitch), 16,
        (ok && tvo[i] != kOOB) ? tvo[i] + ks * 128 : kOOB, 0, 0, 0);
#else
    (void)tile; (void)tvo; (void)st; (void)ok; (void)wave;
#endif
  }
}

// Token rows of K-step ks into registers; rows past the chunk and pieces
// past K read zeros.
template <typename T, int NB>
__device__ __forceinline__ void load_b(uint4 (&xr)[NB], const TileState<NB> &st, int ks) {
  constexpr int KC = 128 / sizeof(T);
  const bool ok = ks * KC + st.kpos_b < st.K;
#pragma unroll
  for (int i = 0; i < NB; ++i)
    xr[i] = bload(st.rb, (ok && st.vob[i] != kOOB) ? st.vob[i] + ks * 128 : kOOB);
}

// Token piece bp of tile row brow + 32 i lands in chunk bp ^ lds_swz(brow)
// of that row (the row's bits 1-3 are brow's: 32 i is a multiple of 32).
template <int NB>
__device__ __forceinline__ void store_b(char *tile, const uint4 (&xr)[NB], int brow, int bp) {
  const int chunk = (bp ^ lds_swz(brow)) * 16;
#pragma unroll
  for (int i = 0; i < NB; ++i)
    *reinterpret_cast<uint4 *>(tile + (brow + 32 * i) * kPitch + chunk) = xr[i];
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations are outstanding, leaving the other counters alone.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Workgroup barrier for the token tile.  The tile is written with ordinary
// LDS stores, so waiting for the LDS counter suffices; the weight slots are
// private to each wave and their direct-to-LDS loads stay in flight across
// the barrier (a full fence would wait for them).  The empty asm statements
// keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int NB>
using TileBuf = char[NB * 32 * kPitch];

// Where a tile sits: expert e, weight row block rb, token rows
// [m0, m0 + mcount), and the K range [k0, k0 + klen) it reduces over (all of
// K except for a split router GEMM, whose slice s writes partial logits).
struct TileLoc {
  int e, rb, m0, mcount;
  int k0, klen, s;
  int mt;  // chunk height of this tile's expert (kHotMT for a hot expert)
};


// Expert-mode tile v -> (expert, row block, token chunk).  Tiles are
// enumerated expert-major; chunk_off holds each expert's first chunk, and the
// expert of chunk c = v / nrb is the last e with chunk_off[e] <= c (a
// uniform binary search over the small prefix table, read through the
// caches).  Within an expert the chunks go in groups of kChunkGroup: group
// by group, row block next, chunk within the group fastest.  The 32 tiles
// one XCD runs at once then cover 4 row blocks x 8 chunks of an expert with
// many tokens, so its weights and its token rows are each shared by several
// concurrent tiles in L2 (the dense FFN's GATE_UP: 14.9 -> 5.2 GB of HBM
// traffic, L2 hit rate 0.41 -> 0.79).  An expert with at most kChunkGroup
// chunks keeps the plain row-block-major, chunk-fastest order.
constexpr int kChunkGroup = 8;
__device__ __forceinline__ TileLoc locate_segment_tile(const int32_t *offs,
                                                       const int32_t *chunk_off, int N, int nrb,
                                                       int v, int MT, int hot_rows = 0) {
  TileLoc t;
  t.k0 = 0;
  t.klen = 0;
  t.s = 0;
  const int c = v / nrb;
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk_off[mid] <= c) lo = mid;
    else hi = mid - 1;
  }
  t.e = lo;
  const int local = v - nrb * chunk_off[t.e];
  const int nch = chunk_off[t.e + 1] - chunk_off[t.e];
  const int nfull = nch / kChunkGroup;  // whole groups; a last, shorter one follows
  const int grp = min(local / (nrb * kChunkGroup), nfull);
  const int gw = grp < nfull ? kChunkGroup : nch - nfull * kChunkGroup;  // chunks in the group
  const int within = local - grp * nrb * kChunkGroup;
  t.rb = within / gw;
  const int ch = grp * kChunkGroup + (within - t.rb * gw);
  const int rows = offs[t.e + 1] - offs[t.e];
  t.mt = hot_rows > 0 && rows >= hot_rows ? kHotMT : MT;  // as the scan kernel chunked it
  t.m0 = offs[t.e] + ch * t.mt;
  t.mcount = min(t.mt, offs[t.e + 1] - t.m0);
  return t;
}

__device__ __forceinline__ TileLoc locate_expert_tile(const GemmArgs &g, int v, int MT) {
  TileLoc t = locate_segment_tile(g.offs, g.chunk_off, g.N, g.nrb, v, MT, g.hot_rows);
  t.klen = g.K;
  return t;
}

// Workgroup -> tile index, so that consecutive tiles land on one XCD
// (workgroups are dealt round-robin over the 8 XCDs).  -1: no tile.
__device__ __forceinline__ int xcd_tile(int ntiles) {
  const int quota = (ntiles + 7) / 8;
  const int loc = blockIdx.x / 8;
  if (loc >= quota) return -1;
  const int v = (blockIdx.x % 8) * quota + loc;
  return v < ntiles ? v : -1;
}

// Workgroup -> tile index for the expert GEMMs: the tiles go to the 8 XCDs
// in groups of G consecutive ones, dealt round-robin (group j to XCD j % 8).
// A group of G >= nrb consecutive tiles (xcd_group) holds whole token
// chunks' row blocks (for experts of more than kChunkGroup chunks, G/8 row
// blocks of an 8-chunk group), which share token rows and weights in that
// XCD's L2.  Dealing the
// groups out keeps the XCDs' loads even when tiles differ in cost: with
// contiguous eighths of the tile list, the XCDs holding a skewed workload's
// hot experts ran 20-25% longer than the others.  Each XCD starts x/8 of the
// way into its list of groups and wraps around, so that at any moment the
// XCDs stream the weights of experts far apart: run in plain order, all XCDs
// worked on neighbouring experts at once and the tiles ran slower (prod DOWN
// +4%).  Measured against contiguous eighths: skewed GATE_UP -5%, DOWN -2%,
// small -6% / -3%, prod unchanged.  The grid must be a multiple of 8G
// (grouped_grid).  -1: no tile.
__device__ __forceinline__ int xcd_tile_grouped(int ntiles, int G) {
  const int x = static_cast<int>(blockIdx.x % 8u), l = static_cast<int>(blockIdx.x / 8u);
  const int ngroups = (ntiles + G - 1) / G;
  const int nx = (ngroups - x + 7) / 8;  // groups x, x + 8, ... of this XCD
  const int lg = l / G;
  if (lg >= nx) return -1;
  const int rot = (lg + (x * nx) / 8) % nx;  // XCD x starts x/8 of the way into its list
  const int v = (rot * 8 + x) * G + l % G;
  return v < ntiles ? v : -1;
}

// Group size of xcd_tile_grouped for a launch with nrb row blocks per chunk:
// at least 32, one tile per CU of an XCD, so that a group holds several row
// blocks of a hot expert's 8-chunk group (they share its token rows) or
// several small experts' chunks.  Against G = nrb: small -2.7%, skewed
// -0.9%, prod -0.2% per step; G = 2 nrb was worse on small and prod.
__host__ __device__ __forceinline__ int xcd_group(int nrb) { return nrb > 32 ? nrb : 32; }

// Launch grid for xcd_tile_grouped covering every tile index below max_tiles.
inline int64_t grouped_grid(int64_t max_tiles, int G) {
  const int64_t q = 8 * static_cast<int64_t>(G);
  return ((max_tiles + q - 1) / q) * q;
}

// bf16 epilogue of the expert modes, staged through LDS.  Written straight
// from the MFMA layout, every store instruction would put 16-byte pieces into
// 32 different token rows; instead each wave writes its 64 (DOWN) or 32
// (GATE_UP; G and U for GATE_UP_RAW) output features of every token row of
// the tile into its own 128-byte LDS rows (16-byte chunks XOR-swizzled by
// row), then stores whole row segments, 8 (or 4) lanes x 16 bytes per row.
// Rows past the chunk and features past nrows fall outside the buffer range
// and are dropped.  Offsets are tile-relative 32-bit values (the validator
// caps d and I so that 160 rows of either fit).
// out (and out2 for GATE_UP_RAW): bf16 [rows, out_ld], the tile's rows
// starting at t.m0; features at or past nrows are not stored.
template <int MODE, int NBR>
__device__ __forceinline__ void stage_epilogue(void *out, void *out2, int out_ld, int nrows,
                                               const TileLoc &t, const floatx16 (&acc)[2][NBR],
                                               char *st, int featbase, int r, int h, int lane) {
  // ---- registers -> LDS
#pragma unroll
  for (int nb = 0; nb < NBR; ++nb) {
    const int col = nb * 32 + r;
    char *row = st + col * 128;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      if (MODE == MODE_DOWN) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int c = a * 4 + gi;
          const floatx16 &v = acc[a][nb];
          *reinterpret_cast<uint2 *>(row + ((c ^ (col & 7)) << 4) + h * 8) =
              make_uint2(pack_bf16x2(v[gi * 4 + 0], v[gi * 4 + 1]),
                         pack_bf16x2(v[gi * 4 + 2], v[gi * 4 + 3]));
        }
      } else if (MODE == MODE_GATE_UP) {
        const floatx16 &ga = acc[0][nb];
        const floatx16 &ua = acc[1][nb];
        *reinterpret_cast<uint2 *>(row + ((gi ^ (col & 7)) << 4) + h * 8) =
            make_uint2(pack_bf16x2(silu_mul(ga[gi * 4 + 0], ua[gi * 4 + 0]),
                                   silu_mul(ga[gi * 4 + 1], ua[gi * 4 + 1])),
                       pack_bf16x2(silu_mul(ga[gi * 4 + 2], ua[gi * 4 + 2]),
                                   silu_mul(ga[gi * 4 + 3], ua[gi * 4 + 3])));
      } else {  // GATE_UP_RAW: G in chunks 0..3, U in chunks 4..7
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int c = a * 4 + gi;
          const floatx16 &v = acc[a][nb];
          *reinterpret_cast<uint2 *>(row + ((c ^ (col & 7)) << 4) + h * 8) =
              make_uint2(pack_bf16x2(v[gi * 4 + 0], v[gi * 4 + 1]),
                         pack_bf16x2(v[gi * 4 + 2], v[gi * 4 + 3]));
        }
      }
    }
  }
  // ---- LDS -> HBM, whole row segments
  const uint32_t rowb = static_cast<uint32_t>(out_ld) * 2;
  const uint32_t tbytes = static_cast<uint32_t>(t.mcount) * rowb;
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(static_cast<bf16_t *>(out) + static_cast<int64_t>(t.m0) * out_ld, tbytes);
  if (MODE == MODE_GATE_UP) {
    // 64 bytes per row: 4 lanes per row, 16 rows per instruction
    const int c = lane & 3;
    const int f0 = featbase + c * 8;
    const uint32_t fo = f0 < nrows ? static_cast<uint32_t>(f0) * 2 : kOOB;
#pragma unroll
    for (int i = 0; i < 2 * NBR; ++i) {
      const int row = i * 16 + (lane >> 2);
      const uint4 v = *reinterpret_cast<const uint4 *>(st + row * 128 + ((c ^ (row & 7)) << 4));
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, ro,
                                             static_cast<int>(row * rowb + fo), 0, kStreamOnce);
    }
  } else {
    // 128 bytes per row: 8 lanes per row, 8 rows per instruction
    const int c = lane & 7;
    const int f0 = featbase + (MODE == MODE_DOWN ? c : (c & 3)) * 8;
    const uint32_t fo = f0 < nrows ? static_cast<uint32_t>(f0) * 2 : kOOB;
    __amdgpu_buffer_rsrc_t ru = ro;
    if (MODE == MODE_GATE_UP_RAW)
      ru = make_rsrc(static_cast<bf16_t *>(out2) + static_cast<int64_t>(t.m0) * out_ld, tbytes);
#pragma unroll
    for (int i = 0; i < 4 * NBR; ++i) {
      const int row = i * 8 + (lane >> 3);
      const uint4 v = *reinterpret_cast<const uint4 *>(st + row * 128 + ((c ^ (row & 7)) << 4));
      const u32x4 d = u32x4{v.x, v.y, v.z, v.w};
      const uint32_t o = row * rowb + fo;
      if (MODE == MODE_DOWN) {
        __builtin_amdgcn_raw_buffer_store_b128(d, ro, static_cast<int>(o), 0, kStreamOnce);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(d, ro, static_cast<int>(c < 4 ? o : kOOB), 0,
                                               kStreamOnce);
        __builtin_amdgcn_raw_buffer_store_b128(d, ru, static_cast<int>(c < 4 ? kOOB : o), 0,
                                               kStreamOnce);
      }
    }
  }
}

}  // namespace moezc
