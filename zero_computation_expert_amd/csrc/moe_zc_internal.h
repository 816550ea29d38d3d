// moe_zc_internal.h -- device helpers and launcher declarations shared by the
// HIP translation units of the MoE forward library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "moe_zc.h"

namespace moezc {

constexpr int kWave = 64;
constexpr int kTokPerBlk = 16;  // tokens per top-k / permutation block (one wave each in top-k)
constexpr int kMaxE = 2048;     // experts the top-k kernel holds in registers
constexpr int kMaxK = 64;       // slots per token (one lane per slot)
constexpr int kMaxKb8 = 96;    // FP8 path: 128-wide K blocks per row (d, I <= 12288)
constexpr int kMaxWidth = 1 << 22;  // d and I (expert GEMM epilogues use tile-relative 32-bit offsets)
// Experts with at least kHotRows permuted rows (more than one 160-row chunk
// holds) are chunked kHotMT rows at a time and run on the hot-expert tile of
// the bf16 8-wave GEMM (256 weight rows x 256 tokens); the others keep the
// plan's chunk height.  Thresholds of 161, 320, 512 and 1024 rows measured
// within 0.5% of each other on the small and skewed workloads; 161 also
// streams the weights of prod's few 161-165-row experts once instead of
// twice (prod DOWN -3%).
constexpr int kHotMT = 256;
constexpr int kHotRows = 161;

// bfloat16 is carried as its 16-bit pattern.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bfloat16, rounded to nearest even by the gfx950 conversion
// instruction (v_cvt_pk_bf16_f32; NaN stays NaN).  pack_bf16x2 converts two
// values into one 32-bit word, lo in the low half.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_hw v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return static_cast<bf16_t>(pack_bf16x2(f, 0.0f));
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <>
struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t *p, int64_t i) {
    return bf16_to_f32(p[i]);
  }
  static __device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Wave reductions by DPP, the result returned to every lane: combines with
// row_shr 1, 2, 4 and 8 give prefix results within each row of 16 lanes,
// then the gfx9 row broadcasts (lane 15 of each row into the next row, lane
// 31 into rows 2 and 3) leave the wave's total in lane 63.  A lane whose DPP
// source lies outside its row, or whose row the row mask leaves out, combines
// with ZERO (max of unsigned values, sums) or with itself (float maximum).
template <int CTRL, int ROW_MASK, bool ZERO>
__device__ __forceinline__ uint32_t dpp_src(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      ZERO ? 0 : static_cast<int>(v), static_cast<int>(v), CTRL, ROW_MASK, 0xF, ZERO));
}

template <bool ZERO, typename Op>
__device__ __forceinline__ uint32_t wave_reduce_dpp(uint32_t v, Op op) {
  v = op(v, dpp_src<0x111, 0xF, ZERO>(v));  // row_shr:1
  v = op(v, dpp_src<0x112, 0xF, ZERO>(v));  // row_shr:2
  v = op(v, dpp_src<0x114, 0xF, ZERO>(v));  // row_shr:4
  v = op(v, dpp_src<0x118, 0xF, ZERO>(v));  // row_shr:8
  v = op(v, dpp_src<0x142, 0xA, ZERO>(v));  // row_bcast:15
  v = op(v, dpp_src<0x143, 0xC, ZERO>(v));  // row_bcast:31
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_dpp<true>(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  return __uint_as_float(wave_reduce_dpp<false>(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  return __uint_as_float(wave_reduce_dpp<true>(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

// Router GEMM partition (host side, a pure function of the sizes so that the
// workspace query and the launch agree).  Token chunks of 32*nb rows (128
// from 512 tokens up; 32 below, so that a decode-sized batch still spreads
// over many tiles: 128 tokens with 768 experts give 12 tiles per K slice
// instead of 3, router 28 -> 14 us), 256 expert rows per workgroup; when
// that leaves the 256 CUs short of work
// (decode-sized batches, few experts), the K range is split into `split`
// slices of `kslice` elements (whole 128-byte steps, at least two per slice)
// whose fp32 partial logits are summed in slice order (at most kMaxSplit
// slices), by the top-k kernel or, for few tokens, by a slice-sum kernel
// spread over the chip just before it.
constexpr int kMaxSplit = 16;
struct RouterSplit {
  int nb, split, kslice;
};
inline RouterSplit router_split(int64_t T, int d, int E, int dtype) {
  const int kc = dtype == MOE_ZC_BF16 ? 64 : 32;  // K elements per 128-byte step
  RouterSplit r;
  r.nb = T >= 512 ? 4 : 1;
  const int64_t chunks = (T + 32 * r.nb - 1) / (32 * r.nb);
  const int64_t tiles = std::max<int64_t>(1, chunks * ((E + 255) / 256));
  const int nks = (d + kc - 1) / kc;
  int64_t want = std::min<int64_t>(std::min<int64_t>(256 / tiles, nks / 2), kMaxSplit);
  want = std::max<int64_t>(want, 1);
  const int steps = static_cast<int>((nks + want - 1) / want);
  r.kslice = steps * kc;
  r.split = (d + r.kslice - 1) / r.kslice;
  return r;
}

// ---- launchers (host side), one per stage ------------------------------
struct Plan;  // defined in moe_zc.cpp

hipError_t launch_router_gemm(const Plan &p, hipStream_t s);
hipError_t launch_topk(const Plan &p, hipStream_t s);
hipError_t launch_scan(const Plan &p, hipStream_t s);
hipError_t launch_permute(const Plan &p, hipStream_t s);
hipError_t launch_gate_up(const Plan &p, hipStream_t s);
hipError_t launch_down(const Plan &p, hipStream_t s);
hipError_t launch_combine(const Plan &p, hipStream_t s);
hipError_t launch_zero_counts(const Plan &p, hipStream_t s);
hipError_t launch_quant_x(const Plan &p, hipStream_t s);
hipError_t launch_gate_up8(const Plan &p, hipStream_t s);
hipError_t launch_down8(const Plan &p, hipStream_t s);
hipError_t launch_dense_route(const Plan &p, hipStream_t s);  // dense FFN as one expert
// zero-padded copies (pad.hip): dst [nmat, rows_p, cols_p] <- src [nmat, rows,
// cols]; dst [rows, cols] <- the first cols columns of src [rows, cols_p];
// es = element bytes (2 or 4)
hipError_t launch_pad(const void *src, int64_t nmat, int rows, int cols, void *dst, int rows_p,
                      int cols_p, int es, hipStream_t s);
hipError_t launch_unpad(const void *src, int64_t rows, int cols_p, void *dst, int cols, int es,
                        hipStream_t s);
// backward
hipError_t launch_bwd_route(const Plan &p, hipStream_t s);      // idx -> counts, permutation
hipError_t launch_bwd_gather(const Plan &p, hipStream_t s);     // x and gate*dout rows, permuted
hipError_t launch_gate_up_raw(const Plan &p, hipStream_t s);    // G, U
hipError_t launch_dgrad_v(const Plan &p, hipStream_t s);        // dG, dU, H, dgate partials
hipError_t launch_router_bwd(const Plan &p, hipStream_t s);     // dl
hipError_t launch_wgrad_down(const Plan &p, hipStream_t s);
hipError_t launch_wgrad_gate_up(const Plan &p, hipStream_t s);
hipError_t launch_dgrad_x(const Plan &p, hipStream_t s);        // permuted dx rows
hipError_t launch_dgrad_router(const Plan &p, hipStream_t s);   // router part of dx
hipError_t launch_dx_gather(const Plan &p, hipStream_t s);      // dx
hipError_t launch_wgrad_router(const Plan &p, hipStream_t s);

// Everything one forward call needs, resolved on the host.
struct Plan {
  // sizes
  int64_t T;
  int d, I, N, Z, E, k;
  int dtype;  // moe_zc_dtype
  int nblk;   // ceil(T / kTokPerBlk)
  int64_t pmax;  // T * min(k, N): upper bound of (token, FFN expert) pairs
  int nbmax;  // 32-token column blocks per GEMM chunk (1, 4 or 5)
  int hot_rows;  // experts with at least this many rows get kHotMT-row chunks (0: none)
  float routed_scale;  // gate = routed_scale * p (1 for the dense FFN)
  RouterSplit rs;  // router GEMM partition
  // caller tensors
  const void *x, *w_router, *w_gate, *w_up, *w_down;
  const float *bias;
  void *out;
  // FP8 experts (moe_zc_forward_fp8): weights are E4M3 bytes, with E8M0
  // exponents per [128,128] block
  bool fp8;
  const uint8_t *s_gate, *s_up, *s_down;
  int32_t *counts;
  int32_t *idx;   // caller's or workspace
  float *gate;    // caller's or workspace
  // workspace
  float *logits;        // [rs.split, T, E] partial router logits (one slice of K each)
  int32_t *blockhist;   // [nblk, E]: per-block counts, then exclusive prefixes
  int32_t *offs;        // [N + 1] row offset of each FFN expert in permuted order
  int32_t *chunk_off;   // [N + 1] exclusive prefix of GEMM chunks per expert
  int32_t *meta;        // [0] total chunks, [1] total pairs P
  int32_t *rowmap;      // [T, k] permuted row of slot (t, j), -1 for zero experts
  int32_t *tok;         // [pmax] token of each permuted row
  void *h;              // [pmax, I] SwiGLU activations (FP8 path: E4M3 bytes)
  void *y;              // [pmax, d] expert outputs
  void *qx;             // FP8 path: [T, d] E4M3 x
  uint8_t *sx;          // FP8 path: [T, d/128] exponents of x
  uint8_t *sxp;         // FP8 path: [d/128, pmax] the same, rows in permuted order,
                        // K-block-major (a step's exponents of a tile's rows are contiguous)
  uint8_t *sh;          // FP8 path: [I/128, pmax] exponents of H, K-block-major
  // backward (moe_zc_backward); idx then holds the sanitized routing
  const void *dout;     // [T, d] output gradient
  void *dx;             // [T, d] input gradient
  float *dw_router, *dw_gate, *dw_up, *dw_down;  // fp32, accumulated into
  const int32_t *idx_in;  // the caller's routing
  float *gate_perm;     // [pmax] gate of each permuted row
  void *bG, *bU, *bH;   // [pmax, I] G and U (then dG and dU), H
  float *dpart;         // [ceil(I/256), pmax] partial dgate sums
  void *dl;             // [T, ldl] router-logit gradient, bf16 (zero padded)
  int ldl;              // E rounded up to 8
  void *xp, *dyp, *dxp; // [pmax, d] x, gate*dout and dx rows in permuted order
  float *dxr;           // [T, d] router part of dx
};

}  // namespace moezc
