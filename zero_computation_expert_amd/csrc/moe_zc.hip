// moe_zc.hip -- host side of the C ABI declared in include/moe_zc.h:
// argument validation, workspace layout and the ordered launch of the
// forward's kernels on the caller's stream (no allocation, no sync).
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "moe_zc_internal.h"

namespace moezc {

static inline size_t align_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

static inline int round8(int v) { return (v + 7) & ~7; }

// pad_ok: the bf16 / fp32 forward, which takes any d, I >= 1 (widths that are
// not multiples of 8 run on zero-padded copies, pad.hip); the other entry
// points need multiples of 8.  Size limits apply to the padded widths.
static bool dims_ok(const moe_zc_dims *dm, int *status, bool pad_ok = false) {
  if (dm == nullptr) {
    *status = MOE_ZC_EINVAL;
    return false;
  }
  if (dm->dtype != MOE_ZC_F32 && dm->dtype != MOE_ZC_BF16) {
    *status = MOE_ZC_EDTYPE;
    return false;
  }
  const int64_t E = static_cast<int64_t>(dm->N) + dm->Z;
  if (dm->T < 0 || dm->N < 0 || dm->Z < 0 || E < 1 || E > kMaxE || dm->k < 1 || dm->k > E ||
      dm->k > kMaxK || dm->d < 1 || (dm->N > 0 && dm->I < 1) ||
      dm->T * static_cast<int64_t>(dm->k) >= (int64_t(1) << 31) ||
      !(dm->routed_scale > 0.0f && dm->routed_scale <= 3.4028234e38f)) {
    *status = MOE_ZC_EINVAL;
    return false;
  }
  // The expert GEMMs address x and one expert matrix through 32-bit buffer
  // offsets: both must stay below 2 GiB.
  const int64_t es = dm->dtype == MOE_ZC_BF16 ? 2 : 4;
  if (dm->d > kMaxWidth || (dm->N > 0 && dm->I > kMaxWidth)) {
    *status = MOE_ZC_EINVAL;
    return false;
  }
  const int64_t d8 = round8(dm->d), I8 = dm->N > 0 ? round8(dm->I) : 0;
  if (dm->T * d8 * es >= (int64_t(1) << 31) || I8 * d8 * es >= (int64_t(1) << 31)) {
    *status = MOE_ZC_EINVAL;
    return false;
  }
  // The expert GEMM epilogues store through tile-relative 32-bit offsets
  // (up to 160 rows of d or I elements).
  if (d8 > kMaxWidth || I8 > kMaxWidth) {
    *status = MOE_ZC_EINVAL;
    return false;
  }
  if (!pad_ok && (dm->d % 8 != 0 || (dm->N > 0 && dm->I % 8 != 0))) {
    *status = MOE_ZC_EALIGN;
    return false;
  }
  *status = MOE_ZC_OK;
  return true;
}

// Workspace layout; returns the total size.  With base == nullptr only sizes.
// fp8: E4M3 x (and its exponents) and E4M3 H (and its exponents) instead of
// an H in the dims' dtype; Y is bfloat16 either way.
static size_t layout(const moe_zc_dims *dm, char *base, Plan *p, bool fp8 = false) {
  const int64_t T = dm->T;
  const int E = dm->N + dm->Z;
  const int64_t nblk = (T + kTokPerBlk - 1) / kTokPerBlk;
  const int64_t pmax = T * std::min(dm->k, dm->N);
  const size_t es = dm->dtype == MOE_ZC_BF16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *ptr = base ? base + off : nullptr;
    off = align_up(off + bytes);
    return ptr;
  };
  const RouterSplit rs = router_split(T, dm->d, E, dm->dtype);
  char *logits = take(static_cast<size_t>(rs.split) * T * E * 4);
  char *blockhist = take(static_cast<size_t>(nblk) * E * 4);
  char *offs = take(static_cast<size_t>(dm->N + 1) * 4);
  char *chunk_off = take(static_cast<size_t>(dm->N + 1) * 4);
  char *meta = take(64);
  char *idx = take(static_cast<size_t>(T) * dm->k * 4);
  char *gate = take(static_cast<size_t>(T) * dm->k * 4);
  char *rowmap = take(static_cast<size_t>(T) * dm->k * 4);
  char *tok = take(static_cast<size_t>(pmax) * 4);
  const int I = dm->N > 0 ? dm->I : 0;
  char *h = take(static_cast<size_t>(pmax) * I * (fp8 ? 1 : es));
  char *y = take(static_cast<size_t>(pmax) * dm->d * es);
  char *qx = fp8 ? take(static_cast<size_t>(T) * dm->d) : nullptr;
  char *sx = fp8 ? take(static_cast<size_t>(T) * (dm->d / 128)) : nullptr;
  char *sh = fp8 ? take(static_cast<size_t>(pmax) * (I / 128)) : nullptr;
  char *sxp = fp8 ? take(static_cast<size_t>(pmax) * (dm->d / 128)) : nullptr;
  if (p) {
    p->logits = reinterpret_cast<float *>(logits);
    p->blockhist = reinterpret_cast<int32_t *>(blockhist);
    p->offs = reinterpret_cast<int32_t *>(offs);
    p->chunk_off = reinterpret_cast<int32_t *>(chunk_off);
    p->meta = reinterpret_cast<int32_t *>(meta);
    p->idx = reinterpret_cast<int32_t *>(idx);
    p->gate = reinterpret_cast<float *>(gate);
    p->rowmap = reinterpret_cast<int32_t *>(rowmap);
    p->tok = reinterpret_cast<int32_t *>(tok);
    p->h = h;
    p->y = y;
    p->qx = qx;
    p->sx = reinterpret_cast<uint8_t *>(sx);
    p->sh = reinterpret_cast<uint8_t *>(sh);
    p->sxp = reinterpret_cast<uint8_t *>(sxp);
  }
  return off;
}

// Widths that are not multiples of 8: the forward runs on the dims with d
// and I rounded up (padded) and zero-padded copies of its operands.
static bool needs_pad(const moe_zc_dims *dm) {
  return dm->d % 8 != 0 || (dm->N > 0 && dm->I % 8 != 0);
}

static moe_zc_dims padded(const moe_zc_dims *dm) {
  moe_zc_dims q = *dm;
  q.d = round8(dm->d);
  if (dm->N > 0) q.I = round8(dm->I);
  return q;
}

struct PadBufs {
  char *x, *wr, *wg, *wu, *wd, *out;  // padded x, W_router, W_gate, W_up, W_down, output
};

// Workspace of the padded copies (placed before the forward's own layout);
// 0 when d and I are multiples of 8.  With base == nullptr only sizes.
static size_t pad_layout(const moe_zc_dims *dm, char *base, PadBufs *b) {
  if (!needs_pad(dm)) return 0;
  const moe_zc_dims q = padded(dm);
  const size_t es = dm->dtype == MOE_ZC_BF16 ? 2 : 4;
  const size_t T = static_cast<size_t>(dm->T), E = static_cast<size_t>(dm->N + dm->Z);
  const size_t N = static_cast<size_t>(dm->N), d8 = static_cast<size_t>(q.d);
  const size_t I8 = dm->N > 0 ? static_cast<size_t>(q.I) : 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *ptr = base ? base + off : nullptr;
    off = align_up(off + bytes);
    return ptr;
  };
  char *x = take(T * d8 * es);
  char *wr = take(E * d8 * es);
  char *wg = take(N * I8 * d8 * es);
  char *wu = take(N * I8 * d8 * es);
  char *wd = take(N * d8 * I8 * es);
  char *out = take(T * d8 * es);
  if (b) *b = PadBufs{x, wr, wg, wu, wd, out};
  return off;
}

// Workspace of the bf16 / fp32 forward.
static size_t forward_bytes(const moe_zc_dims *dm) {
  const moe_zc_dims q = padded(dm);
  return pad_layout(dm, nullptr, nullptr) + layout(&q, nullptr, nullptr);
}

static bool aligned(const void *ptr, size_t a) {
  return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0;
}

static bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace moezc

struct moe_zc_timer {
  int max_calls;
  int ncalls;
  hipEvent_t *ev;  // [max_calls][MOE_ZC_MAX_STAGES + 1]
  int *nst;        // [max_calls] stages recorded by each call
};

using namespace moezc;

// Exponent arrays of FP8 expert weights (nullptr: the bf16 / fp32 path).
struct Fp8Scales {
  const uint8_t *gate, *up, *down;
};

static bool fp8_dims_ok(const moe_zc_dims *dm, int *status) {
  if (!dims_ok(dm, status)) return false;
  if (dm->dtype != MOE_ZC_BF16) {
    *status = MOE_ZC_EDTYPE;
    return false;
  }
  if (dm->d % 128 != 0 || (dm->N > 0 && dm->I % 128 != 0)) {
    *status = MOE_ZC_EALIGN;
    return false;
  }
  if (dm->d / 128 > kMaxKb8 || (dm->N > 0 && dm->I / 128 > kMaxKb8)) {
    *status = MOE_ZC_EINVAL;
    return false;
  }
  // the K-block-major exponent matrices of the permuted rows are addressed
  // through 32-bit offsets
  const int64_t pmax = dm->T * std::min(dm->k, dm->N);
  if (pmax * (std::max(dm->d, dm->N > 0 ? dm->I : 0) / 128) >= (int64_t(1) << 31)) {
    *status = MOE_ZC_EINVAL;
    return false;
  }
  return true;
}

static int forward_impl(const moe_zc_dims *dm, const void *x, const void *w_router,
                        const float *bias, const void *w_gate, const void *w_up,
                        const void *w_down, void *out, int32_t *counts, int32_t *topk_idx,
                        float *topk_gate, void *workspace, size_t workspace_bytes, void *stream,
                        moe_zc_timer *timer, const Fp8Scales *f8 = nullptr,
                        bool launch = true) {
  int st;
  if (!(f8 ? fp8_dims_ok(dm, &st) : dims_ok(dm, &st, true))) return st;
  if (f8 && dm->T > 0 && dm->N > 0 && (!f8->gate || !f8->up || !f8->down)) return MOE_ZC_EINVAL;
  // widths that are not multiples of 8 (never FP8): the kernels run on q
  const bool pad = needs_pad(dm);
  const moe_zc_dims q = padded(dm);
  const size_t padb = pad_layout(dm, nullptr, nullptr);
  const int64_t T = dm->T;
  const size_t es = dm->dtype == MOE_ZC_BF16 ? 2 : 4;
  const size_t xbytes = static_cast<size_t>(T) * dm->d * es;
  if (counts == nullptr) return MOE_ZC_EINVAL;
  if (T > 0) {
    if (!x || !w_router || !bias || !out) return MOE_ZC_EINVAL;
    if (dm->N > 0 && (!w_gate || !w_up || !w_down)) return MOE_ZC_EINVAL;
    if (overlap(x, xbytes, out, xbytes)) return MOE_ZC_EINVAL;
  }
  const void *p16[] = {x, w_router, w_gate, w_up, w_down, out};
  for (const void *ptr : p16)
    if (ptr && !aligned(ptr, 16)) return MOE_ZC_EALIGN;
  const void *p4[] = {bias, counts, topk_idx, topk_gate};
  for (const void *ptr : p4)
    if (ptr && !aligned(ptr, 4)) return MOE_ZC_EALIGN;
  const size_t need = padb + layout(&q, nullptr, nullptr, f8 != nullptr);
  if (T > 0) {
    if (workspace == nullptr || workspace_bytes < need) return MOE_ZC_ENOSPC;
    if (!aligned(workspace, 256)) return MOE_ZC_EALIGN;
  }
  if (timer && timer->ncalls >= timer->max_calls) return MOE_ZC_ENOSPC;
  if (!launch) return MOE_ZC_OK;  // validation only

  Plan p = {};
  p.T = T;
  p.d = q.d;
  p.I = dm->N > 0 ? q.I : 0;
  p.N = dm->N;
  p.Z = dm->Z;
  p.E = dm->N + dm->Z;
  p.k = dm->k;
  p.routed_scale = dm->routed_scale;
  p.dtype = dm->dtype;
  p.nblk = static_cast<int>((T + kTokPerBlk - 1) / kTokPerBlk);
  p.pmax = T * std::min(dm->k, dm->N);
  // Chunk height of the expert GEMMs (32-token blocks): 160 token rows (the
  // tallest chunk whose three token tiles fit in LDS beside the weight
  // slots) when experts receive many rows on average, 128 in between, 32
  // when they receive few (decode-shaped: weight streaming with few rows
  // per expert wants occupancy, not tall tiles).
  const int64_t avg_rows = dm->N > 0 ? p.pmax / dm->N : 0;
  p.nbmax = avg_rows >= 96 ? 5 : (avg_rows >= 24 ? 4 : 1);
  p.fp8 = f8 != nullptr;
  // hot-expert tiles: bf16 experts on the 8-wave kernel (160-row chunks)
  p.hot_rows = p.dtype == MOE_ZC_BF16 && !p.fp8 && p.nbmax == 5 ? kHotRows : 0;
  if (f8) {
    p.s_gate = f8->gate;
    p.s_up = f8->up;
    p.s_down = f8->down;
  }
  p.rs = router_split(T, p.d, p.E, p.dtype);
  PadBufs pb = {};
  pad_layout(dm, static_cast<char *>(workspace), &pb);
  p.x = pad ? pb.x : x;
  p.w_router = pad ? pb.wr : w_router;
  p.w_gate = pad ? pb.wg : w_gate;
  p.w_up = pad ? pb.wu : w_up;
  p.w_down = pad ? pb.wd : w_down;
  p.bias = bias;
  p.out = pad ? pb.out : out;
  p.counts = counts;
  layout(&q, static_cast<char *>(workspace) + padb, &p, f8 != nullptr);
  if (topk_idx) p.idx = topk_idx;
  if (topk_gate) p.gate = topk_gate;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t *ev = timer ? timer->ev + static_cast<size_t>(timer->ncalls) * (MOE_ZC_MAX_STAGES + 1)
                         : nullptr;
  if (timer) timer->nst[timer->ncalls] = MOE_ZC_NSTAGES;
  auto mark = [&](int i) -> bool {
    return ev == nullptr || hipEventRecord(ev[i], s) == hipSuccess;
  };

  if (T == 0) {
    if (launch_zero_counts(p, s) != hipSuccess) return MOE_ZC_EHIP;
    if (timer) {
      for (int i = 0; i <= MOE_ZC_NSTAGES; ++i)
        if (!mark(i)) return MOE_ZC_EHIP;
      timer->ncalls++;
    }
    return MOE_ZC_OK;
  }

  typedef hipError_t (*Launch)(const Plan &, hipStream_t);
  const Launch stages[MOE_ZC_NSTAGES] = {launch_router_gemm, launch_topk, launch_scan,
                                         launch_permute,     launch_gate_up, launch_down,
                                         launch_combine};
  // the FP8 path quantizes x after the permutation (same timer stage) and
  // runs the FP8 expert GEMMs
  const Launch stages8[MOE_ZC_NSTAGES] = {
      launch_router_gemm, launch_topk, launch_scan,
      [](const Plan &q, hipStream_t ss) {
        const hipError_t e = launch_permute(q, ss);
        return (e != hipSuccess || q.N == 0) ? e : launch_quant_x(q, ss);
      },
      launch_gate_up8, launch_down8, launch_combine};
  const Launch *run = p.fp8 ? stages8 : stages;
  if (pad) {  // zero-padded operands (outside the timed stages)
    const int es_i = static_cast<int>(es), E = dm->N + dm->Z;
    if (launch_pad(x, 1, static_cast<int>(T), dm->d, pb.x, static_cast<int>(T), q.d, es_i, s) !=
            hipSuccess ||
        launch_pad(w_router, 1, E, dm->d, pb.wr, E, q.d, es_i, s) != hipSuccess)
      return MOE_ZC_EHIP;
    if (dm->N > 0 &&
        (launch_pad(w_gate, dm->N, dm->I, dm->d, pb.wg, q.I, q.d, es_i, s) != hipSuccess ||
         launch_pad(w_up, dm->N, dm->I, dm->d, pb.wu, q.I, q.d, es_i, s) != hipSuccess ||
         launch_pad(w_down, dm->N, dm->d, dm->I, pb.wd, q.d, q.I, es_i, s) != hipSuccess))
      return MOE_ZC_EHIP;
  }
  if (!mark(0)) return MOE_ZC_EHIP;
  for (int i = 0; i < MOE_ZC_NSTAGES; ++i) {
    const bool ffn = i == MOE_ZC_STAGE_GATE_UP || i == MOE_ZC_STAGE_DOWN;
    if (!(ffn && p.N == 0))
      if (run[i](p, s) != hipSuccess) return MOE_ZC_EHIP;
    if (!mark(i + 1)) return MOE_ZC_EHIP;
  }
  if (pad && launch_unpad(pb.out, T, q.d, out, dm->d, static_cast<int>(es), s) != hipSuccess)
    return MOE_ZC_EHIP;
  if (timer) timer->ncalls++;
  return MOE_ZC_OK;
}

// ---- backward -------------------------------------------------------------
// Workspace of the backward; with base == nullptr only sizes.
static size_t layout_bwd(const moe_zc_dims *dm, char *base, Plan *p) {
  const int64_t T = dm->T;
  const int E = dm->N + dm->Z;
  const int64_t nblk = (T + kTokPerBlk - 1) / kTokPerBlk;
  const int64_t pmax = T * std::min(dm->k, dm->N);
  const int I = dm->N > 0 ? dm->I : 0;
  const int ldl = (E + 7) / 8 * 8;
  const int nrbi = (I + 255) / 256;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *ptr = base ? base + off : nullptr;
    off = align_up(off + bytes);
    return ptr;
  };
  const RouterSplit rs = router_split(T, dm->d, E, MOE_ZC_BF16);
  char *logits = take(static_cast<size_t>(rs.split) * T * E * 4);
  char *blockhist = take(static_cast<size_t>(nblk) * E * 4);
  char *counts = take(static_cast<size_t>(E) * 4);
  char *offs = take(static_cast<size_t>(dm->N + 1) * 4);
  char *chunk_off = take(static_cast<size_t>(dm->N + 1) * 4);
  char *meta = take(64);
  char *idx = take(static_cast<size_t>(T) * dm->k * 4);
  char *rowmap = take(static_cast<size_t>(T) * dm->k * 4);
  char *tok = take(static_cast<size_t>(pmax) * 4);
  char *gate_perm = take(static_cast<size_t>(pmax) * 4);
  char *bG = take(static_cast<size_t>(pmax) * I * 2);
  char *bU = take(static_cast<size_t>(pmax) * I * 2);
  char *bH = take(static_cast<size_t>(pmax) * I * 2);
  char *dpart = take(static_cast<size_t>(nrbi) * pmax * 4);
  char *dl = take(static_cast<size_t>(T) * ldl * 2);
  char *xp = take(static_cast<size_t>(pmax) * dm->d * 2);
  char *dyp = take(static_cast<size_t>(pmax) * dm->d * 2);
  char *dxp = take(static_cast<size_t>(pmax) * dm->d * 2);
  char *dxr = take(static_cast<size_t>(T) * dm->d * 4);
  if (p) {
    p->rs = rs;
    p->logits = reinterpret_cast<float *>(logits);
    p->blockhist = reinterpret_cast<int32_t *>(blockhist);
    p->counts = reinterpret_cast<int32_t *>(counts);
    p->offs = reinterpret_cast<int32_t *>(offs);
    p->chunk_off = reinterpret_cast<int32_t *>(chunk_off);
    p->meta = reinterpret_cast<int32_t *>(meta);
    p->idx = reinterpret_cast<int32_t *>(idx);
    p->rowmap = reinterpret_cast<int32_t *>(rowmap);
    p->tok = reinterpret_cast<int32_t *>(tok);
    p->gate_perm = reinterpret_cast<float *>(gate_perm);
    p->bG = bG;
    p->bU = bU;
    p->bH = bH;
    p->dpart = reinterpret_cast<float *>(dpart);
    p->dl = dl;
    p->ldl = ldl;
    p->xp = xp;
    p->dyp = dyp;
    p->dxp = dxp;
    p->dxr = reinterpret_cast<float *>(dxr);
  }
  return off;
}

static bool bwd_dims_ok(const moe_zc_dims *dm, int *status) {
  if (!dims_ok(dm, status)) return false;
  if (dm->dtype != MOE_ZC_BF16) {
    *status = MOE_ZC_EDTYPE;
    return false;
  }
  // W_router, the router-logit gradient and an expert's rows of dG / dU / H
  // are addressed through 32-bit buffer offsets (x, dout and one expert
  // matrix are bounded by dims_ok)
  const int64_t E = static_cast<int64_t>(dm->N) + dm->Z;
  const int64_t lim = int64_t(1) << 31;
  // (the fp32 weight gradients of one matrix too: the wgrad epilogue reads
  // and writes them through buffer descriptors)
  if (E * dm->d * 4 >= lim || dm->T * ((E + 7) / 8 * 8) * 2 >= lim ||
      (dm->N > 0 && (dm->T * dm->I * 2 >= lim ||
                     static_cast<int64_t>(dm->d) * dm->I * 4 >= lim))) {
    *status = MOE_ZC_EINVAL;
    return false;
  }
  return true;
}

static int backward_impl(const moe_zc_dims *dm, const void *x, const void *w_router,
                         const void *w_gate, const void *w_up, const void *w_down,
                         const int32_t *topk_idx, const float *topk_gate, const void *dout,
                         void *dx, float *dw_router, float *dw_gate, float *dw_up,
                         float *dw_down, void *workspace, size_t workspace_bytes, void *stream,
                         moe_zc_timer *timer) {
  int st;
  if (!bwd_dims_ok(dm, &st)) return st;
  const int64_t T = dm->T;
  const size_t xbytes = static_cast<size_t>(T) * dm->d * 2;
  if (T > 0) {
    if (!x || !w_router || !topk_idx || !topk_gate || !dout || !dx || !dw_router)
      return MOE_ZC_EINVAL;
    if (dm->N > 0 && (!w_gate || !w_up || !w_down || !dw_gate || !dw_up || !dw_down))
      return MOE_ZC_EINVAL;
    if (overlap(dx, xbytes, x, xbytes) || overlap(dx, xbytes, dout, xbytes)) return MOE_ZC_EINVAL;
  }
  const void *p16[] = {x, w_router, w_gate, w_up, w_down, dout, dx};
  for (const void *ptr : p16)
    if (ptr && !aligned(ptr, 16)) return MOE_ZC_EALIGN;
  const void *p4[] = {topk_idx, topk_gate, dw_router, dw_gate, dw_up, dw_down};
  for (const void *ptr : p4)
    if (ptr && !aligned(ptr, 4)) return MOE_ZC_EALIGN;
  const size_t need = layout_bwd(dm, nullptr, nullptr);
  if (T > 0) {
    if (workspace == nullptr || workspace_bytes < need) return MOE_ZC_ENOSPC;
    if (!aligned(workspace, 256)) return MOE_ZC_EALIGN;
  }
  if (timer && timer->ncalls >= timer->max_calls) return MOE_ZC_ENOSPC;

  Plan p = {};
  p.T = T;
  p.d = dm->d;
  p.I = dm->N > 0 ? dm->I : 0;
  p.N = dm->N;
  p.Z = dm->Z;
  p.E = dm->N + dm->Z;
  p.k = dm->k;
  p.routed_scale = dm->routed_scale;
  p.dtype = MOE_ZC_BF16;
  p.nblk = static_cast<int>((T + kTokPerBlk - 1) / kTokPerBlk);
  p.pmax = T * std::min(dm->k, dm->N);
  const int64_t avg_rows = dm->N > 0 ? p.pmax / dm->N : 0;
  p.nbmax = avg_rows >= 96 ? 5 : (avg_rows >= 24 ? 4 : 1);
  p.x = x;
  p.w_router = w_router;
  p.w_gate = w_gate;
  p.w_up = w_up;
  p.w_down = w_down;
  p.idx_in = topk_idx;
  p.gate = const_cast<float *>(topk_gate);
  p.dout = dout;
  p.dx = dx;
  p.dw_router = dw_router;
  p.dw_gate = dw_gate;
  p.dw_up = dw_up;
  p.dw_down = dw_down;
  layout_bwd(dm, static_cast<char *>(workspace), &p);

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t *ev = timer ? timer->ev + static_cast<size_t>(timer->ncalls) * (MOE_ZC_MAX_STAGES + 1)
                         : nullptr;
  if (timer) timer->nst[timer->ncalls] = MOE_ZC_BWD_NSTAGES;
  auto mark = [&](int i) -> bool {
    return ev == nullptr || hipEventRecord(ev[i], s) == hipSuccess;
  };
  if (T == 0) {
    if (timer) {
      for (int i = 0; i <= MOE_ZC_BWD_NSTAGES; ++i)
        if (!mark(i)) return MOE_ZC_EHIP;
      timer->ncalls++;
    }
    return MOE_ZC_OK;
  }
  typedef hipError_t (*Launch)(const Plan &, hipStream_t);
  const Launch stages[MOE_ZC_BWD_NSTAGES] = {
      [](const Plan &q, hipStream_t ss) {  // routing bookkeeping, permuted rows
        hipError_t e = launch_bwd_route(q, ss);
        return (e != hipSuccess || q.N == 0) ? e : launch_bwd_gather(q, ss);
      },
      launch_router_gemm, launch_gate_up_raw, launch_dgrad_v, launch_router_bwd,
      launch_wgrad_down, launch_wgrad_gate_up, launch_dgrad_x,
      [](const Plan &q, hipStream_t ss) {  // dx: router part, then the gather
        hipError_t e = launch_dgrad_router(q, ss);
        return e != hipSuccess ? e : launch_dx_gather(q, ss);
      },
      launch_wgrad_router};
  if (!mark(0)) return MOE_ZC_EHIP;
  for (int i = 0; i < MOE_ZC_BWD_NSTAGES; ++i) {
    const bool ffn = i == MOE_ZC_BSTAGE_RECOMPUTE || i == MOE_ZC_BSTAGE_DGRAD_V ||
                     i == MOE_ZC_BSTAGE_WGRAD_DOWN || i == MOE_ZC_BSTAGE_WGRAD_GATE_UP ||
                     i == MOE_ZC_BSTAGE_DGRAD_X;
    if (!(ffn && p.N == 0))
      if (stages[i](p, s) != hipSuccess) return MOE_ZC_EHIP;
    if (!mark(i + 1)) return MOE_ZC_EHIP;
  }
  if (timer) timer->ncalls++;
  return MOE_ZC_OK;
}

// ---- dense SwiGLU FFN and the two-stream ScMoE schedule --------------------
// The dense FFN y = W2 (silu(W1 x) * (W3 x)) runs on the expert GEMM kernels
// as a single expert that every token uses (identity permutation).
static bool dense_dims_ok(int64_t T, int d, int Id) {
  const int64_t lim = int64_t(1) << 31;
  return T >= 0 && d >= 8 && Id >= 8 && d % 8 == 0 && Id % 8 == 0 && T * d * 2 < lim &&
         static_cast<int64_t>(Id) * d * 2 < lim && T < lim && d <= kMaxWidth && Id <= kMaxWidth;
}

static size_t layout_dense(int64_t T, int Id, char *base, Plan *p) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *ptr = base ? base + off : nullptr;
    off = align_up(off + bytes);
    return ptr;
  };
  char *tok = take(static_cast<size_t>(T) * 4);
  char *offs = take(8);
  char *chunk_off = take(8);
  char *meta = take(64);
  char *h = take(static_cast<size_t>(T) * Id * 2);
  if (p) {
    p->tok = reinterpret_cast<int32_t *>(tok);
    p->offs = reinterpret_cast<int32_t *>(offs);
    p->chunk_off = reinterpret_cast<int32_t *>(chunk_off);
    p->meta = reinterpret_cast<int32_t *>(meta);
    p->h = h;
  }
  return off;
}

static int dense_impl(int64_t T, int d, int Id, const void *x, const void *w1, const void *w3,
                      const void *w2, void *out, void *workspace, size_t workspace_bytes,
                      hipStream_t s, bool launch) {
  if (!dense_dims_ok(T, d, Id)) return (d % 8 || Id % 8) ? MOE_ZC_EALIGN : MOE_ZC_EINVAL;
  if (T == 0) return MOE_ZC_OK;
  const size_t xbytes = static_cast<size_t>(T) * d * 2;
  if (!x || !w1 || !w3 || !w2 || !out) return MOE_ZC_EINVAL;
  if (overlap(x, xbytes, out, xbytes)) return MOE_ZC_EINVAL;
  const void *p16[] = {x, w1, w3, w2, out};
  for (const void *ptr : p16)
    if (!aligned(ptr, 16)) return MOE_ZC_EALIGN;
  if (workspace == nullptr || workspace_bytes < layout_dense(T, Id, nullptr, nullptr))
    return MOE_ZC_ENOSPC;
  if (!aligned(workspace, 256)) return MOE_ZC_EALIGN;
  if (!launch) return MOE_ZC_OK;
  Plan p = {};
  p.T = T;
  p.d = d;
  p.I = Id;
  p.N = 1;
  p.E = 1;
  p.k = 1;
  p.routed_scale = 1.0f;
  p.dtype = MOE_ZC_BF16;
  p.pmax = T;
  p.nbmax = T >= 96 ? 5 : (T >= 24 ? 4 : 1);
  p.hot_rows = p.nbmax == 5 ? kHotRows : 0;
  p.x = x;
  p.w_gate = w1;
  p.w_up = w3;
  p.w_down = w2;
  layout_dense(T, Id, static_cast<char *>(workspace), &p);
  p.y = out;  // the identity permutation writes token rows in place
  if (launch_dense_route(p, s) != hipSuccess || launch_gate_up(p, s) != hipSuccess ||
      launch_down(p, s) != hipSuccess)
    return MOE_ZC_EHIP;
  return MOE_ZC_OK;
}

static int64_t chunk_rows(int64_t T, int nchunks) { return (T + nchunks - 1) / nchunks; }

// ---- the workspace of moe_zc_forward_noalloc --------------------------------
// A fixed array in this translation unit's device image; every GPU that runs
// the library gets its own copy at its own address.  In host code the name
// `noalloc_scratch` is only a stand-in for the symbol: its device address is
// looked up once per device (hipGetSymbolAddress with that device current)
// and only that address is ever handed to kernels.
static __device__ __align__(256) char noalloc_scratch[MOE_ZC_SCRATCH_BYTES];

namespace moezc {
constexpr int kMaxDevices = 64;
static std::once_flag g_scratch_once[kMaxDevices];
static void *g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (nullptr on failure).
static void *scratch_of(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return;
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(noalloc_scratch)) == hipSuccess) g_scratch_ptr[dev] = ptr;
    if (cur != dev) (void)hipSetDevice(cur);
  });
  return g_scratch_ptr[dev];
}
}  // namespace moezc

extern "C" {

int moe_zc_forward_noalloc(const moe_zc_dims *dims, const void *x, const void *W_router,
                           const float *bias, const void *W_gate, const void *W_up,
                           const void *W_down, void *out, int32_t *counts, int32_t *topk_idx,
                           float *topk_gate, void *stream) {
  int st;
  if (!dims_ok(dims, &st, true)) return st;
  const size_t need = forward_bytes(dims);
  if (need > MOE_ZC_SCRATCH_BYTES) return MOE_ZC_ESCRATCH;
  // every other argument, before the device is touched (a stand-in address
  // with the scratch array's alignment takes the workspace's place)
  st = forward_impl(dims, x, W_router, bias, W_gate, W_up, W_down, out, counts, topk_idx,
                    topk_gate, reinterpret_cast<void *>(uintptr_t(256)), MOE_ZC_SCRATCH_BYTES,
                    stream, nullptr, nullptr, false);
  if (st != MOE_ZC_OK) return st;
  hipDevice_t dev = -1;
  if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess) return MOE_ZC_EHIP;
  void *ws = scratch_of(static_cast<int>(dev));
  if (ws == nullptr) return MOE_ZC_EHIP;
  return forward_impl(dims, x, W_router, bias, W_gate, W_up, W_down, out, counts, topk_idx,
                      topk_gate, ws, MOE_ZC_SCRATCH_BYTES, stream, nullptr);
}

size_t moe_zc_workspace_bytes_fp8(const moe_zc_dims *dims) {
  int st;
  if (!fp8_dims_ok(dims, &st)) return 0;
  return layout(dims, nullptr, nullptr, true);
}

int moe_zc_forward_fp8(const moe_zc_dims *dims, const void *x, const void *W_router,
                       const float *bias, const uint8_t *W_gate, const uint8_t *W_gate_exp,
                       const uint8_t *W_up, const uint8_t *W_up_exp, const uint8_t *W_down,
                       const uint8_t *W_down_exp, void *out, int32_t *counts, int32_t *topk_idx,
                       float *topk_gate, void *workspace, size_t workspace_bytes, void *stream,
                       moe_zc_timer *timer) {
  const Fp8Scales f8 = {W_gate_exp, W_up_exp, W_down_exp};
  return forward_impl(dims, x, W_router, bias, W_gate, W_up, W_down, out, counts, topk_idx,
                      topk_gate, workspace, workspace_bytes, stream, timer, &f8);
}

size_t moe_zc_workspace_bytes(const moe_zc_dims *dims) {
  int st;
  if (!dims_ok(dims, &st, true)) return 0;
  return forward_bytes(dims);
}

int moe_zc_forward(const moe_zc_dims *dims, const void *x, const void *W_router,
                   const float *bias, const void *W_gate, const void *W_up, const void *W_down,
                   void *out, int32_t *counts, int32_t *topk_idx, float *topk_gate,
                   void *workspace, size_t workspace_bytes, void *stream) {
  return forward_impl(dims, x, W_router, bias, W_gate, W_up, W_down, out, counts, topk_idx,
                      topk_gate, workspace, workspace_bytes, stream, nullptr);
}

int moe_zc_forward_timed(const moe_zc_dims *dims, const void *x, const void *W_router,
                         const float *bias, const void *W_gate, const void *W_up,
                         const void *W_down, void *out, int32_t *counts, int32_t *topk_idx,
                         float *topk_gate, void *workspace, size_t workspace_bytes, void *stream,
                         moe_zc_timer *timer) {
  if (timer == nullptr) return MOE_ZC_EINVAL;
  return forward_impl(dims, x, W_router, bias, W_gate, W_up, W_down, out, counts, topk_idx,
                      topk_gate, workspace, workspace_bytes, stream, timer);
}

size_t moe_zc_backward_workspace_bytes(const moe_zc_dims *dims) {
  int st;
  if (!bwd_dims_ok(dims, &st)) return 0;
  return layout_bwd(dims, nullptr, nullptr);
}

int moe_zc_backward(const moe_zc_dims *dims, const void *x, const void *W_router,
                    const void *W_gate, const void *W_up, const void *W_down,
                    const int32_t *topk_idx, const float *topk_gate, const void *dout, void *dx,
                    float *dW_router, float *dW_gate, float *dW_up, float *dW_down,
                    void *workspace, size_t workspace_bytes, void *stream, moe_zc_timer *timer) {
  return backward_impl(dims, x, W_router, W_gate, W_up, W_down, topk_idx, topk_gate, dout, dx,
                       dW_router, dW_gate, dW_up, dW_down, workspace, workspace_bytes, stream,
                       timer);
}

size_t moe_zc_dense_workspace_bytes(int64_t T, int32_t d, int32_t I_dense) {
  if (!dense_dims_ok(T, d, I_dense)) return 0;
  return layout_dense(T, I_dense, nullptr, nullptr);
}

int moe_zc_dense_ffn(int64_t T, int32_t d, int32_t I_dense, const void *x, const void *W1,
                     const void *W3, const void *W2, void *out, void *workspace,
                     size_t workspace_bytes, void *stream) {
  return dense_impl(T, d, I_dense, x, W1, W3, W2, out, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream), true);
}

int moe_zc_scmoe_workspace_bytes(const moe_zc_dims *dims, int32_t I_dense, int32_t nchunks,
                                 size_t *ws_moe, size_t *ws_dense) {
  int st;
  if (!ws_moe || !ws_dense || nchunks < 1 || nchunks > 2) return MOE_ZC_EINVAL;
  if (!dims_ok(dims, &st)) return st;
  if (dims->dtype != MOE_ZC_BF16) return MOE_ZC_EDTYPE;
  if (!dense_dims_ok(dims->T, dims->d, I_dense)) return MOE_ZC_EINVAL;
  moe_zc_dims c = *dims;
  c.T = chunk_rows(dims->T, nchunks);
  *ws_moe = layout(&c, nullptr, nullptr);
  *ws_dense = layout_dense(dims->T, I_dense, nullptr, nullptr);
  return MOE_ZC_OK;
}

int moe_zc_scmoe_forward(const moe_zc_dims *dims, int32_t I_dense, int32_t nchunks,
                         const void *x_moe, const void *W_router, const float *bias,
                         const void *W_gate, const void *W_up, const void *W_down,
                         const void *x_dense, const void *W1, const void *W3, const void *W2,
                         void *out_moe, void *out_dense, int32_t *counts, int32_t *topk_idx,
                         float *topk_gate, void *ws_moe, size_t ws_moe_bytes, void *ws_dense,
                         size_t ws_dense_bytes, void *stream_moe, void *stream_dense) {
  size_t need_moe = 0, need_dense = 0;
  const int st0 = moe_zc_scmoe_workspace_bytes(dims, I_dense, nchunks, &need_moe, &need_dense);
  if (st0 != MOE_ZC_OK) return st0;
  (void)need_dense;  // dense_impl checks its own workspace
  const int64_t T = dims->T;
  // validate everything before enqueueing anything: the dense FFN, then
  // each chunk's forward with launches suppressed
  int st = dense_impl(T, dims->d, I_dense, x_dense, W1, W3, W2, out_dense, ws_dense,
                      ws_dense_bytes, static_cast<hipStream_t>(stream_dense), false);
  if (st != MOE_ZC_OK) return st;
  if (counts == nullptr) return MOE_ZC_EINVAL;
  if (T > 0 && ws_moe_bytes < need_moe) return MOE_ZC_ENOSPC;
  const size_t xbytes = static_cast<size_t>(T) * dims->d * 2;
  if (overlap(out_moe, xbytes, out_dense, xbytes) || overlap(out_moe, xbytes, x_dense, xbytes) ||
      overlap(out_dense, xbytes, x_moe, xbytes))
    return MOE_ZC_EINVAL;
  const int64_t rows = chunk_rows(T, nchunks);
  const int E = dims->N + dims->Z;
  for (int pass = 0; pass < 2; ++pass) {
    // MoE chunks in token order on stream_moe (a chunk past T has no rows:
    // its counts are zeroed)
    for (int c = 0; c < nchunks; ++c) {
      const int64_t t0 = std::min<int64_t>(c * rows, T);
      moe_zc_dims cd = *dims;
      cd.T = std::min<int64_t>(rows, T - t0);
      const size_t ro = static_cast<size_t>(t0) * dims->d * 2;
      st = forward_impl(&cd, static_cast<const char *>(x_moe) + ro, W_router, bias, W_gate, W_up,
                        W_down, static_cast<char *>(out_moe) + ro, counts + static_cast<size_t>(c) * E,
                        topk_idx ? topk_idx + t0 * dims->k : nullptr,
                        topk_gate ? topk_gate + t0 * dims->k : nullptr, ws_moe, ws_moe_bytes,
                        stream_moe, nullptr, nullptr, pass == 1);
      if (st != MOE_ZC_OK) return st;
    }
  }
  // then the dense FFN, whole, on stream_dense
  return dense_impl(T, dims->d, I_dense, x_dense, W1, W3, W2, out_dense, ws_dense, ws_dense_bytes,
                    static_cast<hipStream_t>(stream_dense), true);
}

const char *moe_zc_status_string(int status) {
  switch (status) {
    case MOE_ZC_OK: return "ok";
    case MOE_ZC_EINVAL: return "invalid argument (size, count or pointer)";
    case MOE_ZC_EDTYPE: return "unsupported dtype";
    case MOE_ZC_EALIGN:
      return "misaligned pointer, or d / I not a multiple of 8 (FP8: 128) where required";
    case MOE_ZC_ENOSPC: return "workspace missing or too small (or timer full)";
    case MOE_ZC_EHIP: return "HIP launch failed";
    case MOE_ZC_ESCRATCH:
      return "problem needs more workspace than the no-alloc entry point's static scratch "
             "(MOE_ZC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int moe_zc_timer_create(int max_calls, moe_zc_timer **out) {
  if (out == nullptr || max_calls < 1) return MOE_ZC_EINVAL;
  *out = nullptr;
  moe_zc_timer *t = new (std::nothrow) moe_zc_timer;
  if (!t) return MOE_ZC_EINVAL;
  const size_t n = static_cast<size_t>(max_calls) * (MOE_ZC_MAX_STAGES + 1);
  t->ev = new (std::nothrow) hipEvent_t[n];
  t->nst = new (std::nothrow) int[static_cast<size_t>(max_calls)];
  if (!t->ev || !t->nst) {
    delete[] t->ev;
    delete[] t->nst;
    delete t;
    return MOE_ZC_EINVAL;
  }
  t->max_calls = max_calls;
  t->ncalls = 0;
  for (size_t i = 0; i < n; ++i) {
    if (hipEventCreate(&t->ev[i]) != hipSuccess) {
      for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(t->ev[j]);
      delete[] t->ev;
      delete[] t->nst;
      delete t;
      return MOE_ZC_EHIP;
    }
  }
  *out = t;
  return MOE_ZC_OK;
}

int moe_zc_timer_read(moe_zc_timer *t, int *ncalls, float *ms) {
  if (t == nullptr || ms == nullptr) return MOE_ZC_EINVAL;
  for (int s = 0; s < MOE_ZC_MAX_STAGES; ++s) ms[s] = 0.0f;
  for (int c = 0; c < t->ncalls; ++c) {
    hipEvent_t *ev = t->ev + static_cast<size_t>(c) * (MOE_ZC_MAX_STAGES + 1);
    const int ns = t->nst[c];
    if (hipEventSynchronize(ev[ns]) != hipSuccess) return MOE_ZC_EHIP;
    for (int s = 0; s < ns; ++s) {
      float v = 0.0f;
      if (hipEventElapsedTime(&v, ev[s], ev[s + 1]) != hipSuccess) return MOE_ZC_EHIP;
      ms[s] += v;
    }
  }
  if (ncalls) *ncalls = t->ncalls;
  return MOE_ZC_OK;
}

void moe_zc_timer_reset(moe_zc_timer *t) {
  if (t) t->ncalls = 0;
}

void moe_zc_timer_destroy(moe_zc_timer *t) {
  if (!t) return;
  const size_t n = static_cast<size_t>(t->max_calls) * (MOE_ZC_MAX_STAGES + 1);
  for (size_t i = 0; i < n; ++i) (void)hipEventDestroy(t->ev[i]);
  delete[] t->ev;
  delete[] t->nst;
  delete t;
}

}  // extern "C"
