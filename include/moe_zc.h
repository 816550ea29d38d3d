/*
 * moe_zc.h -- C ABI of the MI355X (gfx950) zero-computation-expert MoE forward.
 *
 * The operation (LongCat-Flash technical-report summary page, section 2
 * "architecture", item 1 "zero-computation experts"; model configuration in
 * the same section): every token is routed among N FFN experts and Z
 * zero-computation experts.  A zero-computation expert returns its input
 * unchanged and costs no compute.  An expert-specific bias, driven by a
 * controller from the per-expert selection counts, shifts the routing scores
 * so the share of FFN vs zero experts stays on target.
 *
 * Concretely, for each token t with activations x[t] (length d):
 *   1. l[e]   = <x[t], W_router[e]>          for all E = N + Z experts
 *      p     = softmax(l)                    (over all E, fp32)
 *   2. s[e]   = p[e] + bias[e]               (selection only)
 *      idx   = the k experts of largest s, by s descending, ties -> lower e
 *      gate_j = routed_scale * p[idx_j]      (unbiased, no renormalisation;
 *                                             routed_scale in moe_zc_dims)
 *   3. FFN expert e < N: y_e = W_down[e] (silu(W_gate[e] x) * (W_up[e] x)),
 *      silu(z) = z / (1 + exp(-z))           (SwiGLU, three matrices, no bias)
 *   4. zero expert e >= N: contributes gate * x (identity)
 *   5. out[t] = (sum of zero-slot gates) * x[t] + sum_j gate_j * y_{idx_j},
 *      counts[e] = number of (t, j) with idx_j == e   (sums to T * k)
 * Expert numbering: 0 .. N-1 are FFN experts, N .. N+Z-1 zero experts.
 *
 * Precision: storage in the dims' dtype (fp32 or bfloat16); products are
 * accumulated in fp32; the router softmax is fp32 with the hardware exp2
 * and reciprocal (a few ulp from exactly rounded); for bfloat16 the SwiGLU
 * activations and the expert outputs are rounded to bfloat16 between the
 * two expert GEMMs and before the combine; the combine sums in fp32 in
 * ascending slot order and rounds once.  The combine uses no atomics:
 * results are run-to-run bit-identical.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or synchronises, and is re-entrant per
 *     stream; its only global state is the per-GPU scratch array of
 *     moe_zc_forward_noalloc (below).  `stream` is a hipStream_t (NULL = the
 *     default stream).
 *   - Work is enqueued asynchronously on `stream`.  Arguments are validated
 *     before anything is enqueued; on a validation error nothing is written.
 *     A failed launch returns MOE_ZC_EHIP.  Faults inside kernels surface at
 *     the caller's next synchronisation.
 *   - Apart from the timer calls, an entry point enqueues kernel launches
 *     only (no memset, copy or event), so a call with caller-allocated
 *     buffers can be captured into a HIP graph and replayed.
 */
#ifndef MOE_ZC_H
#define MOE_ZC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_ZC_F32 = 0, MOE_ZC_BF16 = 1 } moe_zc_dtype;

typedef enum {
  MOE_ZC_OK = 0,
  MOE_ZC_EINVAL = -1, /* a size, count or pointer argument is invalid        */
  MOE_ZC_EDTYPE = -2, /* dtype is neither MOE_ZC_F32 nor MOE_ZC_BF16          */
  MOE_ZC_EALIGN = -3, /* a pointer is misaligned, or d / I not a multiple of 8
                         (128 for FP8) where the entry point needs it        */
  MOE_ZC_ENOSPC = -4, /* workspace missing or smaller than the query          */
  MOE_ZC_EHIP = -5,   /* a HIP launch failed                                  */
  MOE_ZC_ESCRATCH = -6 /* moe_zc_forward_noalloc: the problem needs more than
                          MOE_ZC_SCRATCH_BYTES of workspace                   */
} moe_zc_status;

/* The problem.  Limits: T >= 0; d >= 1 and I >= 1 (moe_zc_forward and
 * moe_zc_forward_noalloc; the backward, FP8 and dense-FFN entry points need
 * multiples of 8, and FP8 of 128); N >= 0, Z >= 0, 1 <= N + Z <= 2048;
 * 1 <= k <= min(64, N + Z); T * k < 2^31; with d8 and I8 the widths rounded
 * up to multiples of 8: T * d8 and I8 * d8 (times the element size) below
 * 2 GiB, d8 and I8 at most 2^22; routed_scale finite and > 0.  I is ignored
 * when N == 0.
 * routed_scale (LongCat-Flash-Lite article, part 02: the fused router kernel
 * ends with a scaling step; the pages do not say what it scales): every
 * selected slot's gate is routed_scale * p[idx] (FFN and zero slots alike),
 * the selection does not depend on it, and the backward's router gradient
 * carries it.  1.0f is the unscaled method; a zeroed field is rejected
 * (MOE_ZC_EINVAL) rather than silently zeroing every gate. */
typedef struct {
  int64_t T;          /* tokens                                   */
  int32_t d;          /* model width                               */
  int32_t I;          /* FFN expert width                          */
  int32_t N;          /* FFN experts                               */
  int32_t Z;          /* zero-computation experts                  */
  int32_t k;          /* experts per token                         */
  int32_t dtype;      /* moe_zc_dtype of x, weights and out        */
  float routed_scale; /* gate = routed_scale * p (1.0f: unscaled)  */
} moe_zc_dims;

/* Bytes of device workspace moe_zc_forward needs for `dims` (worst case:
 * every slot an FFN expert; with d or I not a multiple of 8 also room for
 * the zero-padded copies described at moe_zc_forward).  Returns 0 for
 * invalid dims. */
size_t moe_zc_workspace_bytes(const moe_zc_dims *dims);

/* The forward pass, steps 1-5 above.
 *   x          [T, d]        dtype, row-major, 16-byte aligned
 *   W_router   [N+Z, d]      dtype, row e = expert e
 *   bias       [N+Z]         fp32, used for selection only
 *   W_gate     [N, I, d]     dtype (NULL allowed when N == 0)
 *   W_up       [N, I, d]     dtype (NULL allowed when N == 0)
 *   W_down     [N, d, I]     dtype (NULL allowed when N == 0)
 *   out        [T, d]        dtype, overwritten; must not overlap x
 *   counts     [N+Z]         int32, overwritten (zeroed when T == 0)
 *   topk_idx   [T, k]        int32, nullable; biased score descending,
 *                            ties -> lower index
 *   topk_gate  [T, k]        fp32, nullable; the gates, routed_scale times
 *                            the unbiased probabilities
 *   workspace  >= moe_zc_workspace_bytes(dims) bytes, 256-byte aligned;
 *              its contents on entry are ignored
 * Widths that are not multiples of 8: the kernels move 16-byte row pieces,
 * so the call first copies x, W_router, W_gate, W_up and W_down into the
 * workspace with d and I rounded up to multiples of 8 and the new columns
 * and rows zero, runs on those, and copies the first d columns of each
 * output row back.  The result is the same as on the unpadded operands
 * (every added product has an exact zero factor, and the added SwiGLU
 * features, silu(0) * 0 = 0, meet zero columns of W_down).  The copies
 * read all expert weights on every call: this path serves odd shapes, not
 * speed; the stage timer does not include them.
 * Returns a moe_zc_status. */
int moe_zc_forward(const moe_zc_dims *dims, const void *x, const void *W_router,
                   const float *bias, const void *W_gate, const void *W_up, const void *W_down,
                   void *out, int32_t *counts, int32_t *topk_idx, float *topk_gate,
                   void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * The forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results as
 * moe_zc_forward (bit for bit), except that the workspace is a fixed array
 * of MOE_ZC_SCRATCH_BYTES inside the library's device image, one per GPU
 * the library runs on, held until the process ends.  Its address is looked
 * up once per device (hipGetSymbolAddress, on the first call that targets
 * the device of `stream`, with that device made current for the lookup);
 * the call itself allocates nothing.  Nothing in the array needs to start
 * at zero: a call ignores what the previous one left there.
 *   - MOE_ZC_ESCRATCH when moe_zc_workspace_bytes(dims) exceeds
 *     MOE_ZC_SCRATCH_BYTES (e.g. the decode shape T = 128, d = 6144,
 *     I = 2048, 512 + 256 experts, top-12 needs about 32 MB and fits; the
 *     prefill shapes do not); other errors as moe_zc_forward; every argument
 *     is validated before anything is enqueued.
 *   - Every call on one GPU shares that GPU's array: calls that may overlap
 *     on one GPU (on different streams, or from several threads without
 *     ordering) race and corrupt each other's results.  Calls on one stream
 *     are ordered and safe.
 *   - MOE_ZC_EHIP if the array's address cannot be obtained.
 * ------------------------------------------------------------------------ */
#define MOE_ZC_SCRATCH_BYTES ((size_t)64 << 20)

int moe_zc_forward_noalloc(const moe_zc_dims *dims, const void *x, const void *W_router,
                           const float *bias, const void *W_gate, const void *W_up,
                           const void *W_down, void *out, int32_t *counts, int32_t *topk_idx,
                           float *topk_gate, void *stream);

/* Static English text for a status code (never NULL). */
const char *moe_zc_status_string(int status);

/* ------------------------------------------------------------------------
 * Bias controller: the consumer of `counts`, run between forward calls.
 *
 * LongCat-Flash technical-report summary page, section 2 "architecture",
 * computation-budget control (also section 1, main contributions): an
 * expert-specific bias, adjusted by a PID controller, keeps the average
 * share of FFN vs zero-computation experts near its target.  The pages give
 * no formula or gains.  This library's reading, per expert e, in fp32 in
 * this order with no fused operations (bit-reproducible):
 *   err = (target[e] - counts[e]) / T            per-token load error
 *   mode 0 (incremental PID):
 *     u = ki*err + kp*(err - e1) + kd*((err - e1) - (e1 - e2))
 *     bias[e] += lr * u
 *   mode 1 (sign update, aux-loss-free style):
 *     bias[e] += lr * sign(err)                   (sign(0) = 0)
 * An under-selected expert (err > 0) gets a larger bias, so it is selected
 * more.  The caller owns the schedule (pass the decayed lr each call) and
 * the targets (e.g. share * T * k / N for each FFN expert and
 * (1 - share) * T * k / Z for each zero expert; they need not sum to T*k).
 *   counts  [E]    int32, as written by moe_zc_forward for a batch of T tokens
 *   target  [E]    fp32 desired selections per expert for that batch
 *   bias    [E]    fp32, updated in place
 *   state   [2*E]  fp32 (e1, e2) per expert, updated in place (e1 <- err,
 *                  e2 <- old e1); zero it before the first call.  Nullable:
 *                  then e1 = e2 = err, i.e. a pure integral step.
 * Device pointers, 4-byte aligned, owned by the caller; asynchronous on
 * `stream`.  MOE_ZC_EINVAL if E < 1, T < 1, a required pointer is NULL,
 * mode is not 0 or 1, or a gain or lr is not finite; MOE_ZC_EALIGN for a
 * misaligned pointer; nothing is enqueued on error. */
int moe_zc_bias_update(int32_t E, int64_t T, const int32_t *counts, const float *target,
                       float *bias, float *state, float lr, float ki, float kp, float kd,
                       int32_t mode, void *stream);

/* ------------------------------------------------------------------------
 * Per-stage timing (measurement aid).  A timer owns HIP events for up to
 * `max_calls` forward calls; moe_zc_forward_timed records an event before
 * the first and after every stage on `stream`.  moe_zc_timer_read waits for
 * the recorded events and returns, per stage, the summed milliseconds over
 * all recorded calls.  A timer is used by one stream at a time.
 * ------------------------------------------------------------------------ */
enum {
  MOE_ZC_STAGE_ROUTER = 0,  /* step 1: router logits GEMM             */
  MOE_ZC_STAGE_TOPK = 1,    /* steps 1-2: softmax, bias, top-k        */
  MOE_ZC_STAGE_SCAN = 2,    /* step 5 counts + dispatch offsets       */
  MOE_ZC_STAGE_PERMUTE = 3, /* dispatch: token -> expert row map      */
  MOE_ZC_STAGE_GATE_UP = 4, /* step 3: gate/up GEMM + SwiGLU          */
  MOE_ZC_STAGE_DOWN = 5,    /* step 3: down GEMM                      */
  MOE_ZC_STAGE_COMBINE = 6, /* steps 4-5: zero experts + combine      */
  MOE_ZC_NSTAGES = 7,
  /* stages of moe_zc_backward */
  MOE_ZC_BSTAGE_ROUTE = 0,         /* routing bookkeeping, permuted x / dy rows */
  MOE_ZC_BSTAGE_ROUTER = 1,        /* router logits GEMM (recomputed)           */
  MOE_ZC_BSTAGE_RECOMPUTE = 2,     /* G = X W_gate^T, U = X W_up^T              */
  MOE_ZC_BSTAGE_DGRAD_V = 3,       /* W_down^T dout -> dG, dU, H, gate grads    */
  MOE_ZC_BSTAGE_ROUTER_BWD = 4,    /* softmax backward -> router-logit grads    */
  MOE_ZC_BSTAGE_WGRAD_DOWN = 5,    /* dW_down += dY^T H                         */
  MOE_ZC_BSTAGE_WGRAD_GATE_UP = 6, /* dW_gate += dG^T X, dW_up += dU^T X        */
  MOE_ZC_BSTAGE_DGRAD_X = 7,       /* dG W_gate + dU W_up (permuted rows)       */
  MOE_ZC_BSTAGE_DX = 8,            /* router part of dx, gather of dx           */
  MOE_ZC_BSTAGE_WGRAD_ROUTER = 9,  /* dW_router += dl^T x                       */
  MOE_ZC_BWD_NSTAGES = 10,
  MOE_ZC_MAX_STAGES = 10
};

typedef struct moe_zc_timer moe_zc_timer;

/* Creates a timer (HIP events on the current device).  MOE_ZC_EINVAL if
 * max_calls < 1 or out is NULL, MOE_ZC_EHIP if event creation fails. */
int moe_zc_timer_create(int max_calls, moe_zc_timer **out);

/* As moe_zc_forward; also records events into `timer` (MOE_ZC_ENOSPC once
 * it holds max_calls calls; nothing is enqueued then). */
int moe_zc_forward_timed(const moe_zc_dims *dims, const void *x, const void *W_router,
                         const float *bias, const void *W_gate, const void *W_up,
                         const void *W_down, void *out, int32_t *counts, int32_t *topk_idx,
                         float *topk_gate, void *workspace, size_t workspace_bytes, void *stream,
                         moe_zc_timer *timer);

/* Waits for the recorded events; writes the number of recorded calls and
 * the per-stage millisecond sums (ms[MOE_ZC_MAX_STAGES]; a forward call adds
 * to its MOE_ZC_NSTAGES stages, a backward call to its MOE_ZC_BWD_NSTAGES). */
int moe_zc_timer_read(moe_zc_timer *timer, int *ncalls, float *ms);

/* Forgets the recorded calls. */
void moe_zc_timer_reset(moe_zc_timer *timer);

void moe_zc_timer_destroy(moe_zc_timer *timer);

/* ------------------------------------------------------------------------
 * Dense SwiGLU FFN and the two-stream ScMoE schedule.
 *
 * LongCat-Flash technical-report summary page, section 2 "architecture",
 * shortcut-connected MoE (ScMoE): a shortcut from the layer's first
 * attention output feeds the MoE block, so the MoE runs alongside the dense
 * FFN block instead of after it; section 5 "training infrastructure": the
 * MoE layer is split into two chunks along the token dimension, which
 * overlap with the dense FFN and with each other.  The model-configuration
 * paragraph gives the dense FFN path an intermediate width of 12288.
 *
 * moe_zc_dense_ffn: out[t] = W2 (silu(W1 x[t]) * (W3 x[t])), bfloat16,
 *   x [T, d], W1 and W3 [I_dense, d], W2 [d, I_dense], out [T, d] (must not
 *   overlap x); d and I_dense multiples of 8, at most 2^22; workspace of
 *   moe_zc_dense_workspace_bytes(T, d, I_dense) bytes, 256-byte aligned.
 *   It runs on the expert GEMM kernels as one expert that every token uses.
 *
 * moe_zc_scmoe_forward: enqueues the MoE block over x_moe on stream_moe, in
 *   nchunks (1 or 2) consecutive token chunks of ceil(T / nchunks) rows, and
 *   the dense FFN over x_dense on stream_dense; the two inputs are
 *   independent (the shortcut).  Each MoE chunk is moe_zc_forward on its
 *   rows (routing is per token; the chunks share ws_moe, so they run in
 *   order on stream_moe); counts is [nchunks, N+Z], chunk c's counts in row
 *   c; topk_idx / topk_gate [T, k] nullable.  Passing one stream for both is
 *   the serial schedule.  The caller joins the two streams.  Workspace sizes
 *   from moe_zc_scmoe_workspace_bytes.  bfloat16 only.  Everything is
 *   validated before anything is enqueued.
 * ------------------------------------------------------------------------ */
size_t moe_zc_dense_workspace_bytes(int64_t T, int32_t d, int32_t I_dense);

int moe_zc_dense_ffn(int64_t T, int32_t d, int32_t I_dense, const void *x, const void *W1,
                     const void *W3, const void *W2, void *out, void *workspace,
                     size_t workspace_bytes, void *stream);

int moe_zc_scmoe_workspace_bytes(const moe_zc_dims *dims, int32_t I_dense, int32_t nchunks,
                                 size_t *ws_moe, size_t *ws_dense);

int moe_zc_scmoe_forward(const moe_zc_dims *dims, int32_t I_dense, int32_t nchunks,
                         const void *x_moe, const void *W_router, const float *bias,
                         const void *W_gate, const void *W_up, const void *W_down,
                         const void *x_dense, const void *W1, const void *W3, const void *W2,
                         void *out_moe, void *out_dense, int32_t *counts, int32_t *topk_idx,
                         float *topk_gate, void *ws_moe, size_t ws_moe_bytes, void *ws_dense,
                         size_t ws_dense_bytes, void *stream_moe, void *stream_dense);

/* ------------------------------------------------------------------------
 * Backward of the block (training).
 *
 * LongCat-Flash technical-report summary page, section 5 "training
 * infrastructure": grouped GEMMs for the backward, fp32 accumulation of the
 * weight gradients fused into the GEMM ("GemmAdd"), deterministic gradient
 * aggregation.  The formulas are the chain rule through moe_zc_forward with
 * the routing held fixed (selection and bias are not differentiated):
 *   zero slot j:  dgate_j = <dout, x>,  dx += gate_j dout
 *   FFN slot j, expert e (g = W_gate[e] x, u = W_up[e] x, s = sigmoid(g),
 *   h = g s u):  v = W_down[e]^T dout,  dgate_j = <v, h>,  dh = gate_j v,
 *     dg = dh u s (1 + g (1 - s)),  du = dh g s,
 *     dx += W_gate[e]^T dg + W_up[e]^T du,
 *     dW_down[e] += gate_j dout h^T,  dW_gate[e] += dg x^T,  dW_up[e] += du x^T
 *   router (p = softmax(x W_router^T), gate_j = routed_scale * p[idx_j]):
 *     dl = p * (dp - <p, dp>), dp[idx_j] = routed_scale * dgate_j;
 *     dx += W_router^T dl,  dW_router += dl x^T
 *
 *   dims        as for moe_zc_forward; bfloat16 only (MOE_ZC_EDTYPE
 *               otherwise); d and I multiples of 8
 *   x, W_*      the forward's inputs (bfloat16, layouts of moe_zc_forward)
 *   topk_idx    [T, k] int32, topk_gate [T, k] fp32: the forward's routing
 *               outputs (with dims->routed_scale as in the forward).  An
 *               entry outside [0, N+Z), or repeating an earlier expert of
 *               its token, is ignored (that slot gets no gradient).
 *   dout        [T, d] bfloat16, the gradient of the forward's output
 *   dx          [T, d] bfloat16, overwritten (must not overlap x or dout)
 *   dW_router   [N+Z, d] fp32, dW_gate / dW_up [N, I, d] fp32,
 *   dW_down     [N, d, I] fp32: accumulated into (+=); an expert no token
 *               selects is not touched
 *   workspace   device memory of moe_zc_backward_workspace_bytes(dims)
 *               bytes, 256-byte aligned (sized for every slot on an FFN
 *               expert)
 *   stream      hipStream_t; timer nullable (stages MOE_ZC_BSTAGE_*)
 * The result is deterministic: every sum runs in a fixed order, and every
 * gradient element has one writer.  Returns MOE_ZC_OK or an error status;
 * on error nothing is enqueued.
 * ------------------------------------------------------------------------ */
size_t moe_zc_backward_workspace_bytes(const moe_zc_dims *dims);

int moe_zc_backward(const moe_zc_dims *dims, const void *x, const void *W_router,
                    const void *W_gate, const void *W_up, const void *W_down,
                    const int32_t *topk_idx, const float *topk_gate, const void *dout, void *dx,
                    float *dW_router, float *dW_gate, float *dW_up, float *dW_down,
                    void *workspace, size_t workspace_bytes, void *stream, moe_zc_timer *timer);

/* ------------------------------------------------------------------------
 * Block-scaled FP8 experts.
 *
 * LongCat-Flash technical-report summary page, section 6 "inference and
 * deployment", custom kernels, quantization item: fine-grained block
 * quantization as in DeepSeek-V3, activations per [1,128] block and weights
 * per [128,128] block.  This library's reading: values are OCP E4M3 bytes
 * (round to nearest even, saturating at 448), and every block has one
 * power-of-two scale 2^e, the smallest with 2^e >= amax / 448 (e >= -127;
 * e = 0 for an all-zero block), stored as the E8M0 byte e + 127.  The expert
 * GEMMs add, per 128-wide K block, 2^(e_a + e_b) times the fp32 sum of the
 * products of the E4M3 values.  The router stays bfloat16; x is quantized
 * per [1,128] before the gate/up projections and the SwiGLU activations per
 * [1,128] before the down projection; zero experts return the unquantized
 * x; expert outputs are bfloat16 and the combine is as in moe_zc_forward.
 * ------------------------------------------------------------------------ */

/* Quantizes nmat row-major [rows, K] matrices (src: fp32 or bf16 per
 * `dtype`) into q (same shape, E4M3 bytes) and scale_exp
 * [nmat, rows / block_rows, K / 128] (E8M0 bytes).  block_rows = 128 for
 * weights ([128,128] blocks), 1 for activations ([1,128] blocks).  Device
 * pointers, src and q 16-byte aligned; asynchronous on `stream`.
 * MOE_ZC_EDTYPE for another dtype; MOE_ZC_EINVAL for negative sizes, a
 * block_rows other than 1 or 128, or a NULL pointer with non-empty input;
 * MOE_ZC_EALIGN if rows is not a multiple of block_rows, K not a multiple
 * of 128, or a pointer is misaligned.  Empty input: MOE_ZC_OK, nothing
 * enqueued. */
int moe_zc_quantize_fp8(const void *src, int32_t dtype, int64_t nmat, int32_t rows, int32_t K,
                        int32_t block_rows, uint8_t *q, uint8_t *scale_exp, void *stream);

/* Workspace bytes of moe_zc_forward_fp8 for `dims` (0 for invalid dims). */
size_t moe_zc_workspace_bytes_fp8(const moe_zc_dims *dims);

/* The forward pass with FP8 experts: as moe_zc_forward, with
 *   dims->dtype   MOE_ZC_BF16 (x, W_router, out); d and I multiples of 128,
 *                 at most 12288
 *   W_gate, W_up  [N, I, d] E4M3, exponents W_*_exp [N, I/128, d/128]
 *   W_down        [N, d, I] E4M3, exponents W_down_exp [N, d/128, I/128]
 *                 (as produced by moe_zc_quantize_fp8 with block_rows 128)
 *   timer         nullable; as in moe_zc_forward_timed (the activation
 *                 quantization is timed with MOE_ZC_STAGE_PERMUTE)
 * MOE_ZC_EDTYPE unless dims->dtype is MOE_ZC_BF16; MOE_ZC_EALIGN if d or I
 * is not a multiple of 128; MOE_ZC_EINVAL if either exceeds 12288; other
 * errors as moe_zc_forward. */
int moe_zc_forward_fp8(const moe_zc_dims *dims, const void *x, const void *W_router,
                       const float *bias, const uint8_t *W_gate, const uint8_t *W_gate_exp,
                       const uint8_t *W_up, const uint8_t *W_up_exp, const uint8_t *W_down,
                       const uint8_t *W_down_exp, void *out, int32_t *counts, int32_t *topk_idx,
                       float *topk_gate, void *workspace, size_t workspace_bytes, void *stream,
                       moe_zc_timer *timer);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ZC_H */
