/*
 * qlinear.h -- C ABI of libqlinear.so: the quantized linear layer of a
 * diffusion transformer on AMD Instinct MI355X (gfx950).
 *
 *   Y = dequant( Q_w(W') * Q_a(X') )        X' = X H, W' = W H (optional)
 *
 * computed in four steps, each in hand-written HIP kernels:
 *   1. optional block Walsh-Hadamard rotation of X (and of W at plan time)
 *      -- HQ-DM explainer, technical summary 2.1 (block-diagonal H built
 *      from standard Hadamard matrices; the normalisation is a power of two
 *      folded into the float scales so the core stays integer);
 *   2. DualScale activation quantization: one scale for the non-negative
 *      region and one for the negative region, codes int8 or int4, optional
 *      truncation of k low bits of every code -- SegQuant explainer,
 *      technical summary 2.B; TASQ explainer, technical summary 2;
 *   3. integer GEMM of both polarity planes against the weight codes, with
 *      weight scales per output channel, per output segment or per tensor --
 *      SegQuant explainer 2.A (output segmentation) and 2.B (two products
 *      run as one batched GEMM);
 *   4. fp32 epilogue: scaled sum of the two products, optionally fused with
 *      the classifier-free-guidance combine uncond + w * (cond - uncond) --
 *      "Closing the Null Space" explainer, problem statement.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers on the device that was current
 *     when the plan was made, row-major and contiguous, owned by the caller;
 *     the library never frees or retains them. Host pointers are marked HOST.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is enqueued asynchronously on it; no call synchronises the
 *     host or copies device data to the host, except qlinear_plan and
 *     qlinear_plan_lsb_view (below). qlinear_quantize_act, qlinear_gemm,
 *     qlinear_cfg_combine and qlinear_plan_lsb_update enqueue kernel
 *     launches only (no allocation, no memset), so they can be captured
 *     into a HIP graph.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     violation returns QL_ERR_ARG (or QL_ERR_UNSUPPORTED for a valid but
 *     unimplemented combination) and enqueues nothing. A failed HIP launch
 *     or allocation returns QL_ERR_HIP / QL_ERR_OOM. qlinear_last_error()
 *     then gives a message (thread-local; valid until the next call on that
 *     thread).
 *   - Inputs must be finite; non-finite values give unspecified codes.
 *   - A plan is immutable after qlinear_plan returns, except for a small
 *     internal reduction workspace used by qlinear_quantize_act and, with
 *     input branches, a partial-sum workspace used by qlinear_gemm: calls of
 *     qlinear_quantize_act with dynamic scales on one plan must be ordered
 *     (one stream, or explicit events), and so must calls of qlinear_gemm on
 *     one plan with input branches; other calls may run concurrently.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct qlinear_plan* qlinear_plan_t; /* opaque, owned by the library */

typedef enum {
  QL_OK = 0,
  QL_ERR_ARG = 1,
  QL_ERR_UNSUPPORTED = 2,
  QL_ERR_OOM = 3,
  QL_ERR_HIP = 4
} ql_status;

typedef enum { QL_F32 = 0, QL_BF16 = 1 } ql_dtype;

/* Weight-scale granularity (SegQuant explainer 2.A: each output segment of a
 * chunked linear is quantized on its own). PER_TENSOR is one segment. */
typedef enum {
  QL_WSCALE_PER_TENSOR = 0,
  QL_WSCALE_PER_SEGMENT = 1,
  QL_WSCALE_PER_CHANNEL = 2
} ql_wscale;

/* Activation scales: DUAL = separate s+ / s- for the non-negative and the
 * negative region (SegQuant explainer 2.B); SYMMETRIC = one scale
 * max|x|/qmax for both (HQ-DM explainer 2.2 uses symmetric activations). */
typedef enum { QL_ASCALE_DUAL = 0, QL_ASCALE_SYMMETRIC = 1 } ql_ascale;

typedef struct {
  int32_t N, K;              /* W is [N,K]; Y = X W^T. 1 <= N, 16 <= K <= 65536 */
  int32_t w_bits, a_bits;    /* each 8 or 4 */
  int32_t hadamard_block;    /* 0 = no rotation; else B in {4,8,...,128}, K % B == 0 */
  int32_t n_segments;        /* >= 1 output segments partitioning [0,N) */
  const int32_t* seg_offsets;/* HOST [n_segments+1]: 0 = o_0 < o_1 < ... < o_n = N;
                                NULL means one segment [0,N) */
  ql_wscale w_scale_mode;
  ql_ascale a_scale_mode;
  ql_dtype x_dtype;          /* dtype of X given to qlinear_quantize_act */
  int32_t single_hadamard;   /* 0: rotate X and W (two-sided); 1: rotate X only
                                (HQ-DM explainer 2.1, single transform): W is
                                quantized unrotated and enters the product as
                                H W_int^T. Needs hadamard_block > 0 and
                                a_scale_mode SYMMETRIC (HQ-DM explainer 2.2). */
  int32_t n_k_segments;      /* input branches S (SegQuant explainer 2.A, input
                                segmentation: the input is a concatenation along
                                K and each branch is quantized on its own):
                                0 or 1 = none, at most 4 */
  const int32_t* k_seg_offsets;/* HOST [S+1]: 0 = k_0 < k_1 < ... < k_S = K, the
                                inner ones multiples of 128; NULL when S <= 1 */
} ql_desc;

/* Shape rules checked by every call: K % 16 == 0 when both w_bits and
 * a_bits are 8, K % 32 == 0 when either is 4. */

/*
 * Build a plan for one linear layer: rotate the rows of W block-wise by the
 * unnormalised Sylvester Hadamard matrix of order hadamard_block (stages of
 * butterfly distance 1, 2, ..., B/2, each (a,b) -> (a+b, a-b) in fp32), take
 * the symmetric absmax weight scale per channel / segment / tensor
 * (s = absmax / qmax_w, qmax_w = 2^(w_bits-1) - 1), quantize
 * (round half to even, clamp to [-qmax_w, qmax_w]); with input branches,
 * each branch's columns get their own scales, s_w[j][n], by the same rule
 * over those columns only. Storage: 4-bit codes (in [-7, 7]) are kept two
 * per byte, [N, K/2], code 2i in the low nibble of byte i (the layout of
 * the 4-bit activation codes), and unpacked by the GEMM in LDS; 8-bit codes
 * one per byte. Exceptions, one byte per code: single_hadamard plans and
 * plans with 3 or 4 input branches.
 *   d   : HOST descriptor (copied; seg_offsets and k_seg_offsets copied too).
 *   W   : DEVICE fp32 [N,K]; read only, may be freed after the call.
 *   out : HOST; receives the plan handle.
 * Allocates device memory for the plan and synchronises `stream` before it
 * returns (plan building is offline work). Errors: QL_ERR_ARG for a bad
 * descriptor or NULL pointer, QL_ERR_UNSUPPORTED for more than 4 input
 * branches, an inner branch offset that is not a multiple of 128, or input
 * branches with single_hadamard, QL_ERR_OOM, QL_ERR_HIP.
 * Method: DualScale weight side -- SegQuant explainer 2.B; per-segment
 * scales -- SegQuant explainer 2.A; rotation -- HQ-DM explainer 2.1.
 */
ql_status qlinear_plan(const ql_desc* d, const float* W, void* stream, qlinear_plan_t* out);
/* With single_hadamard = 1 the plan quantizes W without rotation (scales and
 * codes W_int as above) and keeps, besides W_int, the exact integer matrix
 * V = H W_int^T (|V| <= B * qmax_w) as two int8 planes V = 128 hi + lo. The
 * GEMM then computes acc = sum_k c[m,k] V[k,n] exactly and the epilogue
 * y = ((float)acc * s) * s_w[n] * (1/B), (float) rounding the exact sum once:
 * X W^T = (1/B) (X H)(H W^T) because H H = B I. */

/* Free a plan's device memory (weights shared with views are freed with
 * the last of them). The caller ensures no enqueued work still uses it
 * (synchronise first). NULL is accepted. */
ql_status qlinear_plan_destroy(qlinear_plan_t p);

/* Copy a plan's weights out for inspection: w_codes DEVICE int8 [N,K]
 * (one code per byte, unpacked if stored packed; a view's codes with its
 * depth applied; the unrotated W_int for single_hadamard; 16-byte aligned
 * for a view), w_scales DEVICE fp32 [S,N] (S input branches, 1 without).
 * Either may be NULL to skip it. */
ql_status qlinear_plan_weights(qlinear_plan_t p, int8_t* w_codes, float* w_scales, void* stream);

/*
 * Weight-side operating precision of TASQ (TASQ explainer, technical summary
 * 2, shared weights with an LSB mask): one stored set of weight codes, run
 * at a per-layer, per-step precision by dropping low bits of every code.
 * Reading of the mask equation there: a layer run with w_lsb_k dropped bits
 * uses c' = sign(c) * (|c| with its w_lsb_k low bits cleared), the same
 * truncation as lsb_k of qlinear_quantize_act, and keeps its weight scales.
 *
 * qlinear_plan_lsb_view: make a new plan whose weight codes are base's
 * truncated by w_lsb_k and whose descriptor, segments and scales are base's.
 * As on the page, there is one stored buffer: the view shares base's codes
 * and scales and carries the depth, which qlinear_gemm applies to the codes
 * as it loads them (a view of a view clears max of the two depths). The
 * view holds its own reduction workspace, is destroyed with
 * qlinear_plan_destroy in any order relative to base (the shared buffer
 * goes with the last of them), and is used in every call like a plan.
 * Exceptions: views of single_hadamard plans (whose GEMM planes are built
 * from the truncated codes) and of plans with 3 or 4 input branches hold a
 * truncated copy of the codes and scales. Allocates device memory and
 * synchronises `stream` before it returns.
 *   base     : plan on the current device.
 *   w_lsb_k  : 0 <= w_lsb_k < w_bits (0 gives a copy of base).
 *   out      : HOST; receives the view handle.
 * Errors: QL_ERR_ARG (NULL, w_lsb_k out of range, base on another device),
 * QL_ERR_OOM, QL_ERR_HIP.
 */
ql_status qlinear_plan_lsb_view(qlinear_plan_t base, int32_t w_lsb_k, void* stream,
                                qlinear_plan_t* out);

/*
 * Set the depth of an existing view for a new step: view's codes = base's
 * truncated by w_lsb_k, view's scales = base's (TASQ explainer, technical
 * summary 2). For a view sharing base's buffer this moves no data: calls
 * made on the view after this returns use the new depth, calls enqueued
 * before keep theirs. For a view with its own copy (see
 * qlinear_plan_lsb_view) the rewrite is enqueued on `stream` with no
 * allocation and no host synchronisation, and work already enqueued on the
 * view must be ordered before this call (same stream or events). Errors:
 * QL_ERR_ARG (NULL, view == base, w_lsb_k out of range, view and base with
 * different descriptors or segments), QL_ERR_HIP.
 */
ql_status qlinear_plan_lsb_update(qlinear_plan_t view, qlinear_plan_t base, int32_t w_lsb_k,
                                  void* stream);

/*
 * Quantize activations X [M,K] (x_dtype of the plan) to codes.
 * Steps per element: optional block rotation (as for W), then per-tensor
 * scales over all M*K rotated values: s+ = max(0, max x)/qa and
 * s- = max(0, -min x)/qa with qa = 2^(a_bits-1) - 1 (SYMMETRIC: both equal
 * max(0, max x, -min x)/qa), or the given static scales; then
 * x >= 0 -> round_half_even(x / s+) clamped to [0, qa], x < 0 ->
 * round_half_even(x / s-) clamped to [-qa, 0] (a zero scale gives 0;
 * division is IEEE fp32, correctly rounded); then, when lsb_k > 0, the k low
 * bits of the code's magnitude are cleared with the sign kept.
 * With S > 1 input branches every branch (the columns [k_j, k_j+1) of all
 * rows) gets its own scale pair, taken and applied as above over its values
 * only.
 *   X             : DEVICE [M,K], fp32 or bf16 per the plan.
 *   M             : rows, >= 0 (0 enqueues nothing).
 *   lsb_k         : 0 <= lsb_k < a_bits.
 *   static_scales : DEVICE fp32 [2S] {s+, s-} per branch, or NULL for
 *                   dynamic scales (S = 1 without input branches).
 *   codes         : DEVICE out: int8 [M,K] (a_bits 8) or uint8 [M,K/2]
 *                   (a_bits 4), two 4-bit two's-complement codes per byte:
 *                   element 2j in bits 0-3 and 2j+1 in bits 4-7 of byte j.
 *   act_scales    : DEVICE out fp32 [2S] {s+, s-} per branch, as used.
 * Method: rotation -- HQ-DM explainer 2.1; DualScale scales and the two
 * polarity regions -- SegQuant explainer 2.B; per-branch scales -- SegQuant
 * explainer 2.A (input segmentation); low-bit truncation -- TASQ explainer,
 * technical summary 2.
 */
ql_status qlinear_quantize_act(qlinear_plan_t p, const void* X, int32_t M, int32_t lsb_k,
                               const float* static_scales, void* codes, float* act_scales,
                               void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, arguments, results and errors as qlinear_quantize_act, but
 * the per-block partial maxima of a dynamic-scale call go to a scratch array
 * that the library keeps in device memory (96.25 KiB per device, reserved when
 * the library is loaded, held until the process ends) instead of the plan's
 * workspace. The scratch holds every partial a call writes (at most 1024 per
 * input branch, whatever M), so no size is refused for its sake; a call
 * never allocates, frees or synchronises. All calls on one device share its
 * scratch: two such calls with dynamic scales that overlap in time on one
 * device (different streams without ordering) race and give undefined
 * codes; calls ordered on one stream are safe (each writes all the partials
 * it reads). The first call on a device looks up the scratch's address
 * there (host-side, no allocation).
 */
ql_status qlinear_quantize_act_noalloc(qlinear_plan_t p, const void* X, int32_t M,
                                       int32_t lsb_k, const float* static_scales, void* codes,
                                       float* act_scales, void* stream);

/*
 * Integer GEMM of the codes against the plan's weight codes with the fp32
 * epilogue. DUAL: acc+ = sum_k max(c,0) w, acc- = sum_k min(c,0) w (int32,
 * exact), y = ((float)acc+ * s+ + (float)acc- * s-) * s_w[n];
 * SYMMETRIC: y = ((float)(acc+ + acc-) * s) * s_w[n]; then y *= 1/B when the
 * plan rotates (B = hadamard_block). With S > 1 input branches, y_j is the
 * above (before 1/B) over branch j's columns with its own scales s_j and
 * weight scales s_w[j][n], and y = (((y_0 + y_1) + y_2) + ...) * (1/B).
 * All fp32 operations are rounded
 * individually in this order (no fused multiply-add).
 *   codes      : DEVICE, as written by qlinear_quantize_act, M rows.
 *   act_scales : DEVICE fp32 [2S].
 *   M          : rows, >= 0; must be even when cfg = 1.
 *   cfg        : 0 -> Y [M,N] = y.
 *                1 -> rows [0,M/2) are conditional, [M/2,M) unconditional;
 *                     Y [M/2,N] = yu + w * (yc - yu), with d = yc - yu,
 *                     t = w * d, Y = yu + t rounded in that order.
 *   w          : guidance weight (used when cfg = 1).
 *   Y          : DEVICE fp32 out, [M,N] or [M/2,N].
 *   acc_dbg    : NULL, or DEVICE int32 [2S,M,N] out: plane 2j = acc+, plane
 *                2j+1 = acc- of branch j for every row (SYMMETRIC: plane 0 = acc+ + acc-,
 *                plane 1 = 0; single_hadamard: the exact sum is 128 * plane 0
 *                + plane 1, the products with the hi and lo planes). For
 *                parity checks; costs extra stores.
 * Errors besides the common ones: QL_ERR_UNSUPPORTED when M > 2^23, when
 * codes or weights reach 2 GiB, or when a 128-row block of Y does (N * 512
 * bytes >= 2^31: output offsets are 32-bit).
 * Method: the two products and their fused rescaled sum -- SegQuant
 * explainer 2.B; per-branch parts -- SegQuant explainer 2.A; normalisation
 * 1/B -- HQ-DM explainer 2.1; CFG combine -- "Closing the Null Space"
 * explainer, problem statement; a view's weight depth -- TASQ explainer,
 * technical summary 2.
 */
ql_status qlinear_gemm(qlinear_plan_t p, const void* codes, const float* act_scales, int32_t M,
                       int32_t cfg, float w, float* Y, int32_t* acc_dbg, void* stream);

/*
 * Standalone classifier-free-guidance combine ("Closing the Null Space"
 * explainer, problem statement): for r < M/2,
 * out[r,n] = Y[r+M/2,n] + w * (Y[r,n] - Y[r+M/2,n]), rounded as in
 * qlinear_gemm. Y DEVICE fp32 [M,N] (M even), out DEVICE fp32 [M/2,N];
 * out must not overlap Y.
 */
ql_status qlinear_cfg_combine(const float* Y, int32_t M, int32_t N, float w, float* out,
                              void* stream);

/*
 * Measurement aid, not a step of the method: the int8 matrix-core rate the
 * device sustains, reported beside the spec peak as the GEMM's measured
 * ceiling. One workgroup per compute unit of the current device, with
 * waves_per_simd waves on each SIMD; every wave loads the same 16 operand
 * fragments and issues 16 * iters v_mfma_i32_16x16x64_i8 into 16
 * independent accumulators, successive instructions taking different
 * fragment pairs (accumulator j multiplies activation-side fragment j % 8
 * by weight-side fragment (j + j / 8) % 8). No memory access inside the
 * loop, no barrier, no epilogue. Each thread then writes the int32 sum,
 * wrapped modulo 2^32, of its accumulator registers.
 *   operands       : DEVICE int8 [16][64][16]: fragment f (0-7 activation
 *                    side, 8-15 weight side), lane l, byte i. In the
 *                    instruction's layout lane l holds row (column) l % 16
 *                    and the 16 K elements 16 * (l / 16) ... + 15. Random
 *                    bytes give the rate with operand switching, constant
 *                    bytes the rate without it.
 *   iters          : in [0, 2^24].
 *   waves_per_simd : 1 or 2.
 *   sink           : DEVICE int32 out [compute units * 256 * waves_per_simd],
 *                    thread t of workgroup b at b * 256 * waves_per_simd + t.
 *   sink_len       : int32 elements of sink; a shorter sink is refused
 *                    (QL_ERR_ARG) before anything is enqueued.
 * Total int8 operations of a call: compute units * 4 * waves_per_simd *
 * iters * 16 * 2 * 16 * 16 * 64.
 * Errors besides the common ones: QL_ERR_ARG for NULL or misaligned
 * pointers, out-of-range sizes and a sink shorter than the grid.
 */
ql_status qlinear_probe_mfma(const void* operands, int32_t iters, int32_t waves_per_simd,
                             int32_t* sink, int64_t sink_len, void* stream);

/* Message for the last non-OK status on this thread ("" if none). */
const char* qlinear_last_error(void);

/* Library version string. */
const char* qlinear_version(void);

/*
 * Host-only (no device work, usable without a GPU): GAMP's activation-bit
 * allocation -- "Closing the Null Space" explainer, methodology (allocation
 * strategy), with BOPs counted over the guided step as its key contribution
 * 4 asks. Weights stay at w_bits; every layer starts at 4-bit activations;
 * layers are ranked by gain[l] / (macs[l] * w_bits * 4), the sensitivity
 * removed per bit operation added by a promotion (equal ratios keep layer
 * order), and promoted to 8-bit activations in that order whenever the
 * total still fits the budget (a layer that does not fit is skipped and the
 * scan goes on).
 *   n_layers    : >= 1.
 *   macs        : HOST int64 [n_layers], multiply-accumulates of each layer
 *                 over the guided step (both CFG branches), in [1, 2^52].
 *   gain        : HOST double [n_layers], finite, >= 0: the guided-output
 *                 error removed by running layer l at 8 instead of 4 bits.
 *   w_bits      : 4 or 8.
 *   budget_bops : total BOPs allowed, sum of macs * w_bits * a_bits; at
 *                 least the all-4-bit total.
 *   a_bits      : HOST out int32 [n_layers], 4 or 8.
 *   bops        : HOST out, the allocation's total BOPs (exact).
 * Errors: QL_ERR_ARG (NULL, bad sizes or values, budget below the all-4-bit
 * total, totals beyond int64).
 */
ql_status qlinear_gamp_allocate(int32_t n_layers, const int64_t* macs, const double* gain,
                                int32_t w_bits, int64_t budget_bops, int32_t* a_bits,
                                int64_t* bops);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
