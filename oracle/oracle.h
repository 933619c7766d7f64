/*
 * CPU oracle for the quantized linear layer of a diffusion transformer.
 *
 * TEST INFRASTRUCTURE ONLY. This is the plain, slow, single-threaded
 * reference that the GPU path is checked against. Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the product path
 * never does. It shares no code, header, table or helper with the GPU
 * library.
 *
 * Arithmetic: fp32 with IEEE round-to-nearest-even, correctly rounded
 * division, no fused multiply-add (built with -ffp-contract=off), no
 * threads, no SIMD intrinsics. Integer accumulation in int32 (checked
 * against int64 for overflow).
 *
 * Sources (the pages):
 *   [SQ]  "SegQuant: A Semantics-Aware and Generalizable Quantization
 *          Framework for Diffusion Models" (gist.science explainer, es and ko),
 *          technical summary section 2: A SegLinear, B DualScale.
 *   [CFG] "Closing the Null Space: Guidance-Aware Quantization for
 *          Classifier-Free Diffusion", problem statement (guided prediction)
 *          and methodology (dual-branch calibration, greedy allocation of
 *          activation bits).
 *   [HQ]  "HQ-DM: Single Hadamard Transformation-Based Quantization-Aware
 *          Training for Low-Bit Diffusion Models", technical summary 2.1
 *          (block rotation, single transform) and 2.2 (symmetric scales).
 *   [TQ]  "TASQ: Temporal-Adaptive Bit Sparsification Quantization for
 *          Diffusion Models", technical summary section 2 (LSB mask, on the
 *          activation codes and on the shared weight codes).
 * Input segmentation ([SQ] 2.A) and the pipeline helpers are composed in
 * oracle/__init__.py from the functions below.
 *
 * Parity pins: every function is pinned by tests against closed forms,
 * invariants, library routines or brute force (see the oracle tests).
 */
#ifndef QL_ORACLE_H
#define QL_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Activation-scale modes (oracle-local numbering). */
#define ORC_ASCALE_DUAL 0
#define ORC_ASCALE_SYMMETRIC 1
/* Weight-scale modes (oracle-local numbering). */
#define ORC_WSCALE_TENSOR 0
#define ORC_WSCALE_SEGMENT 1
#define ORC_WSCALE_CHANNEL 2

/* Return codes. */
#define ORC_OK 0
#define ORC_EARG 1
#define ORC_ENONFINITE 2
#define ORC_EOVERFLOW 3

/* [HQ] 2.1: unnormalised Sylvester Walsh-Hadamard transform of one block of
 * B (power of two) floats, in place, stages h = 1, 2, ..., B/2. */
int orc_fwht_block(float* v, int32_t B);
/* Block-diagonal rotation: every row of x [rows, K], every B-block along K. */
int orc_rotate_rows(float* x, int64_t rows, int64_t K, int32_t B);

/* [SQ] 2.B: per-tensor act scales over n values.
 * s[0] = s_plus, s[1] = s_minus. */
int orc_act_scales(const float* x, int64_t n, int32_t a_bits, int32_t mode, float* s);

/* [SQ] 2.B + [TQ] 2: quantize one value / a whole tensor to signed codes
 * (unpacked int8, range [-qa, qa]), then truncate lsb_k low magnitude bits. */
int32_t orc_quant_value(float v, float s_plus, float s_minus, int32_t qa);
int32_t orc_truncate_lsb(int32_t c, int32_t k);
int orc_quantize_act(const float* x, int64_t n, const float* s, int32_t a_bits,
                     int32_t lsb_k, int8_t* codes);

/* [TQ] 2 on the stored weights: the operating weight codes of a layer at a
 * stage with k dropped bits, one orc_truncate_lsb per code (scales kept).
 * Codes must lie in [-qw, qw] of w_bits; 0 <= k < w_bits. */
int orc_truncate_codes(const int8_t* in, int64_t n, int32_t w_bits, int32_t k, int8_t* out);

/* Code storage for 4-bit codes: byte j of a row holds element 2j in bits 0-3
 * and element 2j+1 in bits 4-7, each a 4-bit two's-complement value. */
int orc_pack_int4(const int8_t* codes, int64_t rows, int64_t K, uint8_t* out);
int orc_unpack_int4(const uint8_t* packed, int64_t rows, int64_t K, int8_t* out);

/* [SQ] 2.A + weight quantization: symmetric absmax scales per channel, per
 * output segment or per tensor (seg = HOST [nseg+1] offsets; NULL = 1). */
int orc_weight_scales(const float* w, int64_t N, int64_t K, int32_t w_bits, int32_t mode,
                      int32_t nseg, const int32_t* seg, float* sw);
int orc_quantize_weight(const float* w, int64_t N, int64_t K, const float* sw,
                        int32_t w_bits, int8_t* wc);

/* [SQ] 2.B: the two integer contractions on a list of rows of c [*, K]:
 * accp[i,n] = sum_k max(c[row_i,k],0) * wc[n,k]; accn uses min(c,0). */
int orc_gemm_dual(const int8_t* c, const int8_t* wc, const int64_t* rows, int64_t nrows,
                  int64_t N, int64_t K, int32_t* accp, int32_t* accn);

/* [SQ] 2.B fused epilogue + [HQ] 2.1 normalisation folded into the scales:
 * y = ((float)accp*s+ + (float)accn*s-) * sw[n], then * (1/B) when B > 0.
 * SYMMETRIC: y = ((float)(accp+accn) * s+) * sw[n] (* 1/B). */
int orc_epilogue(const int32_t* accp, const int32_t* accn, int64_t nrows, int64_t N,
                 const float* s, const float* sw, int32_t B, int32_t mode, float* y);

/* [CFG]: out = y_u + w * (y_c - y_u), elementwise over nrows x N. */
int orc_cfg_combine(const float* y_c, const float* y_u, int64_t nrows, int64_t N, float w,
                    float* out);

/* [HQ] 2.1 single Hadamard: only the activations are rotated, so the
 * weights enter as H * W_int^T. v[n,k] = sum over k' in the B-block of k of
 * H[k mod B][k' mod B] * wc[n,k'], with H[i][j] = (-1)^popcount(i & j)
 * written out entry by entry (exact integers). */
int orc_hadamard_weight_int(const int8_t* wc, int64_t N, int64_t K, int32_t B, int32_t* v);

/* Exact int64 contraction of activation codes c [*, K] (rows listed) with
 * integer weights v [N, K]: acc[i,n] = sum_k c[row_i,k] * v[n,k]. */
int orc_gemm_int64(const int8_t* c, const int32_t* v, const int64_t* rows, int64_t nrows,
                   int64_t N, int64_t K, int64_t* acc);

/* [HQ] 2.1 + 2.2 (symmetric activations): y = fl(fl(fl(a * s) * sw[n]) * (1/B))
 * with a = acc rounded once to fp32 (nearest even). */
int orc_epilogue_single(const int64_t* acc, int64_t nrows, int64_t N, float s, const float* sw,
                        int32_t B, float* y);

/* [CFG] methodology (allocation strategy): weights fixed at w_bits, every
 * layer starts at 4-bit activations, layers are ranked by sensitivity per
 * bit operation, and promoted to 8-bit activations greedily while the
 * guided step's BOPs stay within the budget.
 *   macs[l]  : multiply-accumulates of layer l over the guided step (> 0)
 *   gain[l]  : sensitivity removed by promoting layer l (finite, >= 0)
 *   budget   : BOPs limit, >= the all-4-bit BOPs
 * BOPs of a layer = macs * w_bits * a_bits (exact int64). Equal ratios rank
 * by layer index. Out: a_bits[l] in {4, 8}, *bops = total BOPs. */
int orc_gamp_allocate(int32_t n, const int64_t* macs, const double* gain, int32_t w_bits,
                      int64_t budget, int32_t* a_bits, int64_t* bops);

/* bf16 bit patterns -> fp32 (exact). */
int orc_bf16_to_f32(const uint16_t* in, int64_t n, float* out);

#ifdef __cplusplus
}
#endif

#endif
