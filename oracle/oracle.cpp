// CPU oracle for the quantized linear layer of a diffusion transformer.
//
// TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
// benchmark's CPU-baseline leg. Never part of the product path. Shares no
// code with the GPU library.
//
// Plain single-threaded C++; fp32 arithmetic with round-to-nearest-even,
// correctly rounded division, no contraction into fused multiply-add
// (compiled with -ffp-contract=off), no fast-math, no intrinsics, no threads.
// Each function states the passage of the pages it follows; oracle.h lists
// the pages.
#include "oracle.h"

#include <cfenv>
#include <cmath>
#include <vector>
#include <cstdint>

namespace {

bool is_pow2(int64_t b) { return b > 0 && (b & (b - 1)) == 0; }

int32_t qmax_for_bits(int32_t bits) { return (1 << (bits - 1)) - 1; }

bool valid_bits(int32_t bits) { return bits == 4 || bits == 8; }

// Round to nearest, ties to even (the default IEEE rounding mode).
float round_even(float q) { return std::nearbyint(q); }

}  // namespace

extern "C" {

// [HQ] 2.1: the rotation is a block-diagonal Hadamard matrix built from
// standard Hadamard matrices. Here: the unnormalised Sylvester matrix of order
// B, H[i][j] = (-1)^popcount(i & j), applied as the fast transform. The stage
// order (butterfly distance h = 1, 2, 4, ..., B/2) fixes the fp32 rounding, so
// it is part of the definition. Each butterfly maps (a, b) to (a + b, a - b).
int orc_fwht_block(float* v, int32_t B) {
  if (!is_pow2(B)) return ORC_EARG;
  for (int32_t h = 1; h < B; h *= 2) {
    for (int32_t i = 0; i < B; i += 2 * h) {
      for (int32_t j = i; j < i + h; ++j) {
        const float a = v[j];
        const float b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
  return ORC_OK;
}

// [HQ] 2.1: rotate every row of x [rows, K] by diag(H_B, ..., H_B).
int orc_rotate_rows(float* x, int64_t rows, int64_t K, int32_t B) {
  if (!is_pow2(B) || K % B != 0 || rows < 0) return ORC_EARG;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < K; j += B) orc_fwht_block(x + r * K + j, B);
  return ORC_OK;
}

// [SQ] 2.B DualScale: one scale for the non-negative region and one for the
// negative region of the activations. Per tensor: s+ = max(x)/qa and
// s- = |min(x)|/qa with qa = 2^(bits-1) - 1; an empty region gets scale 0.
// [HQ] 2 uses symmetric activation quantization: one scale max(|x|)/qa for
// both regions. [CFG] methodology: the range is taken over both branches, so
// the reduction runs over all n values (conditional and unconditional rows).
int orc_act_scales(const float* x, int64_t n, int32_t a_bits, int32_t mode, float* s) {
  if (!valid_bits(a_bits) || n < 0) return ORC_EARG;
  if (mode != ORC_ASCALE_DUAL && mode != ORC_ASCALE_SYMMETRIC) return ORC_EARG;
  float mx = +0.0f;  // max(+0, max x)
  float mn = +0.0f;  // max(+0, -min x)
  for (int64_t i = 0; i < n; ++i) {
    const float v = x[i];
    if (!std::isfinite(v)) return ORC_ENONFINITE;
    if (v > mx) mx = v;
    if (-v > mn) mn = -v;
  }
  const float qa = (float)qmax_for_bits(a_bits);
  if (mode == ORC_ASCALE_DUAL) {
    s[0] = mx / qa;
    s[1] = mn / qa;
  } else {
    const float m = mx > mn ? mx : mn;
    s[0] = m / qa;
    s[1] = s[0];
  }
  return ORC_OK;
}

// [SQ] 2.B: the value goes to the plane of its sign. Non-negative values
// (zero and -0 included) use s+, codes in [0, qa]; negative values use s-,
// codes in [-qa, 0]. Code = round-half-even(v / s) clamped to the plane's
// range; a zero scale gives code 0.
int32_t orc_quant_value(float v, float s_plus, float s_minus, int32_t qa) {
  if (v >= 0.0f) {
    if (!(s_plus > 0.0f)) return 0;
    float r = round_even(v / s_plus);
    if (r > (float)qa) r = (float)qa;
    if (r < 0.0f) r = 0.0f;
    return (int32_t)r;
  }
  if (!(s_minus > 0.0f)) return 0;
  float r = round_even(v / s_minus);
  if (r < -(float)qa) r = -(float)qa;
  if (r > 0.0f) r = 0.0f;
  return (int32_t)r;
}

// [TQ] 2: the operating code at a (step, layer) drops k least significant
// bits of the stored code (bit-plane truncation / right shift). Applied to
// the magnitude, sign kept: |c'| = |c| with its k low bits cleared.
int32_t orc_truncate_lsb(int32_t c, int32_t k) {
  const int32_t keep = ~((1 << k) - 1);
  if (c >= 0) return c & keep;
  return -((-c) & keep);
}

// [TQ] 2: one stored weight buffer; the layer's precision at a stage is set
// by how many low bits its mask drops from every stored code.
int orc_truncate_codes(const int8_t* in, int64_t n, int32_t w_bits, int32_t k, int8_t* out) {
  if (!valid_bits(w_bits) || k < 0 || k >= w_bits || n < 0) return ORC_EARG;
  const int32_t qw = qmax_for_bits(w_bits);
  for (int64_t i = 0; i < n; ++i) {
    if (in[i] < -qw || in[i] > qw) return ORC_EARG;
    out[i] = (int8_t)orc_truncate_lsb(in[i], k);
  }
  return ORC_OK;
}

int orc_quantize_act(const float* x, int64_t n, const float* s, int32_t a_bits,
                     int32_t lsb_k, int8_t* codes) {
  if (!valid_bits(a_bits) || lsb_k < 0 || lsb_k >= a_bits || n < 0) return ORC_EARG;
  const int32_t qa = qmax_for_bits(a_bits);
  for (int64_t i = 0; i < n; ++i) {
    if (!std::isfinite(x[i])) return ORC_ENONFINITE;
    int32_t c = orc_quant_value(x[i], s[0], s[1], qa);
    c = orc_truncate_lsb(c, lsb_k);
    codes[i] = (int8_t)c;
  }
  return ORC_OK;
}

int orc_pack_int4(const int8_t* codes, int64_t rows, int64_t K, uint8_t* out) {
  if (K % 2 != 0 || rows < 0) return ORC_EARG;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t j = 0; j < K / 2; ++j) {
      const int32_t a = codes[r * K + 2 * j];
      const int32_t b = codes[r * K + 2 * j + 1];
      if (a < -8 || a > 7 || b < -8 || b > 7) return ORC_EARG;
      out[r * (K / 2) + j] = (uint8_t)((a & 0xF) | ((b & 0xF) << 4));
    }
  }
  return ORC_OK;
}

int orc_unpack_int4(const uint8_t* packed, int64_t rows, int64_t K, int8_t* out) {
  if (K % 2 != 0 || rows < 0) return ORC_EARG;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t j = 0; j < K / 2; ++j) {
      const int32_t byte = packed[r * (K / 2) + j];
      int32_t lo = byte & 0xF;
      int32_t hi = (byte >> 4) & 0xF;
      if (lo >= 8) lo -= 16;
      if (hi >= 8) hi -= 16;
      out[r * K + 2 * j] = (int8_t)lo;
      out[r * K + 2 * j + 1] = (int8_t)hi;
    }
  }
  return ORC_OK;
}

// [SQ] 2.A SegLinear output segmentation: when a linear's output is chunked,
// the weight rows of each chunk are quantized on their own. A segment's scale
// is the symmetric absmax over all its rows and columns divided by qw;
// per-tensor is one segment; per-channel gives each row its own scale.
int orc_weight_scales(const float* w, int64_t N, int64_t K, int32_t w_bits, int32_t mode,
                      int32_t nseg, const int32_t* seg, float* sw) {
  if (!valid_bits(w_bits) || N <= 0 || K <= 0) return ORC_EARG;
  const float qw = (float)qmax_for_bits(w_bits);
  for (int64_t i = 0; i < N * K; ++i)
    if (!std::isfinite(w[i])) return ORC_ENONFINITE;
  if (mode == ORC_WSCALE_CHANNEL) {
    for (int64_t n = 0; n < N; ++n) {
      float m = +0.0f;
      for (int64_t k = 0; k < K; ++k) {
        const float a = std::fabs(w[n * K + k]);
        if (a > m) m = a;
      }
      sw[n] = m / qw;
    }
    return ORC_OK;
  }
  int32_t one[2] = {0, (int32_t)N};
  if (mode == ORC_WSCALE_TENSOR || seg == nullptr) {
    nseg = 1;
    seg = one;
  } else if (mode != ORC_WSCALE_SEGMENT) {
    return ORC_EARG;
  }
  if (nseg < 1 || seg[0] != 0 || seg[nseg] != N) return ORC_EARG;
  for (int32_t g = 0; g < nseg; ++g)
    if (seg[g + 1] <= seg[g]) return ORC_EARG;
  for (int32_t g = 0; g < nseg; ++g) {
    float m = +0.0f;
    for (int64_t n = seg[g]; n < seg[g + 1]; ++n)
      for (int64_t k = 0; k < K; ++k) {
        const float a = std::fabs(w[n * K + k]);
        if (a > m) m = a;
      }
    const float s = m / qw;
    for (int64_t n = seg[g]; n < seg[g + 1]; ++n) sw[n] = s;
  }
  return ORC_OK;
}

// Symmetric weight codes: round-half-even(w / s_w[n]) clamped to [-qw, qw];
// a zero scale gives code 0.
int orc_quantize_weight(const float* w, int64_t N, int64_t K, const float* sw,
                        int32_t w_bits, int8_t* wc) {
  if (!valid_bits(w_bits) || N <= 0 || K <= 0) return ORC_EARG;
  const float qw = (float)qmax_for_bits(w_bits);
  for (int64_t n = 0; n < N; ++n) {
    const float s = sw[n];
    for (int64_t k = 0; k < K; ++k) {
      const float v = w[n * K + k];
      if (!std::isfinite(v)) return ORC_ENONFINITE;
      float r = 0.0f;
      if (s > 0.0f) {
        r = round_even(v / s);
        if (r > qw) r = qw;
        if (r < -qw) r = -qw;
      }
      wc[n * K + k] = (int8_t)(int32_t)r;
    }
  }
  return ORC_OK;
}

// [SQ] 2.B: X is split into its non-negative part and its negative part and
// each is multiplied by the weight codes (two matrix products). Exact integer
// sums; any value outside int32 is reported instead of wrapped.
int orc_gemm_dual(const int8_t* c, const int8_t* wc, const int64_t* rows, int64_t nrows,
                  int64_t N, int64_t K, int32_t* accp, int32_t* accn) {
  if (nrows < 0 || N <= 0 || K <= 0) return ORC_EARG;
  for (int64_t i = 0; i < nrows; ++i) {
    const int8_t* a = c + rows[i] * K;
    for (int64_t n = 0; n < N; ++n) {
      const int8_t* b = wc + n * K;
      int64_t sp = 0;
      int64_t sn = 0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t av = a[k];
        const int64_t bv = b[k];
        if (av > 0)
          sp += av * bv;
        else
          sn += av * bv;
      }
      if (sp > INT32_MAX || sp < INT32_MIN || sn > INT32_MAX || sn < INT32_MIN)
        return ORC_EOVERFLOW;
      accp[i * N + n] = (int32_t)sp;
      accn[i * N + n] = (int32_t)sn;
    }
  }
  return ORC_OK;
}

// [SQ] 2.B: the two products are rescaled by their own activation scale and
// summed in the epilogue, then multiplied by the weight scale of the output
// channel. [HQ] 2.1: the Hadamard normalisation is a power of two folded
// into the float scales; with both operands rotated by unnormalised H_B it is
// 1/B (exact). Fixed order, no fused multiply-add.
int orc_epilogue(const int32_t* accp, const int32_t* accn, int64_t nrows, int64_t N,
                 const float* s, const float* sw, int32_t B, int32_t mode, float* y) {
  if (nrows < 0 || N <= 0 || (B != 0 && !is_pow2(B))) return ORC_EARG;
  if (mode != ORC_ASCALE_DUAL && mode != ORC_ASCALE_SYMMETRIC) return ORC_EARG;
  const float invb = B > 0 ? 1.0f / (float)B : 1.0f;
  for (int64_t i = 0; i < nrows; ++i) {
    for (int64_t n = 0; n < N; ++n) {
      const int64_t e = i * N + n;
      float v;
      if (mode == ORC_ASCALE_DUAL) {
        const float tp = (float)accp[e] * s[0];
        const float tn = (float)accn[e] * s[1];
        v = (tp + tn) * sw[n];
      } else {
        const int64_t a = (int64_t)accp[e] + (int64_t)accn[e];
        if (a > INT32_MAX || a < INT32_MIN) return ORC_EOVERFLOW;
        v = ((float)(int32_t)a * s[0]) * sw[n];
      }
      if (B > 0) v = v * invb;
      y[e] = v;
    }
  }
  return ORC_OK;
}

// [CFG] problem statement: guided prediction = unconditional output plus the
// guidance weight times (conditional - unconditional). Evaluated as
// d = yc - yu; t = w * d; out = yu + t.
int orc_cfg_combine(const float* y_c, const float* y_u, int64_t nrows, int64_t N, float w,
                    float* out) {
  if (nrows < 0 || N < 0) return ORC_EARG;
  for (int64_t e = 0; e < nrows * N; ++e) {
    const float d = y_c[e] - y_u[e];
    const float t = w * d;
    out[e] = y_u[e] + t;
  }
  return ORC_OK;
}

// [HQ] 2.1, single transform: X W^T = (1/B) (X H)(H W^T) since H H = B I.
// The weight side is kept as the integer matrix H W_int^T, from the entries
// of the Sylvester matrix directly (no fast transform).
int orc_hadamard_weight_int(const int8_t* wc, int64_t N, int64_t K, int32_t B, int32_t* v) {
  if (!is_pow2(B) || K % B != 0 || N < 0) return ORC_EARG;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const int64_t blk = k - k % B;
      int64_t sum = 0;
      for (int32_t j = 0; j < B; ++j) {
        const int sign = (__builtin_popcount((unsigned)((k % B) & j)) & 1) ? -1 : 1;
        sum += sign * (int64_t)wc[n * K + blk + j];
      }
      v[n * K + k] = (int32_t)sum;
    }
  return ORC_OK;
}

int orc_gemm_int64(const int8_t* c, const int32_t* v, const int64_t* rows, int64_t nrows,
                   int64_t N, int64_t K, int64_t* acc) {
  if (nrows < 0 || N < 0 || K < 0) return ORC_EARG;
  for (int64_t i = 0; i < nrows; ++i)
    for (int64_t n = 0; n < N; ++n) {
      int64_t sum = 0;
      for (int64_t k = 0; k < K; ++k) sum += (int64_t)c[rows[i] * K + k] * (int64_t)v[n * K + k];
      acc[i * N + n] = sum;
    }
  return ORC_OK;
}

int orc_epilogue_single(const int64_t* acc, int64_t nrows, int64_t N, float s, const float* sw,
                        int32_t B, float* y) {
  if (nrows < 0 || N <= 0 || !is_pow2(B)) return ORC_EARG;
  const float inv_b = 1.0f / (float)B;
  for (int64_t i = 0; i < nrows; ++i)
    for (int64_t n = 0; n < N; ++n) {
      const float a = (float)acc[i * N + n];
      const float t = a * s;
      const float u = t * sw[n];
      y[i * N + n] = u * inv_b;
    }
  return ORC_OK;
}

// [CFG] methodology, allocation strategy: a greedy knapsack over layers,
// items ranked by sensitivity per BOP, each promotion from 4 to 8 activation
// bits costing macs * w_bits * 4 BOPs. Selection by repeated scans for the
// best remaining item (first index wins a tie).
int orc_gamp_allocate(int32_t n, const int64_t* macs, const double* gain, int32_t w_bits,
                      int64_t budget, int32_t* a_bits, int64_t* bops) {
  if (n < 1 || !valid_bits(w_bits)) return ORC_EARG;
  int64_t total = 0;
  for (int32_t l = 0; l < n; ++l) {
    if (macs[l] <= 0 || !std::isfinite(gain[l]) || gain[l] < 0.0) return ORC_EARG;
    a_bits[l] = 4;
    total += macs[l] * w_bits * 4;
  }
  if (budget < total) return ORC_EARG;
  std::vector<bool> seen(n, false);
  for (int32_t round = 0; round < n; ++round) {
    int32_t best = -1;
    double best_ratio = 0.0;
    for (int32_t l = 0; l < n; ++l) {
      if (seen[l]) continue;
      const double ratio = gain[l] / (double)(macs[l] * w_bits * 4);
      if (best < 0 || ratio > best_ratio) {
        best = l;
        best_ratio = ratio;
      }
    }
    seen[best] = true;
    const int64_t cost = macs[best] * w_bits * 4;
    if (total + cost <= budget) {
      a_bits[best] = 8;
      total += cost;
    }
  }
  *bops = total;
  return ORC_OK;
}

int orc_bf16_to_f32(const uint16_t* in, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t b = (uint32_t)in[i] << 16;
    float f;
    static_assert(sizeof(f) == sizeof(b), "fp32 size");
    __builtin_memcpy(&f, &b, sizeof(f));
    out[i] = f;
  }
  return ORC_OK;
}

}  // extern "C"
