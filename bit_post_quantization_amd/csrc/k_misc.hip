// K0 (offline plan kernels) and K3 (standalone CFG combine).
//
// K0 follows the weight side of the method: optional block Walsh-Hadamard
// rotation of the weight rows (HQ-DM explainer 2.1 applied to both operands),
// symmetric absmax scales per output channel or per output segment
// (SegQuant explainer 2.A: each chunk of a segmented linear's output is
// quantized on its own), round-half-even codes, and the weight-side LSB
// truncation of TASQ (TASQ explainer, technical summary 2: a per-layer,
// per-step operating precision over one stored set of codes).
// For HQ-DM's single transform (activations only) the plan keeps H W_int^T
// as two int8 planes (k0_fwht_split).
// K3 is the guided prediction of the "Closing the Null Space" explainer,
// problem statement.
#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

// In-place rotation of W [N,K] as a flat stream of 4-float units.
template <int HB>
__global__ __launch_bounds__(256) void k0_rotate(float* W, int64_t nunits) {
  const int lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64;
  const int64_t idx = base + lane;
  float e[4] = {0.f, 0.f, 0.f, 0.f};
  float4* p = reinterpret_cast<float4*>(W);
  if (idx < nunits) {
    const float4 v = p[idx];
    e[0] = v.x;
    e[1] = v.y;
    e[2] = v.z;
    e[3] = v.w;
  }
  fwht_block<HB>(e, lane);
  if (idx < nunits) p[idx] = make_float4(e[0], e[1], e[2], e[3]);
}

// Bits of max |W[n,k]| over the columns [c0, c0 + cw) per row (one block per row).
__global__ __launch_bounds__(256) void k0_row_absmax(const float* W, int K, int c0, int cw,
                                                     uint32_t* rowmax) {
  const int64_t n = blockIdx.x;
  const float* row = W + n * K + c0;
  uint32_t m = 0;
  for (int k = threadIdx.x; k < cw; k += 256) {
    const uint32_t b = __float_as_uint(row[k]) & 0x7FFFFFFFu;
    m = b > m ? b : m;
  }
  m = wave_max_u32(m);
  __shared__ uint32_t sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) rowmax[n] = max(max(sm[0], sm[1]), max(sm[2], sm[3]));
}

// Per channel: s[n] = rowmax[n] / qw. Per segment: one block per segment,
// s = (max over its rows) / qw written to every row of the segment.
__global__ __launch_bounds__(256) void k0_scales_channel(const uint32_t* rowmax, int N, float qw,
                                                         float* sw) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n < N) sw[n] = __uint_as_float(rowmax[n]) / qw;
}

__global__ __launch_bounds__(256) void k0_scales_segment(const uint32_t* rowmax, const int32_t* seg,
                                                         float qw, float* sw) {
  const int lo = seg[blockIdx.x], hi = seg[blockIdx.x + 1];
  uint32_t m = 0;
  for (int n = lo + threadIdx.x; n < hi; n += 256) m = rowmax[n] > m ? rowmax[n] : m;
  m = wave_max_u32(m);
  __shared__ uint32_t sm[4];
  __shared__ float s;
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) s = __uint_as_float(max(max(sm[0], sm[1]), max(sm[2], sm[3]))) / qw;
  __syncthreads();
  for (int n = lo + threadIdx.x; n < hi; n += 256) sw[n] = s;
}

__device__ __forceinline__ int quant_sym(float v, float s, float q) {
  float r = rintf(v / s);
  r = fminf(fmaxf(r, -q), q);
  return s > 0.0f ? (int)r : 0;
}

// Codes of 4 consecutive weights of one row per thread, over the columns
// [c0, c0 + cw) of every row (K, c0, cw multiples of 4), one int8 per code
// for both widths (4-bit codes lie in [-7, 7]).
__global__ __launch_bounds__(256) void k0_quant_w(const float* W, const float* sw, int K, int c0,
                                                  int cw, int64_t nunits, float qw,
                                                  uint8_t* out) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= nunits) return;
  const int64_t n = (u * 4) / cw;
  const int64_t e = n * K + c0 + (u * 4 - n * cw);  // first element of the unit
  const float s = sw[n];
  const float4 v = *reinterpret_cast<const float4*>(W + e);
  const int q0 = quant_sym(v.x, s, qw), q1 = quant_sym(v.y, s, qw);
  const int q2 = quant_sym(v.z, s, qw), q3 = quant_sym(v.w, s, qw);
  *reinterpret_cast<uint32_t*>(out + e) =
      (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) | ((uint32_t)(q2 & 0xFF) << 16) |
      ((uint32_t)(q3 & 0xFF) << 24);
}

// TASQ on the weight side: clear the k low bits of every code's magnitude,
// sign kept (keep = ~(2^k - 1)), 16 codes per thread; the first N threads
// also copy the weight scales, so a rewrite is one launch.
__device__ __forceinline__ uint32_t truncate4(uint32_t v, int32_t keep) {
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = (int)(int8_t)((v >> (8 * i)) & 0xFFu);
    const int t = c >= 0 ? (c & keep) : -((-c) & keep);
    r |= ((uint32_t)t & 0xFFu) << (8 * i);
  }
  return r;
}

__global__ __launch_bounds__(256) void k0_truncate_w(const uint4* in, int64_t n16, int32_t keep,
                                                     uint4* out, const float* sw_in, float* sw_out,
                                                     int nsw) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u < nsw) sw_out[u] = sw_in[u];
  if (u >= n16) return;
  const uint4 v = in[u];
  out[u] = make_uint4(truncate4(v.x, keep), truncate4(v.y, keep), truncate4(v.z, keep),
                      truncate4(v.w, keep));
}

// 4-bit weight codes stored two per byte (the layout of the packed
// activation codes: element 2i in the low nibble of byte i, element 2i + 1
// in the high nibble); 16 codes per thread.
__global__ __launch_bounds__(256) void k0_pack4(const uint4* in, int64_t n16, uint2* out) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= n16) return;
  const uint4 v = in[u];
  auto pk = [](uint32_t w) {  // 4 codes -> 2 bytes
    return (w & 0xFu) | ((w >> 4) & 0xF0u) | ((w >> 8) & 0xF00u) | ((w >> 12) & 0xF000u);
  };
  out[u] = make_uint2(pk(v.x) | (pk(v.y) << 16), pk(v.z) | (pk(v.w) << 16));
}

// The inverse: int8 codes (sign-extended nibbles), the k low magnitude bits
// cleared (keep = ~(2^k - 1)); 16 codes per thread.
__global__ __launch_bounds__(256) void k0_unpack4(const uint2* in, int64_t n16, int32_t keep,
                                                  uint4* out) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= n16) return;
  const uint2 v = in[u];
  auto up = [keep](uint32_t h) {  // 2 packed bytes -> 4 codes
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = (int)(int8_t)(uint8_t)(((h >> (4 * i)) & 0xFu) << 4) >> 4;
      const int t = c >= 0 ? (c & keep) : -((-c) & keep);
      r |= ((uint32_t)t & 0xFFu) << (8 * i);
    }
    return r;
  };
  out[u] = make_uint4(up(v.x & 0xFFFFu), up(v.x >> 16), up(v.y & 0xFFFFu), up(v.y >> 16));
}

// Single-Hadamard weights ([HQ-DM explainer 2.1: only the activations are
// rotated]): V = H W_int^T row by row, exact (integers below 2^24 in fp32),
// split into two int8 planes V = 128 * hi + lo with lo in [0, 127] and hi in
// [-127, 127]. Output rows: for output channels 16g .. 16g+15, rows 32g ..
// 32g+15 hold hi and rows 32g+16 .. 32g+31 hold lo, so a GEMM tile sees each
// channel's two planes in adjacent 16-row fragments. Four codes per thread.
template <int HB>
__global__ __launch_bounds__(256) void k0_fwht_split(const uint32_t* codes, int K, int64_t nunits,
                                                     uint8_t* out) {
  const int lane = threadIdx.x & 63;
  const int64_t idx = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64 + lane;
  float e[4] = {0.f, 0.f, 0.f, 0.f};
  if (idx < nunits) {
    const uint32_t v = codes[idx];
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = (float)(int)(int8_t)((v >> (8 * i)) & 0xFFu);
  }
  fwht_block<HB>(e, lane);
  if (idx >= nunits) return;
  const int64_t n = (idx * 4) / K;
  const int64_t k = idx * 4 - n * K;
  uint32_t hi = 0, lo = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = (int)e[i];
    hi |= ((uint32_t)(v >> 7) & 0xFFu) << (8 * i);
    lo |= ((uint32_t)(v & 127)) << (8 * i);
  }
  const int64_t row = 32 * (n >> 4) + (n & 15);
  *reinterpret_cast<uint32_t*>(out + row * K + k) = hi;
  *reinterpret_cast<uint32_t*>(out + (row + 16) * K + k) = lo;
}

// K3: out = yu + w * (yc - yu); yc = Y[e], yu = Y[e + half].
__global__ __launch_bounds__(256) void k3_cfg(const float* Y, int64_t half, float w, float* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < half; e += stride) {
    const float yc = Y[e];
    const float yu = Y[e + half];
    const float d = __fsub_rn(yc, yu);
    const float t = __fmul_rn(w, d);
    out[e] = __fadd_rn(yu, t);
  }
}

int blocks_for(int64_t n, int64_t per) {
  int64_t b = (n + per - 1) / per;
  return (int)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_rotate_rows(float* W, int64_t nunits, int hb, hipStream_t s) {
  const dim3 grid(blocks_for(nunits, 256));
  switch (hb) {
    case 4: hipLaunchKernelGGL((k0_rotate<4>), grid, dim3(256), 0, s, W, nunits); break;
    case 8: hipLaunchKernelGGL((k0_rotate<8>), grid, dim3(256), 0, s, W, nunits); break;
    case 16: hipLaunchKernelGGL((k0_rotate<16>), grid, dim3(256), 0, s, W, nunits); break;
    case 32: hipLaunchKernelGGL((k0_rotate<32>), grid, dim3(256), 0, s, W, nunits); break;
    case 64: hipLaunchKernelGGL((k0_rotate<64>), grid, dim3(256), 0, s, W, nunits); break;
    case 128: hipLaunchKernelGGL((k0_rotate<128>), grid, dim3(256), 0, s, W, nunits); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_row_absmax(const float* W, int N, int K, int c0, int cw, uint32_t* rowmax,
                             hipStream_t s) {
  hipLaunchKernelGGL(k0_row_absmax, dim3(N), dim3(256), 0, s, W, K, c0, cw, rowmax);
  return hipGetLastError();
}

hipError_t launch_weight_scales(const uint32_t* rowmax, int N, int mode, const int32_t* seg,
                                int nseg, float qw, float* sw, hipStream_t s) {
  if (mode == 2) {
    hipLaunchKernelGGL(k0_scales_channel, dim3(blocks_for(N, 256)), dim3(256), 0, s, rowmax, N,
                       qw, sw);
  } else {
    hipLaunchKernelGGL(k0_scales_segment, dim3(nseg), dim3(256), 0, s, rowmax, seg, qw, sw);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_weights(const float* W, const float* sw, int N, int K, int c0, int cw,
                                   float qw, uint8_t* out, hipStream_t s) {
  if (K % 4 || c0 % 4 || cw % 4 || cw <= 0 || c0 + cw > K) return hipErrorInvalidValue;
  const int64_t nunits = (int64_t)N * cw / 4;
  hipLaunchKernelGGL(k0_quant_w, dim3(blocks_for(nunits, 256)), dim3(256), 0, s, W, sw, K, c0, cw,
                     nunits, qw, out);
  return hipGetLastError();
}

hipError_t launch_truncate_weights(const uint8_t* in, int64_t nbytes, int k, uint8_t* out,
                                   const float* sw_in, float* sw_out, int nsw, hipStream_t s) {
  if (nbytes % 16 != 0 || k < 0 || k > 7) return hipErrorInvalidValue;
  const int64_t n16 = nbytes / 16;
  const int32_t keep = ~((1 << k) - 1);
  const int64_t threads = n16 > nsw ? n16 : nsw;
  hipLaunchKernelGGL(k0_truncate_w, dim3(blocks_for(threads, 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(in), n16, keep, reinterpret_cast<uint4*>(out),
                     sw_in, sw_out, nsw);
  return hipGetLastError();
}

hipError_t launch_pack4(const uint8_t* codes, int64_t n, uint8_t* packed, hipStream_t s) {
  if (n % 16 != 0) return hipErrorInvalidValue;
  const int64_t n16 = n / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(k0_pack4, dim3(blocks_for(n16, 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(codes), n16, reinterpret_cast<uint2*>(packed));
  return hipGetLastError();
}

hipError_t launch_unpack4(const uint8_t* packed, int64_t n, int k, uint8_t* codes, hipStream_t s) {
  if (n % 16 != 0 || k < 0 || k > 3) return hipErrorInvalidValue;
  const int64_t n16 = n / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(k0_unpack4, dim3(blocks_for(n16, 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint2*>(packed), n16, (int32_t)~((1 << k) - 1),
                     reinterpret_cast<uint4*>(codes));
  return hipGetLastError();
}

hipError_t launch_fwht_split(const uint8_t* codes, int N, int K, int hb, uint8_t* out,
                             hipStream_t s) {
  if (K % 4 != 0 || K % hb != 0) return hipErrorInvalidValue;
  const int64_t nunits = (int64_t)N * K / 4;
  const dim3 grid(blocks_for(nunits, 256));
  const uint32_t* in = reinterpret_cast<const uint32_t*>(codes);
  switch (hb) {
    case 4: hipLaunchKernelGGL((k0_fwht_split<4>), grid, dim3(256), 0, s, in, K, nunits, out); break;
    case 8: hipLaunchKernelGGL((k0_fwht_split<8>), grid, dim3(256), 0, s, in, K, nunits, out); break;
    case 16: hipLaunchKernelGGL((k0_fwht_split<16>), grid, dim3(256), 0, s, in, K, nunits, out); break;
    case 32: hipLaunchKernelGGL((k0_fwht_split<32>), grid, dim3(256), 0, s, in, K, nunits, out); break;
    case 64: hipLaunchKernelGGL((k0_fwht_split<64>), grid, dim3(256), 0, s, in, K, nunits, out); break;
    case 128: hipLaunchKernelGGL((k0_fwht_split<128>), grid, dim3(256), 0, s, in, K, nunits, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cfg_combine(const float* Y, int64_t half, float w, float* out, hipStream_t s) {
  int64_t b = (half + 255) / 256;
  if (b > 8192) b = 8192;
  if (b < 1) b = 1;
  hipLaunchKernelGGL(k3_cfg, dim3((int)b), dim3(256), 0, s, Y, half, w, out);
  return hipGetLastError();
}

}  // namespace ql
