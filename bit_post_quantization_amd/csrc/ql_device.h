// Device-side building blocks shared by the gfx950 kernels of libqlinear.
// Written for CDNA4 wave64; no other target is supported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

constexpr int kWave = 64;

// ------------------------------------------------------------ cross-lane ----

// Exchange with lane ^ m (m < 32) inside each 32-lane half: ds_swizzle in
// bit-mask mode (and_mask 0x1f, or_mask 0, xor_mask m); no LDS traffic.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  static_assert(M > 0 && M < 32, "swizzle xor mask");
  constexpr int pat = 0x1f | (M << 10);
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), pat));
}

template <int M>
__device__ __forceinline__ uint32_t xor_lane_u(uint32_t v) {
  constexpr int pat = 0x1f | (M << 10);
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, pat);
}

// Maximum over the 64 lanes of a wave (result valid in every lane).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, xor_lane_u<1>(v));
  v = max(v, xor_lane_u<2>(v));
  v = max(v, xor_lane_u<4>(v));
  v = max(v, xor_lane_u<8>(v));
  v = max(v, xor_lane_u<16>(v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  return a > b ? a : b;
}

// ------------------------------------------------- Walsh-Hadamard (FWHT) ----
// Four consecutive elements of a block sit in one lane (one 128-bit load);
// a block of B elements spans B/4 consecutive lanes of a 32-lane half.
// Stages run in the order h = 1, 2, 4, ..., B/2 and every butterfly maps
// (a, b) at positions (j, j+h) to (a + b, a - b): the same fp32 operations,
// in the same stage order, as the Sylvester-order fast transform, so the
// result is bit-for-bit that transform.

__device__ __forceinline__ void fwht_in_lane(float& e0, float& e1, float& e2, float& e3) {
  // h = 1
  float a0 = e0 + e1, a1 = e0 - e1, a2 = e2 + e3, a3 = e2 - e3;
  // h = 2
  e0 = a0 + a2;
  e2 = a0 - a2;
  e1 = a1 + a3;
  e3 = a1 - a3;
}

// Cross-lane stage h = 4L. The lower lane holds a (position j) and takes
// a + b; the upper lane holds b (position j + h) and takes a - b. Both are
// one fused multiply-add o + sg * e with sg = +1 or -1 per lane: sg * e is
// exact, so the single rounding gives exactly the correctly rounded sum or
// difference (signed zeros included), in one instruction instead of an add,
// a subtract and a select.
template <int L>  // lane distance L = h / 4
__device__ __forceinline__ void fwht_cross_stage(float& e, float sg) {
  const float o = xor_lane<L>(e);
  e = __builtin_fmaf(e, sg, o);
}

// Sign of the upper lanes of stage h = 4L.
template <int L>
__device__ __forceinline__ float fwht_sign(int lane) {
  return (lane & L) ? -1.0f : 1.0f;
}

template <int B>
__device__ __forceinline__ void fwht_block(float (&e)[4], int lane) {
  static_assert(B >= 4 && B <= 128 && (B & (B - 1)) == 0, "block size");
  fwht_in_lane(e[0], e[1], e[2], e[3]);
  if constexpr (B >= 8) {
    const float sg = fwht_sign<1>(lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) fwht_cross_stage<1>(e[i], sg);
  }
  if constexpr (B >= 16) {
    const float sg = fwht_sign<2>(lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) fwht_cross_stage<2>(e[i], sg);
  }
  if constexpr (B >= 32) {
    const float sg = fwht_sign<4>(lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) fwht_cross_stage<4>(e[i], sg);
  }
  if constexpr (B >= 64) {
    const float sg = fwht_sign<8>(lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) fwht_cross_stage<8>(e[i], sg);
  }
  if constexpr (B >= 128) {
    const float sg = fwht_sign<16>(lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) fwht_cross_stage<16>(e[i], sg);
  }
}

// ---------------------------------------------------------- quantization ----

// Code of one value under DualScale: the non-negative region (including -0)
// uses s+ and codes [0, qa]; the negative region uses s- and codes [-qa, 0].
// round-half-even of an IEEE correctly rounded fp32 quotient; zero scale -> 0.
__device__ __forceinline__ int quant_dual(float v, float sp, float sn, float qa) {
  const bool pos = v >= 0.0f;
  const float s = pos ? sp : sn;
  float r = rintf(v / s);
  const float lo = pos ? 0.0f : -qa;
  const float hi = pos ? qa : 0.0f;
  r = fminf(fmaxf(r, lo), hi);
  return (s > 0.0f) ? (int)r : 0;
}

// Clear the k low bits of the code's magnitude, keeping its sign.
__device__ __forceinline__ int truncate_lsb(int c, int keep_mask) {
  const int m = c < 0 ? -c : c;
  const int t = m & keep_mask;
  return c < 0 ? -t : t;
}

// 0xFF in every byte of c that is negative as int8, 0x00 elsewhere.
// v_perm_b32 selectors 8..11 replicate the sign bit of bytes 1, 3, 5, 7 of
// the 64-bit pair {src0, src1}; with src0 = c and src1 = c << 8 those are the
// sign bits of c's bytes 0, 2, 1, 3. Two full-rate instructions.
__device__ __forceinline__ uint32_t neg_byte_mask(uint32_t c) {
  return __builtin_amdgcn_perm(c, c << 8, 0x0B090A08u);
}

// Non-negative plane of four packed int8 codes (negative bytes zeroed).
__device__ __forceinline__ uint32_t pos_plane(uint32_t c) { return c & ~neg_byte_mask(c); }

// Polarity planes of four packed int8 codes: bytes < 0 go to `neg`, the
// others to `pos` (the planes have disjoint support, so pos + neg = codes).
__device__ __forceinline__ void split_polarity(uint32_t c, uint32_t& pos, uint32_t& neg) {
  const uint32_t m = neg_byte_mask(c);
  pos = c & ~m;
  neg = c & m;
}

// Unpack 8 packed 4-bit codes (element 2j in the low nibble of byte j) into
// two dwords of int8, natural element order, each code multiplied by 16
// (the nibble placed in the high half of its byte, exact in int8).
__device__ __forceinline__ void unpack4_x16(uint32_t p, uint32_t& d0, uint32_t& d1) {
  const uint32_t lo = (p << 4) & 0xF0F0F0F0u;  // even elements, bytes 0..3
  const uint32_t hi = p & 0xF0F0F0F0u;         // odd elements
  // d0 = [lo.b0, hi.b0, lo.b1, hi.b1], d1 = [lo.b2, hi.b2, lo.b3, hi.b3]
  // v_perm_b32: selector bytes 0-3 pick from src1 (lo), 4-7 from src0 (hi).
  d0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  d1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// TASQ's truncation of four int8 codes (|c| <= 127): the kk low bits of each
// magnitude cleared, sign kept, i.e. rounding toward zero to a multiple of
// 2^kk. A negative byte gets 2^kk - 1 added before its low bits are
// cleared; the add runs on the low 7 bits (at most 127 + 127, so no carry
// leaves a byte) and the sign bit is put back by exclusive or. The bias
// comes from a byte table: v_perm_b32 with selector 0 or 1 per byte (the
// byte's sign bit) picks byte 0 (= 0) or byte 1 (= 2^kk - 1) of lut. Five
// VALU instructions.
// lut = (2^kk - 1) << 8; keep = the byte ~(2^kk - 1) in every byte.
__device__ __forceinline__ uint32_t trunc_mag4(uint32_t b, uint32_t lut, uint32_t keep) {
  const uint32_t h = b & 0x80808080u;
  const uint32_t bias = __builtin_amdgcn_perm(0u, lut, h >> 7);
  uint32_t s;
  asm("v_xad_u32 %0, %1, %2, %3" : "=v"(s) : "v"(b), "v"(h), "v"(bias));  // (b ^ h) + bias
  return (s ^ h) & keep;
}

// Nine floats at p, p + 16, ..., p + 128 (LDS), read in one asm block that
// waits for them itself. The scale ring is written by DMA, and the compiler,
// unable to tell which DMA wrote it, would otherwise wait for every load in
// flight before a plain LDS read of it; the ring entry read here was written
// tiles earlier and published by the step barriers since.
__device__ __forceinline__ void lds_read9_stride16(const float* p, float* v) {
  const uint32_t a = (uint32_t)reinterpret_cast<uintptr_t>(p);  // LDS offset of a shared pointer
  asm volatile(
      "ds_read_b32 %0, %9\n\t"
      "ds_read_b32 %1, %9 offset:64\n\t"
      "ds_read_b32 %2, %9 offset:128\n\t"
      "ds_read_b32 %3, %9 offset:192\n\t"
      "ds_read_b32 %4, %9 offset:256\n\t"
      "ds_read_b32 %5, %9 offset:320\n\t"
      "ds_read_b32 %6, %9 offset:384\n\t"
      "ds_read_b32 %7, %9 offset:448\n\t"
      "ds_read_b32 %8, %9 offset:512\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7]), "=&v"(v[8])
      : "v"(a)
      : "memory");
}

}  // namespace ql
