// K1: optional block Walsh-Hadamard rotation + DualScale per-tensor scales +
// quantization + LSB truncation + packing of the activations.
//
// Method (pages): HQ-DM explainer 2.1 (block rotation of the activations
// before quantization), SegQuant explainer 2.B (separate scales for the
// non-negative and the negative region), TASQ explainer 2 (k least
// significant bits of every code dropped for a given step and layer).
//
// The tensor is processed as a flat stream of 4-element units (one 128-bit
// fp32 load or one 64-bit bf16 load per lane); consecutive lanes take
// consecutive units, so every wave instruction moves one contiguous span.
// A rotation block of B elements (B divides K, so blocks never straddle a
// row) occupies B/4 consecutive lanes of one load instruction and is rotated
// with in-lane butterflies and cross-lane swizzles, without LDS.
//
// Dynamic scales need the maximum over the whole tensor before any code is
// written, so there are two kernels: a max-reduction writing one partial
// maximum pair per block (plain stores, no atomics), then the quantizer,
// whose every block folds the partials into the scales first.
//
// With input branches (SegQuant explainer 2.A, input segmentation: a linear
// fed by a concatenation quantizes each branch apart) the same two kernels
// keep one maximum pair and one scale pair per branch; a unit's branch
// follows from its column, tracked incrementally along the stream.
#include <type_traits>

#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 8;                        // units per lane per chunk
constexpr int kChunk = kThreads * kUnroll;        // units per chunk
constexpr int kQuantBlocks = 2048;                // grid cap of the quantizer

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Branch of a unit from its column in units (branch starts past the last
// branch equal k_units, so they never match).
__device__ __forceinline__ int branch_of(const QuantArgs& a, int c) {
  return (c >= a.ks_units[1]) + (c >= a.ks_units[2]) + (c >= a.ks_units[3]);
}

// Column (in units) of this lane's first unit of a chunk, and the step to
// the next unit of the lane (kThreads units further, modulo the row).
__device__ __forceinline__ int first_col(const QuantArgs& a, int64_t first_unit) {
  return (int)((first_unit + threadIdx.x) % a.k_units);
}
__device__ __forceinline__ int next_col(const QuantArgs& a, int c, int step) {
  c += step;
  return c >= a.k_units ? c - a.k_units : c;
}

// The kUnroll units of chunk `c` that this lane owns: unit c*kChunk + u*256 + tid.
// Every load goes through a range-checked descriptor of the chunk (units past
// the end of the tensor read as zeros), so all of them are issued back to back.
template <bool BF16>
__device__ __forceinline__ void load_chunk(const void* X, int64_t nunits, int64_t c,
                                           float (&e)[kUnroll][4]) {
  constexpr uint32_t kUnitBytes = BF16 ? 8 : 16;
  const int64_t first = c * kChunk;
  const int64_t left = nunits - first;
  const uint32_t here = (uint32_t)(left < kChunk ? left : kChunk);
  const __amdgpu_buffer_rsrc_t r =
      buffer_rsrc(reinterpret_cast<const uint8_t*>(X) + first * kUnitBytes, here * kUnitBytes);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t off = (uint32_t)(u * kThreads + threadIdx.x) * kUnitBytes;
    if constexpr (BF16) {
      const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
      e[u][0] = __uint_as_float(v.x << 16);
      e[u][1] = __uint_as_float(v.x & 0xFFFF0000u);
      e[u][2] = __uint_as_float(v.y << 16);
      e[u][3] = __uint_as_float(v.y & 0xFFFF0000u);
    } else {
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
      e[u][0] = __uint_as_float(v.x);
      e[u][1] = __uint_as_float(v.y);
      e[u][2] = __uint_as_float(v.z);
      e[u][3] = __uint_as_float(v.w);
    }
  }
}

// Block-wide max of (mp, mn) into the partials of branch j.
__device__ __forceinline__ void store_partials(const QuantArgs& a, int j, uint32_t mp,
                                               uint32_t mn) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  mn &= 0x7FFFFFFFu;  // magnitude of the most negative value (0 if none)
  mp = wave_max_u32(mp);
  mn = wave_max_u32(mn);
  __shared__ uint32_t sm[2][kWaves];
  if (lane == 0) {
    sm[0][wave] = mp;
    sm[1][wave] = mn;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      mp = max(mp, sm[0][w]);
      mn = max(mn, sm[1][w]);
    }
    a.ws->part[j][0][blockIdx.x] = mp;
    a.ws->part[j][1][blockIdx.x] = mn;
  }
  __syncthreads();  // sm is reused by the next branch
}

template <bool BF16, int HB, bool KS>
__global__ __launch_bounds__(kThreads) void k1_reduce(QuantArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int NJ = KS ? kMaxKSeg : 1;
  uint32_t mp[NJ], mn[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    mp[j] = 0;
    mn[j] = 0x80000000u;
  }
  const int cstep = KS ? kThreads % a.k_units : 0;
  const int64_t nchunks = (a.nunits + kChunk - 1) / kChunk;
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    float e[kUnroll][4];
    load_chunk<BF16>(a.X, a.nunits, c, e);
    if constexpr (HB > 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) fwht_block<HB>(e[u], lane);
    }
    // On the bit patterns: non-negative floats order like their bits as
    // signed integers (negative floats are negative integers), and negative
    // floats order by magnitude like their bits as unsigned integers above
    // 0x80000000 (non-negative floats lie below it). One integer max each.
    // (Units past the end read as +0, which no maximum can lose to.)
    int col = KS ? first_col(a, c * kChunk) : 0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int br = KS ? branch_of(a, col) : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t b = __float_as_uint(e[u][i]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const bool mine = !KS || br == j;
          mp[j] = mine ? (uint32_t)max((int32_t)mp[j], (int32_t)b) : mp[j];
          mn[j] = mine ? max(mn[j], b) : mn[j];
        }
      }
      if constexpr (KS) col = next_col(a, col, cstep);
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (j < a.nks) store_partials(a, j, mp[j], mn[j]);
}

// Scales of branch j from the reduce kernel's per-block maxima (every block
// of the quantize kernel does this; max is exact and order-free, so all agree).
__device__ __forceinline__ void scales_from_partials(const QuantArgs& a, int j, float& sp,
                                                     float& sn) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  uint32_t mp = 0, mn = 0;
  for (int i = threadIdx.x; i < a.reduce_blocks; i += kThreads) {
    mp = max(mp, a.ws->part[j][0][i]);
    mn = max(mn, a.ws->part[j][1][i]);
  }
  mp = wave_max_u32(mp);
  mn = wave_max_u32(mn);
  __shared__ uint32_t sm[2][kWaves];
  if (lane == 0) {
    sm[0][wave] = mp;
    sm[1][wave] = mn;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mp = max(mp, sm[0][w]);
    mn = max(mn, sm[1][w]);
  }
  __syncthreads();  // sm is reused by the next branch
  const float mx = __uint_as_float(mp);
  const float mnv = __uint_as_float(mn);
  if (a.sym) {
    sp = (mx > mnv ? mx : mnv) / a.qa;
    sn = sp;
  } else {
    sp = mx / a.qa;
    sn = mnv / a.qa;
  }
}

// Codes of the four values of a unit, packed one per byte (element i in
// byte i); the same codes as quant_dual (round half even of the correctly
// rounded quotient Q = fl(v / s), clamped), computed from t = fl(v * fl(1/s)).
// With u = 2^-24: fl(1/s) and t each carry one relative rounding error of
// at most u, and Q one more, so |t - Q| <= 3u|q|(1 + u) (q the exact
// quotient), below |t| * 2^-22. The guard below computes
// z = fl(|t| * 2^-22 + d), d = |t - rint(t)| exactly (Sterbenz), and takes
// the product's integer when z < 0.5 - 2^-23; then the distance from t to
// every half-integer, 0.5 - d, exceeds |t| * 2^-22 + 2^-24 > |t - Q|, so t
// and Q lie strictly on one side of every half-integer and round alike
// (a Q that rounds onto a half-integer is caught too). Units with a closer
// value (and non-finite t, or |t| >= 2^21) are redone with the division;
// that is rare and wave-uniform work is skipped when no lane needs it.
// Rounding: m = t + 1.5 * 2^23 is t rounded
// half to even into the units of [2^23, 2^24) (the sum's even mantissas are
// the even integers), so m - 1.5 * 2^23 = rint(t) for |t| < 2^22, and after
// clamping m to 1.5 * 2^23 +- qa the code is the low byte of m's bits (the
// mantissa is 0x400000 + code). With r = 0 for a zero scale, t = 0 and the
// code is 0 as the definition requires; the sign of t follows v, so one
// symmetric clamp serves both polarity regions. SYM: one scale.
template <bool SYM>
__device__ __forceinline__ uint32_t quant_pack(const float (&e)[4], float sp, float sn, float rp,
                                               float rn, float qa) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  float m[4];
  bool slow = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v = e[i];
    const float t = v * (SYM ? rp : (v >= 0.0f ? rp : rn));
    const float s = t + kMagic;
    const float r = s - kMagic;
    const float z = fmaf(fabsf(t), 0x1p-22f, fabsf(t - r));
    slow |= !(z < 0x1.fffff8p-2f);  // 0.5 - 2^-23
    m[i] = __builtin_amdgcn_fmed3f(s, kMagic - qa, kMagic + qa);
  }
  if (slow) {
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = kMagic + (float)quant_dual(e[i], sp, sn, qa);
  }
  // bytes: [m0.b0, m1.b0, 0, 0] | [0, 0, m2.b0, m3.b0]
  const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(m[1]), __float_as_uint(m[0]), 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(m[3]), __float_as_uint(m[2]), 0x04000c0cu);
  return lo | hi;
}

// quant_pack for scales taken from the tensor's own maxima (s = fl(mx/qa)
// with every |v| <= mx), so |v/s| <= qa(1 + 2^-23) and no code needs
// clamping. With r = fl(1/s), the exact product P = v*r is within
// 2^-23 |q| <= qa 2^-23 (1 + 3u) of the correctly rounded quotient Q (both
// carry one relative rounding of at most u = 2^-24 from q = v/s).
// s = fma(v, r, 1.5 * 2^23) rounds P itself half to even into the integers
// (the code c = s - 1.5 * 2^23, exact, is s's low byte), and
// e = fma(v, r, -c) = fl(P - c). |e| < lim = 0.5 - (qa + 1) 2^-23 puts P
// more than qa 2^-23 + 2^-24 from every half-integer, so Q lies strictly
// between the same two half-integers and rint(Q) = c. Other units (and
// non-finite products) take the division, as in quant_pack.
template <bool SYM>
__device__ __forceinline__ uint32_t quant_pack_own(const float (&e)[4], float sp, float sn, float rp,
                                                   float rn, float qa, float lim) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  float m[4];
  bool slow = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v = e[i];
    const float r = SYM ? rp : (v >= 0.0f ? rp : rn);
    const float s = fmaf(v, r, kMagic);
    const float d = fmaf(v, r, -(s - kMagic));
    slow |= !(fabsf(d) < lim);
    m[i] = s;
  }
  if (slow) {
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = kMagic + (float)quant_dual(e[i], sp, sn, qa);
  }
  const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(m[1]), __float_as_uint(m[0]), 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(m[3]), __float_as_uint(m[2]), 0x04000c0cu);
  return lo | hi;
}

// TASQ truncation of a packed unit (k = lsb_k low magnitude bits cleared),
// then the store: 4 bytes, or (4-bit codes) two bytes of two nibbles each,
// element 2j in the low nibble of byte j.
struct LsbMask {
  bool on;
  uint32_t lut, keep;
  __device__ explicit LsbMask(int keep_mask) {
    const int k = keep_mask == -1 ? 0 : __builtin_ctz((uint32_t)keep_mask);
    on = k > 0;
    lut = ((1u << k) - 1u) << 8;
    keep = 0x01010101u * (0xFFu & (uint32_t)keep_mask);
  }
};

// LSB: truncation known at compile time (1: on, 0: off); -1: test mk.on.
template <bool A4, int LSB = -1>
__device__ __forceinline__ void store_unit(const __amdgpu_buffer_rsrc_t& rc, uint32_t off,
                                           uint32_t p, const LsbMask& mk) {
  if (LSB == 1 || (LSB == -1 && mk.on)) p = trunc_mag4(p, mk.lut, mk.keep);
  if constexpr (A4) {
    const uint32_t q = p & 0x0F0F0F0Fu;
    const uint32_t r = q | (q >> 4);  // byte 0 = c0 | c1 << 4, byte 2 = c2 | c3 << 4
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)__builtin_amdgcn_perm(0u, r, 0x0c0c0200u),
                                          rc, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(p, rc, off, 0, 0);
  }
}

template <bool BF16, int HB, bool A4, bool KS>
__global__ __launch_bounds__(kThreads) void k1_quantize(QuantArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int NJ = KS ? kMaxKSeg : 1;
  float sps[NJ], sns[NJ], rps[NJ], rns[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    float sp = 0.0f, sn = 0.0f;
    if (j < a.nks) {
      if (a.static_scales) {
        sp = a.static_scales[2 * j];
        sn = a.static_scales[2 * j + 1];
      } else {
        scales_from_partials(a, j, sp, sn);
      }
      if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.act_scales[2 * j] = sp;
        a.act_scales[2 * j + 1] = sn;
      }
    }
    sps[j] = sp;
    sns[j] = sn;
    rps[j] = sp > 0.0f ? 1.0f / sp : 0.0f;
    rns[j] = sn > 0.0f ? 1.0f / sn : 0.0f;
  }
  const int cstep = KS ? kThreads % a.k_units : 0;
  constexpr uint32_t kCodeBytes = A4 ? 2 : 4;
  const LsbMask mk(a.keep_mask);
  // dynamic scales are the maxima of the very values quantized here
  // (per branch), so the one-pass kernel's shorter exact test applies
  const bool own = a.static_scales == nullptr;
  const float lim = 0.5f - (a.qa + 1.0f) * 0x1p-23f;
  const int64_t nchunks = (a.nunits + kChunk - 1) / kChunk;
  for (int64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    float e[kUnroll][4];
    load_chunk<BF16>(a.X, a.nunits, ch, e);
    if constexpr (HB > 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) fwht_block<HB>(e[u], lane);
    }
    const int64_t first = ch * kChunk;
    const int64_t left = a.nunits - first;
    const uint32_t here = (uint32_t)(left < kChunk ? left : kChunk);
    const __amdgpu_buffer_rsrc_t rc =
        buffer_rsrc(reinterpret_cast<uint8_t*>(a.codes) + first * kCodeBytes, here * kCodeBytes);
    int col = KS ? first_col(a, first) : 0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float sp = sps[0], sn = sns[0], rp = rps[0], rn = rns[0];
      if constexpr (KS) {
        const int br = branch_of(a, col);
#pragma unroll
        for (int j = 1; j < NJ; ++j) {
          sp = br == j ? sps[j] : sp;
          sn = br == j ? sns[j] : sn;
          rp = br == j ? rps[j] : rp;
          rn = br == j ? rns[j] : rn;
        }
        col = next_col(a, col, cstep);
      }
      uint32_t p;
      if (HB == 0 && own)
        p = a.sym ? quant_pack_own<true>(e[u], sp, sn, rp, rn, a.qa, lim)
                  : quant_pack_own<false>(e[u], sp, sn, rp, rn, a.qa, lim);
      else
        p = a.sym ? quant_pack<true>(e[u], sp, sn, rp, rn, a.qa)
                  : quant_pack<false>(e[u], sp, sn, rp, rn, a.qa);
      store_unit<A4>(rc, (uint32_t)(u * kThreads + threadIdx.x) * kCodeBytes, p, mk);
    }
  }
}

// ---- One pass, for tensors that fit on chip (dynamic scales, one or two
// input branches). One workgroup per compute unit holds its slice of X in
// registers (up to kFUnits units per lane) and publishes its partial maxima
// (one pair per branch); workgroup 0 gathers them and publishes the
// tensor's maxima; every
// workgroup then quantizes from registers: X is read once (5 bytes per fp32
// element moved in all, instead of 9). Every wait is bounded: a workgroup
// that gives up (only possible if the grid was not all resident) scans X
// for the maxima itself, so the kernel always ends and its codes are always
// those of the two-pass path.
constexpr int kFThreads = 512;               // 8 waves, 2 per SIMD
constexpr int kFWaves = kFThreads / kWave;
constexpr int kFUnits = 40;                  // units per lane held in registers, at most
constexpr uint32_t kFSpin = 1u << 18;        // barrier polls before scanning X

template <bool BF16>
__device__ __forceinline__ void load_unit(const __amdgpu_buffer_rsrc_t& r, uint32_t off,
                                          float (&e)[4]) {
  if constexpr (BF16) {
    const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    e[0] = __uint_as_float(v.x << 16);
    e[1] = __uint_as_float(v.x & 0xFFFF0000u);
    e[2] = __uint_as_float(v.y << 16);
    e[3] = __uint_as_float(v.y & 0xFFFF0000u);
  } else {
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    e[0] = __uint_as_float(v.x);
    e[1] = __uint_as_float(v.y);
    e[2] = __uint_as_float(v.z);
    e[3] = __uint_as_float(v.w);
  }
}

// Fold four values into the maxima pair (bit patterns, as k1_reduce keeps them).
__device__ __forceinline__ void max4(const float (&e)[4], uint32_t& mp, uint32_t& mn) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = __float_as_uint(e[i]);
    mp = (uint32_t)max((int32_t)mp, (int32_t)b);
    mn = max(mn, b);
  }
}

// Workgroup-wide max of (mp, mn) (mn as a magnitude), returned to every thread.
__device__ __forceinline__ void block_max2(uint32_t& mp, uint32_t& mn, uint32_t (&sm)[2][kFWaves]) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  mp = wave_max_u32(mp);
  mn = wave_max_u32(mn);
  if (lane == 0) {
    sm[0][wave] = mp;
    sm[1][wave] = mn;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kFWaves; ++w) {
    mp = max(mp, sm[0][w]);
    mn = max(mn, sm[1][w]);
  }
  __syncthreads();
}

// Column (in units) of unit g of the tensor, stepped lane-wise: each lane's
// next unit lies kFThreads units further, and kFThreads % k_units < k_units,
// so one conditional subtract keeps the column in range.
__device__ __forceinline__ int step_col(int c, int step, int k_units) {
  const int d = c + step;
  return (uint32_t)(d - k_units) < (uint32_t)d ? d - k_units : d;
}

// NS: maxima pairs kept (1: the tensor's; 2: two input branches, whose
// boundary ks_units[1] splits every row; a unit never straddles it).
template <bool BF16, int HB, bool A4, int NS>
__global__ __launch_bounds__(kFThreads, 1) void k1_fused(QuantArgs a, int U) {
  static_assert(NS == 1 || NS == 2, "one or two maxima pairs");
  __shared__ uint32_t sm[2][kFWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int G = gridDim.x, b = blockIdx.x;
  constexpr uint32_t kUnitBytes = BF16 ? 8 : 16;
  const int64_t span = (int64_t)U * kFThreads;
  const int64_t first = (int64_t)b * span;
  const int64_t left = a.nunits - first;
  const uint32_t here = (uint32_t)(left <= 0 ? 0 : (left < span ? left : span));
  const __amdgpu_buffer_rsrc_t rx =
      buffer_rsrc(reinterpret_cast<const uint8_t*>(a.X) + first * kUnitBytes, here * kUnitBytes);
  // Unit u of this lane: first + u * kFThreads + tid (consecutive lanes on
  // consecutive units; units past the end read as zeros).
  float e[kFUnits][4];
#pragma unroll
  for (int u = 0; u < kFUnits; ++u) {
    if (u < U) {
      load_unit<BF16>(rx, (uint32_t)(u * kFThreads + tid) * kUnitBytes, e[u]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) e[u][i] = 0.0f;
    }
  }
  if constexpr (HB > 0) {
#pragma unroll
    for (int u = 0; u < kFUnits; ++u)
      if (u < U) fwht_block<HB>(e[u], lane);
  }
  // Branch tracking (NS = 2): column of this lane's first unit and the
  // column step between its units; branch 1 starts at column kb1.
  const int kun = a.k_units;
  const int cstep = NS > 1 ? kFThreads % kun : 0;
  const int col0 = NS > 1 ? (int)((first + tid) % kun) : 0;
  const int kb1 = a.ks_units[1];
  uint32_t mp[NS], mn[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    mp[j] = 0;             // +0: zeros never win
    mn[j] = 0x80000000u;   // -0
  }
  if constexpr (NS == 1) {
#pragma unroll
    for (int u = 0; u < kFUnits; ++u) max4(e[u], mp[0], mn[0]);
  } else {
    int col = col0;
#pragma unroll
    for (int u = 0; u < kFUnits; ++u) {
      uint32_t up = 0, un = 0x80000000u;
      max4(e[u], up, un);  // the unit's maxima, then its branch's
      const bool b1 = col >= kb1;
      mp[0] = b1 ? mp[0] : (uint32_t)max((int32_t)mp[0], (int32_t)up);
      mn[0] = b1 ? mn[0] : max(mn[0], un);
      mp[1] = b1 ? (uint32_t)max((int32_t)mp[1], (int32_t)up) : mp[1];
      mn[1] = b1 ? max(mn[1], un) : mn[1];
      col = step_col(col, cstep, kun);
    }
  }
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    mn[j] &= 0x7FFFFFFFu;
    block_max2(mp[j], mn[j], sm);
  }

  // Exchange: publish this workgroup's maxima; workgroup 0 gathers all of
  // them and publishes the tensor's (per branch); the others wait for that.
  GridSync* gs = &a.ws->sync;
  const uint64_t tag = (uint64_t)a.seq << 32;
  __shared__ uint32_t got[1 + 2 * NS];
  if (tid == 0) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      __hip_atomic_store(&gs->word[2 * j][b], tag | mp[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&gs->word[2 * j + 1][b], tag | mn[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  bool ok = false;
  uint32_t gp[NS], gn[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) gp[j] = gn[j] = 0;
  if (b == 0) {
    for (uint32_t it = 0; it < kFSpin; ++it) {
      bool mine = true;
      if (tid < G) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const uint64_t w0 = __hip_atomic_load(&gs->word[2 * j][tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint64_t w1 = __hip_atomic_load(&gs->word[2 * j + 1][tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          mine = mine && (w0 & ~0xFFFFFFFFull) == tag && (w1 & ~0xFFFFFFFFull) == tag;
          gp[j] = (uint32_t)w0;
          gn[j] = (uint32_t)w1;
        }
      }
      if (__syncthreads_and(mine)) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  } else {
    if (tid == 0) {
      got[0] = 0;
      for (uint32_t it = 0; it < kFSpin; ++it) {
        uint64_t r[2 * NS];
        bool all = true;
#pragma unroll
        for (int i = 0; i < 2 * NS; ++i) {
          r[i] = __hip_atomic_load(&gs->result[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          all = all && (r[i] & ~0xFFFFFFFFull) == tag;
        }
        if (all) {
          got[0] = 1;
#pragma unroll
          for (int i = 0; i < 2 * NS; ++i) got[1 + i] = (uint32_t)r[i];
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
    }
    __syncthreads();
    ok = got[0] != 0;
    // every thread takes the tensor's maxima (the max below leaves them as they are)
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      gp[j] = ok ? got[1 + 2 * j] : 0;
      gn[j] = ok ? got[2 + 2 * j] : 0;
    }
  }
  if (!ok) {
    // Fallback: the maxima of the whole tensor, read here.
    if (tid == 0) __hip_atomic_fetch_add(&gs->fallbacks, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const __amdgpu_buffer_rsrc_t rall = buffer_rsrc(a.X, (uint32_t)(a.nunits * kUnitBytes));
    uint32_t fp[NS], fn[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      fp[j] = 0;
      fn[j] = 0x80000000u;
    }
    for (int64_t i = tid; i < a.nunits; i += kFThreads) {
      float f[4];
      load_unit<BF16>(rall, (uint32_t)i * kUnitBytes, f);
      if constexpr (HB > 0) fwht_block<HB>(f, lane);
      if constexpr (NS == 1) {
        max4(f, fp[0], fn[0]);
      } else {
        const int j = (int)(i % kun) >= kb1 ? 1 : 0;
        uint32_t up = 0, un = 0x80000000u;
        max4(f, up, un);
        fp[j] = (uint32_t)max((int32_t)fp[j], (int32_t)up);
        fn[j] = max(fn[j], un);
      }
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      gp[j] = fp[j];
      gn[j] = fn[j] & 0x7FFFFFFFu;
    }
  }
  float sps[NS], sns[NS], rps[NS], rns[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    block_max2(gp[j], gn[j], sm);
    if (b == 0 && tid == 0) {  // the tensor's maxima, for the other workgroups
      __hip_atomic_store(&gs->result[2 * j], tag | gp[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&gs->result[2 * j + 1], tag | gn[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const float mx = __uint_as_float(gp[j]), mnv = __uint_as_float(gn[j]);
    float sp, sn;
    if (a.sym) {
      sp = (mx > mnv ? mx : mnv) / a.qa;
      sn = sp;
    } else {
      sp = mx / a.qa;
      sn = mnv / a.qa;
    }
    if (b == 0 && tid == 0) {
      a.act_scales[2 * j] = sp;
      a.act_scales[2 * j + 1] = sn;
    }
    sps[j] = sp;
    sns[j] = sn;
    rps[j] = sp > 0.0f ? 1.0f / sp : 0.0f;
    rns[j] = sn > 0.0f ? 1.0f / sn : 0.0f;
  }
  constexpr uint32_t kCodeBytes = A4 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rc =
      buffer_rsrc(reinterpret_cast<uint8_t*>(a.codes) + first * kCodeBytes, here * kCodeBytes);
  const LsbMask mk(a.keep_mask);
  const float lim = 0.5f - (a.qa + 1.0f) * 0x1p-23f;  // the scales are the tensor's own
  auto quant_all = [&](auto symc, auto lsbc) __attribute__((always_inline)) {
    constexpr bool SYM = decltype(symc)::value;
    constexpr int LSB = decltype(lsbc)::value ? 1 : 0;
    int col = col0;
#pragma unroll
    for (int u = 0; u < kFUnits; ++u) {
      if (u < U) {
        float sp = sps[0], sn = sns[0], rp = rps[0], rn = rns[0];
        if constexpr (NS == 2) {
          const bool b1 = col >= kb1;
          sp = b1 ? sps[1] : sp;
          sn = b1 ? sns[1] : sn;
          rp = b1 ? rps[1] : rp;
          rn = b1 ? rns[1] : rn;
          col = step_col(col, cstep, kun);
        }
        // (with the rotation in registers too, the shorter form makes the
        // compiler spill, so rotated tensors keep quant_pack)
        uint32_t p;
        if constexpr (HB == 0)
          p = quant_pack_own<SYM>(e[u], sp, sn, rp, rn, a.qa, lim);
        else
          p = quant_pack<SYM>(e[u], sp, sn, rp, rn, a.qa);
        store_unit<A4, LSB>(rc, (uint32_t)(u * kFThreads + tid) * kCodeBytes, p, mk);
      }
    }
  };
  // the scale mode and the truncation are uniform: one straight-line
  // quantize phase per combination, no per-unit test
  if (a.sym) {
    if (mk.on)
      quant_all(std::true_type{}, std::true_type{});
    else
      quant_all(std::true_type{}, std::false_type{});
  } else {
    if (mk.on)
      quant_all(std::false_type{}, std::true_type{});
    else
      quant_all(std::false_type{}, std::false_type{});
  }
}

int chunks_of(int64_t nunits) {
  const int64_t c = (nunits + kChunk - 1) / kChunk;
  return (int)(c < 1 ? 1 : (c > (1 << 30) ? (1 << 30) : c));
}

// At most `cap` workgroups, each taking the same number of chunks (up to one
// fewer for the last ones), so no workgroup runs a long tail alone.
int balanced_grid(int nch, int cap) {
  const int per = (nch + cap - 1) / cap;
  return (nch + per - 1) / per;
}

// One-pass launch when the tensor fits in the registers of one workgroup
// per compute unit (dynamic scales, one or two input branches, HB 0 or 128):
// returns false to let the caller run the two passes.
template <bool BF16, int HB, bool A4, int NS>
bool run_fused(const QuantArgs& a, hipStream_t s, hipError_t& e) {
  if constexpr (HB != 0 && HB != 128) {
    return false;
  } else {
    if (a.static_scales || a.nks != NS || a.nunits <= 0 || a.seq == 0) return false;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return false;
    const int64_t per = (int64_t)cus * kFThreads;
    const int64_t U = (a.nunits + per - 1) / per;
    // workgroup 0 gathers one workgroup's words per thread
    static_assert(kFThreads <= kMaxReduceBlocks, "exchange words per workgroup");
    if (U > kFUnits || cus > kFThreads) return false;
    const int G = (int)((a.nunits + U * kFThreads - 1) / (U * kFThreads));
    hipLaunchKernelGGL((k1_fused<BF16, HB, A4, NS>), dim3(G), dim3(kFThreads), 0, s, a, (int)U);
    e = hipGetLastError();
    return true;
  }
}

template <bool BF16, int HB, bool A4, bool KS>
hipError_t run_ks(QuantArgs a, hipStream_t s) {
  {
    hipError_t e = hipSuccess;
    if (run_fused<BF16, HB, A4, KS ? 2 : 1>(a, s, e)) return e;
  }
  const int nch = chunks_of(a.nunits);
  const int g = balanced_grid(nch, kQuantBlocks);
  if (!a.static_scales) {
    a.reduce_blocks = balanced_grid(nch, kMaxReduceBlocks);
    hipLaunchKernelGGL((k1_reduce<BF16, HB, KS>), dim3(a.reduce_blocks), dim3(kThreads), 0, s,
                       a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k1_quantize<BF16, HB, A4, KS>), dim3(g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <bool BF16, int HB, bool A4>
hipError_t run(const QuantArgs& a, hipStream_t s) {
  if (a.nks > 1) return run_ks<BF16, HB, A4, true>(a, s);
  return run_ks<BF16, HB, A4, false>(a, s);
}

template <bool BF16, bool A4>
hipError_t run_hb(const QuantArgs& a, int hb, hipStream_t s) {
  switch (hb) {
    case 0: return run<BF16, 0, A4>(a, s);
    case 4: return run<BF16, 4, A4>(a, s);
    case 8: return run<BF16, 8, A4>(a, s);
    case 16: return run<BF16, 16, A4>(a, s);
    case 32: return run<BF16, 32, A4>(a, s);
    case 64: return run<BF16, 64, A4>(a, s);
    case 128: return run<BF16, 128, A4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, int x_bf16, int hadamard_block, int a4,
                           hipStream_t s) {
  if (x_bf16) return a4 ? run_hb<true, true>(a, hadamard_block, s) : run_hb<true, false>(a, hadamard_block, s);
  return a4 ? run_hb<false, true>(a, hadamard_block, s) : run_hb<false, false>(a, hadamard_block, s);
}

}  // namespace ql
