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

// Codes of the four values of a unit; the same codes as quant_dual (round
// half even of the correctly rounded quotient v / s, clamped), computed as
// t = v * (1/s): the quotient and t differ by less than |t| * 2^-22, so
// wherever t lies farther than |t| * 2^-20 + 2^-20 from every half-integer
// both round to the same integer. Units with a value closer than that (and
// non-finite t) are redone with the division; that is rare and
// wave-uniform work is skipped when no lane needs it. With r = 0 for a zero
// scale, t = 0 and the code is 0 as the definition requires; the sign of t
// follows v, so one symmetric clamp serves both polarity regions.
__device__ __forceinline__ void quant_unit(const float (&e)[4], float sp, float sn, float rp,
                                           float rn, float qa, int (&c)[4]) {
  bool slow = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v = e[i];
    const float t = v * (v >= 0.0f ? rp : rn);
    const float r = rintf(t);
    const float z = fmaf(fabsf(t), 0x1p-20f, fabsf(t - r));
    slow |= !(z < 0x1.fffcp-2f);  // 0.5 - 2^-19
    c[i] = (int)__builtin_amdgcn_fmed3f(r, -qa, qa);
  }
  if (slow) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = quant_dual(e[i], sp, sn, qa);
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
      int c[4];
      quant_unit(e[u], sp, sn, rp, rn, a.qa, c);
      if (a.keep_mask != -1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = truncate_lsb(c[i], a.keep_mask);
      }
      const uint32_t off = (uint32_t)(u * kThreads + threadIdx.x) * kCodeBytes;
      if constexpr (A4) {
        const uint32_t p = (c[0] & 0xF) | ((c[1] & 0xF) << 4) | ((c[2] & 0xF) << 8) |
                           ((c[3] & 0xF) << 12);
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)p, rc, off, 0, 0);
      } else {
        const uint32_t p = (c[0] & 0xFF) | ((c[1] & 0xFF) << 8) | ((c[2] & 0xFF) << 16) |
                           ((uint32_t)(c[3] & 0xFF) << 24);
        __builtin_amdgcn_raw_buffer_store_b32(p, rc, off, 0, 0);
      }
    }
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

template <bool BF16, int HB, bool A4, bool KS>
hipError_t run_ks(QuantArgs a, hipStream_t s) {
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
