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
#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 4;  // units per lane per iteration

template <bool BF16>
__device__ __forceinline__ void load_unit(const void* X, int64_t idx, int64_t n, float (&e)[4]) {
  if (idx < n) {
    if constexpr (BF16) {
      const uint2 v = reinterpret_cast<const uint2*>(X)[idx];
      e[0] = __uint_as_float(v.x << 16);
      e[1] = __uint_as_float(v.x & 0xFFFF0000u);
      e[2] = __uint_as_float(v.y << 16);
      e[3] = __uint_as_float(v.y & 0xFFFF0000u);
    } else {
      const float4 v = reinterpret_cast<const float4*>(X)[idx];
      e[0] = v.x;
      e[1] = v.y;
      e[2] = v.z;
      e[3] = v.w;
    }
  } else {
    e[0] = e[1] = e[2] = e[3] = 0.0f;
  }
}

template <bool BF16, int HB>
__global__ __launch_bounds__(kThreads) void k1_reduce(QuantArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  uint32_t mp = 0, mn = 0;
  const int64_t step = (int64_t)gridDim.x * kWaves * kWave * kUnroll;
  for (int64_t base = ((int64_t)blockIdx.x * kWaves + wave) * kWave * kUnroll; base < a.nunits;
       base += step) {
    float e[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) load_unit<BF16>(a.X, base + u * kWave + lane, a.nunits, e[u]);
    if constexpr (HB > 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) fwht_block<HB>(e[u], lane);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = e[u][i];
        const uint32_t b = __float_as_uint(v) & 0x7FFFFFFFu;
        mp = (v > 0.0f && b > mp) ? b : mp;
        mn = (v < 0.0f && b > mn) ? b : mn;
      }
  }
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
    a.ws->part[0][blockIdx.x] = mp;
    a.ws->part[1][blockIdx.x] = mn;
  }
}

// Scales from the reduce kernel's per-block maxima (every block of the
// quantize kernel does this; max is exact and order-free, so all agree).
__device__ __forceinline__ void scales_from_partials(const QuantArgs& a, float& sp, float& sn) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  uint32_t mp = 0, mn = 0;
  for (int i = threadIdx.x; i < a.reduce_blocks; i += kThreads) {
    mp = max(mp, a.ws->part[0][i]);
    mn = max(mn, a.ws->part[1][i]);
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

template <bool BF16, int HB, bool A4>
__global__ __launch_bounds__(kThreads) void k1_quantize(QuantArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  float sp, sn;
  if (a.static_scales) {
    sp = a.static_scales[0];
    sn = a.static_scales[1];
  } else {
    scales_from_partials(a, sp, sn);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.act_scales[0] = sp;
    a.act_scales[1] = sn;
  }
  const int64_t step = (int64_t)gridDim.x * kWaves * kWave * kUnroll;
  for (int64_t base = ((int64_t)blockIdx.x * kWaves + wave) * kWave * kUnroll; base < a.nunits;
       base += step) {
    float e[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) load_unit<BF16>(a.X, base + u * kWave + lane, a.nunits, e[u]);
    if constexpr (HB > 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) fwht_block<HB>(e[u], lane);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t idx = base + u * kWave + lane;
      int c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = truncate_lsb(quant_dual(e[u][i], sp, sn, a.qa), a.keep_mask);
      if (idx < a.nunits) {
        if constexpr (A4) {
          const uint32_t p = (c[0] & 0xF) | ((c[1] & 0xF) << 4) | ((c[2] & 0xF) << 8) |
                             ((c[3] & 0xF) << 12);
          reinterpret_cast<uint16_t*>(a.codes)[idx] = (uint16_t)p;
        } else {
          const uint32_t p = (c[0] & 0xFF) | ((c[1] & 0xFF) << 8) | ((c[2] & 0xFF) << 16) |
                             ((uint32_t)(c[3] & 0xFF) << 24);
          reinterpret_cast<uint32_t*>(a.codes)[idx] = p;
        }
      }
    }
  }
}

int grid_for(int64_t nunits) {
  const int64_t per_block = (int64_t)kThreads * kUnroll;
  int64_t g = (nunits + per_block - 1) / per_block;
  if (g > 2048) g = 2048;
  if (g < 1) g = 1;
  return (int)g;
}

template <bool BF16, int HB, bool A4>
hipError_t run(QuantArgs a, hipStream_t s) {
  const int g = grid_for(a.nunits);
  if (!a.static_scales) {
    a.reduce_blocks = g < kMaxReduceBlocks ? g : kMaxReduceBlocks;
    hipLaunchKernelGGL((k1_reduce<BF16, HB>), dim3(a.reduce_blocks), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k1_quantize<BF16, HB, A4>), dim3(g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
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
