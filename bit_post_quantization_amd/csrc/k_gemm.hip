// K2: integer GEMM of the activation codes against the weight codes on the
// int8 matrix cores of gfx950, both DualScale polarity planes in one kernel,
// with the fp32 epilogue (scales, Hadamard normalisation, CFG combine) fused.
//
// Method (pages): SegQuant explainer 2.B -- X is split into its
// non-negative and negative parts, each multiplied by the weight codes; the
// two products run side by side in one batched kernel and their rescaled
// results are summed in the epilogue. "Closing the Null Space" explainer,
// problem statement -- guided output uncond + w (cond - uncond).
//
// Design for CDNA4 (MI355X):
//  * v_mfma_i32_16x16x64_i8. Each 16x64 activation fragment is split in
//    registers into its two polarity planes (byte sign masks) and both are
//    multiplied by the same weight fragment into two accumulator sets: the
//    batch-2 GEMM of the method shares every weight fragment it reads.
//  * Tile 128 rows x (16*NB) columns, 4 waves of 32 rows each, one workgroup
//    per CU. NB = 9 (144 columns) makes the DiT-XL/2 widths (1152, 3456,
//    4608 = 8, 24, 32 x 144) give exactly 1, 3 or 4 tiles per CU at M = 4096.
//  * Operands move HBM -> LDS by buffer_load ... lds (no VGPR staging) into
//    a ring of kStages K-steps, issued kStages-1 steps ahead. The buffer
//    resource's range check turns every out-of-range row or K-chunk into
//    zeros, so ragged M, N and K need no special path.
//  * LDS holds operands in fragment order: the 16 bytes lane l feeds to the
//    MFMA sit at lane*16, so fragment reads are linear and conflict-free.
//    4-bit codes stay packed in LDS (half the bytes) and are unpacked on the
//    LDS -> register path, each code multiplied by 16 (nibble placed in the
//    high half of its byte: two ANDs, a shift, two byte permutes); the
//    accumulators are shifted back exactly at the end.
//  * CFG pairing: a tile holds 64 conditional rows and their 64
//    unconditional partners; a wave's fragment 0 is 16 conditional rows and
//    fragment 1 their partners, so a lane holds both accumulators of a pair
//    in the same register slot and combines them with no data exchange.
//  * Workgroups are mapped to tiles so that each XCD (workgroup id mod 8)
//    works on one contiguous band of tiles, which share rows in its L2.
#include <type_traits>

#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
template <int V>
using IC = std::integral_constant<int, V>;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int BK = 64;        // K elements per ring stage
constexpr int kStages = 6;    // ring depth
constexpr unsigned kOOB = 0x80000000u;  // offset beyond every buffer: loads return 0

template <bool P4>
struct Op {
  static constexpr int kFragBytes = P4 ? 512 : 1024;  // one 16 x 64 fragment
  static constexpr int kLoads = P4 ? 2 : 1;           // DMA instructions per fragment
};

template <bool A4, bool W4, int NB>
struct Layout {
  static constexpr int kAFrags = 8;                       // 128 rows
  static constexpr int kWPerWave = (NB + kWaves - 1) / kWaves;
  static constexpr int kABytes = kAFrags * Op<A4>::kFragBytes;
  static constexpr int kWBytes = NB * Op<W4>::kFragBytes;
  static constexpr int kStage = kABytes + kWBytes;
  static constexpr int kSink = Op<W4>::kFragBytes;       // target of padding loads
  static constexpr int kLds = kStages * kStage + kSink;
  // DMA instructions one wave issues per stage (same for every wave)
  static constexpr int kLoadsPerStage = 2 * Op<A4>::kLoads + kWPerWave * Op<W4>::kLoads;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// vmcnt-only wait (expcnt / lgkmcnt left at their maxima), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One fragment (16 rows x 64 K) from global into LDS at `dst` (wave-uniform).
// row_off: byte offset of this lane's row, or kOOB. Lane l covers K-chunk
// l/16 (16 elements) of row l%16.
template <bool P4>
__device__ __forceinline__ void dma_frag(__amdgpu_buffer_rsrc_t r, uint8_t* dst, unsigned row_off,
                                         int k0, int K, int lane) {
  const int kk = k0 + 16 * (lane >> 4);
  const bool ok = row_off != kOOB && kk < K;
  if constexpr (P4) {
    const unsigned v = ok ? row_off + (unsigned)(kk >> 1) : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, v, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + 256), 4, v + 4u, 0, 0, 0);
  } else {
    const unsigned v = ok ? row_off + (unsigned)kk : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, v, 0, 0, 0);
  }
}

// Raw fragment data of one lane: int8 -> 4 dwords, 4-bit -> 2 dwords.
template <bool P4>
struct Raw {
  uint32_t d[P4 ? 2 : 4];
};

template <bool P4>
__device__ __forceinline__ void read_frag(Raw<P4>& f, const uint8_t* src, int lane) {
  if constexpr (P4) {
    f.d[0] = *reinterpret_cast<const uint32_t*>(src + lane * 4);
    f.d[1] = *reinterpret_cast<const uint32_t*>(src + 256 + lane * 4);
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(src + lane * 16);
    f.d[0] = v.x;
    f.d[1] = v.y;
    f.d[2] = v.z;
    f.d[3] = v.w;
  }
}

// MFMA operand (16 int8 in natural K order) from raw fragment data.
template <bool P4>
__device__ __forceinline__ v4i operand(const Raw<P4>& f) {
  v4i o;
  if constexpr (P4) {
    uint32_t a, b, c, d;
    unpack4_x16(f.d[0], a, b);
    unpack4_x16(f.d[1], c, d);
    o[0] = (int)a;
    o[1] = (int)b;
    o[2] = (int)c;
    o[3] = (int)d;
  } else {
    o[0] = (int)f.d[0];
    o[1] = (int)f.d[1];
    o[2] = (int)f.d[2];
    o[3] = (int)f.d[3];
  }
  return o;
}

__device__ __forceinline__ void split(v4i c, v4i& p, v4i& n) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t pp, nn;
    split_polarity((uint32_t)c[i], pp, nn);
    p[i] = (int)pp;
    n[i] = (int)nn;
  }
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// y from the two accumulators in the documented order, no contraction.
template <bool SYM>
__device__ __forceinline__ float epi(int accp, int accn, float sp, float sn, float sw, float inv_b) {
  float y;
  if constexpr (SYM) {
    y = __fmul_rn(__fmul_rn((float)accp, sp), sw);
  } else {
    const float tp = __fmul_rn((float)accp, sp);
    const float tn = __fmul_rn((float)accn, sn);
    y = __fmul_rn(__fadd_rn(tp, tn), sw);
  }
  return __fmul_rn(y, inv_b);
}

template <bool A4, bool W4, bool SYM, bool CFG, bool DBG, int NB>
__global__ __launch_bounds__(kThreads, 1) void k2_gemm(GemmArgs g) {
  using Lay = Layout<A4, W4, NB>;
  constexpr int NP = SYM ? 1 : 2;                       // accumulator planes
  constexpr int SHIFT = (A4 ? 4 : 0) + (W4 ? 4 : 0);    // undo the x16 unpack
  constexpr int BN = 16 * NB;
  // One LDS object per ring stage: the compiler tracks DMA -> LDS writes per
  // object, so a fragment read waits only for the DMA of its own stage.
  __shared__ __attribute__((aligned(16))) uint8_t st0[Lay::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[Lay::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st2[Lay::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st3[Lay::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st4[Lay::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st5[Lay::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t sink[Lay::kSink];
  static_assert(kStages == 6, "one LDS object per stage");
  uint8_t* const slots[kStages] = {st0, st1, st2, st3, st4, st5};

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // ---- tile of this workgroup (XCD-banded order) ----
  const int rows = CFG ? g.Mh : g.M;
  const int rt = (rows + (CFG ? 63 : 127)) / (CFG ? 64 : 128);
  const int ct = (g.N + BN - 1) / BN;
  const int T = rt * ct;
  int t = blockIdx.x;
  if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
  const int tr = t / ct, tc = t - tr * ct;
  const int m0 = tr * (CFG ? 64 : 128);
  const int n0 = tc * BN;

  // ---- per-lane row offsets for this wave's DMA work ----
  const int i16 = lane & 15;
  unsigned aoff[2];
#pragma unroll
  for (int fi = 0; fi < 2; ++fi) {
    const int f = 2 * wave + fi;
    int grow;
    bool ok;
    if constexpr (CFG) {
      const int crow = m0 + 16 * (f >> 1) + i16;
      ok = crow < g.Mh;
      grow = crow + (f & 1) * g.Mh;
    } else {
      grow = m0 + 16 * f + i16;
      ok = grow < g.M;
    }
    aoff[fi] = ok ? (unsigned)grow * (unsigned)g.lda : kOOB;
  }
  unsigned woff[Lay::kWPerWave];
#pragma unroll
  for (int i = 0; i < Lay::kWPerWave; ++i) {
    const int j = wave + kWaves * i;
    const int n = n0 + 16 * j + i16;
    woff[i] = (j < NB && n < g.N) ? (unsigned)n * (unsigned)g.ldw : kOOB;
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)((int64_t)g.M * g.lda));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.W, (uint32_t)((int64_t)g.N * g.ldw));

  auto issue = [&](int s, uint8_t* slot) {
    const int k0 = s * BK;
#pragma unroll
    for (int fi = 0; fi < 2; ++fi)
      dma_frag<A4>(ra, slot + (2 * wave + fi) * Op<A4>::kFragBytes, aoff[fi], k0, g.K, lane);
#pragma unroll
    for (int i = 0; i < Lay::kWPerWave; ++i) {
      const int j = wave + kWaves * i;
      uint8_t* dst = j < NB ? slot + Lay::kABytes + j * Op<W4>::kFragBytes
                            : sink;  // padding load
      dma_frag<W4>(rw, dst, woff[i], k0, g.K, lane);
    }
  };

  struct Frags {
    Raw<A4> a[2];
    Raw<W4> w[NB];
  };
  auto read_all = [&](Frags& F, const uint8_t* slot) {
#pragma unroll
    for (int fi = 0; fi < 2; ++fi) read_frag<A4>(F.a[fi], slot + (2 * wave + fi) * Op<A4>::kFragBytes, lane);
#pragma unroll
    for (int j = 0; j < NB; ++j) read_frag<W4>(F.w[j], slot + Lay::kABytes + j * Op<W4>::kFragBytes, lane);
  };

  v4i acc[NP][2][NB];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int fi = 0; fi < 2; ++fi)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[p][fi][j] = v4i{0, 0, 0, 0};

  auto compute = [&](const Frags& F) {
#pragma unroll
    for (int fi = 0; fi < 2; ++fi) {
      const v4i a = operand<A4>(F.a[fi]);
      if constexpr (SYM) {
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[0][fi][j] = mfma(a, operand<W4>(F.w[j]), acc[0][fi][j]);
      } else {
        v4i ap, an;
        split(a, ap, an);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const v4i b = operand<W4>(F.w[j]);
          acc[0][fi][j] = mfma(ap, b, acc[0][fi][j]);
          acc[1][fi][j] = mfma(an, b, acc[1][fi][j]);
        }
      }
    }
  };

  const int nk = (g.K + BK - 1) / BK;
  // prologue: stages 0 .. kStages-2 in flight, stage 0 landed
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nk) issue(s, slots[s]);
  if (nk >= kStages - 1)
    wait_vmcnt<(kStages - 2) * Lay::kLoadsPerStage>();
  else
    wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  Frags F[2];
  read_all(F[0], slots[0]);

  // One K step: wait for stage k+1, barrier, refill the ring, prefetch the
  // fragments of stage k+1, run the MFMAs of stage k. u = k % kStages is a
  // compile-time constant at every call site (the loops below are unrolled
  // by the ring depth), so slots and fragment buffers are static.
  auto step = [&](int k, auto uc) {
    constexpr int u = decltype(uc)::value;
    if (k + kStages - 2 < nk)
      wait_vmcnt<(kStages - 3) * Lay::kLoadsPerStage>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // stage k+1 visible to all; slot of k-1 free
    if (k + kStages - 1 < nk) issue(k + kStages - 1, slots[(u + kStages - 1) % kStages]);
    // (on the last step this reads a stale slot; the values are never used)
    read_all(F[(u + 1) & 1], slots[(u + 1) % kStages]);
    compute(F[u & 1]);
  };
  int kb = 0;
  for (; kb + kStages <= nk; kb += kStages) {
    step(kb + 0, IC<0>{});
    step(kb + 1, IC<1>{});
    step(kb + 2, IC<2>{});
    step(kb + 3, IC<3>{});
    step(kb + 4, IC<4>{});
    step(kb + 5, IC<5>{});
  }
  if (kb + 0 < nk) step(kb + 0, IC<0>{});
  if (kb + 1 < nk) step(kb + 1, IC<1>{});
  if (kb + 2 < nk) step(kb + 2, IC<2>{});
  if (kb + 3 < nk) step(kb + 3, IC<3>{});
  if (kb + 4 < nk) step(kb + 4, IC<4>{});

  // ---- epilogue ----
  const float sp = g.act_scales[0];
  const float sn = g.act_scales[1];
  const int rsub = (lane >> 4) * 4;
  float sw[NB];
  int col[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    col[j] = n0 + 16 * j + i16;
    sw[j] = col[j] < g.N ? g.w_scales[col[j]] : 0.0f;
  }

  auto grow_of = [&](int fi, int i, bool& ok) {
    const int f = 2 * wave + fi;
    if constexpr (CFG) {
      const int crow = m0 + 16 * (f >> 1) + i;
      ok = crow < g.Mh;
      return crow + (f & 1) * g.Mh;
    } else {
      const int r = m0 + 16 * f + i;
      ok = r < g.M;
      return r;
    }
  };

  if constexpr (DBG) {
    const int64_t plane = (int64_t)g.M * g.N;
#pragma unroll
    for (int fi = 0; fi < 2; ++fi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bool ok;
        const int grow = grow_of(fi, rsub + r, ok);
        if (!ok) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (col[j] >= g.N) continue;
          const int64_t e = (int64_t)grow * g.N + col[j];
          g.dbg[e] = acc[0][fi][j][r] >> SHIFT;
          g.dbg[plane + e] = SYM ? 0 : (acc[NP - 1][fi][j][r] >> SHIFT);
        }
      }
  }

  if constexpr (CFG) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int crow = m0 + 16 * wave + rsub + r;
      if (crow >= g.Mh) continue;
      float* yrow = g.Y + (int64_t)crow * g.N;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (col[j] >= g.N) continue;
        const float yc = epi<SYM>(acc[0][0][j][r] >> SHIFT, acc[NP - 1][0][j][r] >> SHIFT, sp, sn,
                                  sw[j], g.inv_b);
        const float yu = epi<SYM>(acc[0][1][j][r] >> SHIFT, acc[NP - 1][1][j][r] >> SHIFT, sp, sn,
                                  sw[j], g.inv_b);
        const float d = __fsub_rn(yc, yu);
        const float tt = __fmul_rn(g.guidance, d);
        yrow[col[j]] = __fadd_rn(yu, tt);
      }
    }
  } else {
#pragma unroll
    for (int fi = 0; fi < 2; ++fi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bool ok;
        const int grow = grow_of(fi, rsub + r, ok);
        if (!ok) continue;
        float* yrow = g.Y + (int64_t)grow * g.N;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (col[j] >= g.N) continue;
          yrow[col[j]] = epi<SYM>(acc[0][fi][j][r] >> SHIFT, acc[NP - 1][fi][j][r] >> SHIFT, sp,
                                  sn, sw[j], g.inv_b);
        }
      }
  }
}

template <bool A4, bool W4, bool SYM, bool CFG, int NB>
hipError_t run(const GemmArgs& g, hipStream_t s) {
  const int rows = CFG ? g.Mh : g.M;
  const int rt = (rows + (CFG ? 63 : 127)) / (CFG ? 64 : 128);
  const int ct = (g.N + 16 * NB - 1) / (16 * NB);
  const dim3 grid(rt * ct);
  if (g.dbg)
    hipLaunchKernelGGL((k2_gemm<A4, W4, SYM, CFG, true, NB>), grid, dim3(kThreads), 0, s, g);
  else
    hipLaunchKernelGGL((k2_gemm<A4, W4, SYM, CFG, false, NB>), grid, dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

template <bool A4, bool W4, bool SYM, bool CFG>
hipError_t run_nb(const GemmArgs& g, hipStream_t s) {
  // 144-column tiles when they divide N, else 128.
  if (g.N % 144 == 0) return run<A4, W4, SYM, CFG, 9>(g, s);
  return run<A4, W4, SYM, CFG, 8>(g, s);
}

template <bool A4, bool W4>
hipError_t run_mode(const GemmArgs& g, int sym, int cfg, hipStream_t s) {
  if (sym) return cfg ? run_nb<A4, W4, true, true>(g, s) : run_nb<A4, W4, true, false>(g, s);
  return cfg ? run_nb<A4, W4, false, true>(g, s) : run_nb<A4, W4, false, false>(g, s);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, int a4, int w4, int sym, int cfg, hipStream_t s) {
  if (a4) return w4 ? run_mode<true, true>(g, sym, cfg, s) : run_mode<true, false>(g, sym, cfg, s);
  return w4 ? run_mode<false, true>(g, sym, cfg, s) : run_mode<false, false>(g, sym, cfg, s);
}

}  // namespace ql
