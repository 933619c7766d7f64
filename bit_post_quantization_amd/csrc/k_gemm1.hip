// K2: integer GEMM of the activation codes against the weight codes on the
// int8 matrix cores of gfx950, both DualScale polarity planes in one kernel,
// with the fp32 epilogue (scales, input-branch sum, Hadamard normalisation,
// CFG combine) fused. Serves every plan but the single-Hadamard one.
//
// Method (pages): SegQuant explainer 2.B -- X is split into its
// non-negative and negative parts, each multiplied by the weight codes; the
// two products run side by side in one batched kernel and their rescaled
// results are summed in the epilogue. SegQuant explainer 2.A -- input
// segmentation: each input branch has its own scales, and the branch
// products are summed. TASQ explainer, technical summary 2 -- one stored
// weight buffer; a layer's operating precision at a stage drops k low bits
// of every stored code. "Closing the Null Space" explainer, problem
// statement -- guided output uncond + w (cond - uncond).
//
// Design for CDNA4 (MI355X):
//  * v_mfma_i32_16x16x64_i8; each activation fragment is split in registers
//    into its non-negative plane, and both the full codes and that plane are
//    multiplied by the same weight fragment (two accumulator sets).
//  * 4 waves, one per SIMD, so each wave has the whole register file:
//    accumulators in AGPRs, operands and prefetch in VGPRs. A tile is 128
//    activation rows x 16*NB weight rows; wave w owns 32 activation rows
//    (with CFG: 16 conditional rows and their 16 unconditional partners)
//    against all NB weight fragments, so each weight fragment read from LDS
//    feeds 4 MFMAs (DualScale) and a step reads 4 x NB x 2 KB of weights and
//    4 x 4 KB of activations per CU.
//  * Both operands go HBM -> LDS by buffer_load ... lds into a ring of 3
//    step slots, loads two to three steps ahead of the MFMAs, issued one per
//    weight fragment between the MFMAs (a single wave issues in order: a
//    burst of loads would stall its matrix core).
//  * Weight transform stage: 4-bit weights are stored packed, two codes per
//    byte, and TASQ's operating precision is a per-call depth k over the one
//    stored buffer. Each wave unpacks (x16, see unpack4_x16) and/or masks
//    the weight bytes its own DMA brought into the ring, in LDS, half a step
//    before the barrier that publishes them, so every weight byte is
//    transformed once per workgroup, not once per reading wave.
//  * Persistent workgroups walking XCD-banded tile lists as one continuous
//    stream of K steps, so the loads of a tile's first steps overlap the
//    previous tile's epilogue. Input branches are padded to whole ring
//    cycles of steps; at a branch end its epilogue part is added, in branch
//    order, to fp32 sums kept in registers, and the accumulators restart.
//  * Out-of-range rows and K chunks read as zero (buffer range checks and
//    explicit out-of-range offsets), so ragged M, N and K need no special
//    path.
#include <type_traits>

#include "ql_device.h"
#include "ql_kernels.h"

#if !defined(QL_G1_A4) || !defined(QL_G1_SYM)
#error "k_gemm1.hip is compiled once per (QL_G1_A4, QL_G1_SYM) pair"
#endif

namespace ql {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
template <int V>
using IC = std::integral_constant<int, V>;

constexpr int kThreads = 256;
constexpr int BK = 128;                 // K elements per step
constexpr int kStages = 3;              // LDS ring depth (= unroll of the step loop)
constexpr unsigned kOOB = 0x80000000u;  // offset beyond every buffer: loads return 0

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

// lgkmcnt-only wait.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// LDS image of one int8 fragment pair (16 rows x 128 K = the two 16 x 64
// MFMA operands of a step), 2 KB: row r, 16-byte chunk c (elements 16c ..
// 16c+15) sits at at(r, c). Filled by two DMA instructions of 1 KB: DMA lane
// p of instruction i loads row 8i + p/8, chunk (p%8) ^ ((row/2)%8) (8 lanes
// read one whole 128-byte line), which lands at i*1024 + p*16. MFMA lane l
// of half h (row l%16, chunk 4h + l/16) finds its 16 bytes at the same
// swizzled place; the 16 lanes reading together hit 16 distinct bank groups.
struct WFrag {
  __device__ static __forceinline__ int at(int r, int c) {
    return (r >> 3) * 1024 + (8 * (r & 7) + (c ^ ((r >> 1) & 7))) * 16;
  }
  __device__ static __forceinline__ int dma_row(int i, int p) { return 8 * i + (p >> 3); }
  __device__ static __forceinline__ int dma_chunk(int i, int p) {
    return (p & 7) ^ ((dma_row(i, p) >> 1) & 7);
  }
  __device__ static __forceinline__ int read_off(int l, int h) { return at(l & 15, 4 * h + (l >> 4)); }
};

// LDS image of one packed 4-bit activation fragment pair (16 rows x 128 K
// = 64 bytes per row), 1 KB, one DMA instruction: lane p loads row p/4,
// 16-byte chunk (p%4) ^ ((p/16)%4) of the row; MFMA lane l of half h reads
// the 8 bytes of element group 4h + l/16 (half of one of those chunks).
struct PFrag {
  __device__ static __forceinline__ int dma_row(int, int p) { return p >> 2; }
  __device__ static __forceinline__ int dma_chunk(int, int p) {
    return (p & 3) ^ ((p >> 4) & 3);
  }
  __device__ static __forceinline__ int read_off(int l, int h) {
    const int r = l & 15;
    const int e = 4 * h + (l >> 4);
    return (4 * r + ((e >> 1) ^ ((r >> 2) & 3))) * 16 + (e & 1) * 8;
  }
};

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Non-negative polarity plane of an operand (negative bytes zeroed).
__device__ __forceinline__ v4i positive(v4i c) {
  v4i p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = (int)pos_plane((uint32_t)c[i]);
  return p;
}

// y from the two accumulators in the documented order, no contraction.
template <bool SYM>
__device__ __forceinline__ float epi_part(int accp, int accn, float sp, float sn, float sw) {
  if constexpr (SYM) {
    return __fmul_rn(__fmul_rn((float)accp, sp), sw);
  } else {
    const float tp = __fmul_rn((float)accp, sp);
    const float tn = __fmul_rn((float)accn, sn);
    return __fmul_rn(__fadd_rn(tp, tn), sw);
  }
}

// Tiles of workgroup b. When grid and tile counts divide by 8, each XCD
// (workgroup id mod 8) owns a band of consecutive tiles; when that band is
// R whole tile rows and its workgroups divide into R rows of C columns, the
// workgroups run the band as successive R x C blocks, so the concurrent
// tiles of an XCD share R activation row panels and C weight panels in its
// L2. Otherwise tiles are taken in row-major order within the band, or
// strided over the grid.
struct TileList {
  int first, stride, count;
  int ct, C;
  int row0, r, c;
  __device__ __forceinline__ int at(int i) const {
    if (C) return (row0 + r) * ct + i * C + c;
    return first + i * stride;
  }
};

__device__ __forceinline__ TileList my_tiles(int T, int ct) {
  const int G = gridDim.x, b = blockIdx.x;
  TileList L;
  L.C = 0;
  L.ct = ct;
  if ((G & 7) == 0 && (T & 7) == 0) {
    const int x = b & 7, j = b >> 3, per_x = G >> 3, band = T >> 3;
    L.first = x * band + j;
    L.stride = per_x;
    L.count = j < band ? (band - j + per_x - 1) / per_x : 0;
    if (band % ct == 0 && band % per_x == 0) {
      const int R = band / ct;
      if (per_x % R == 0 && ct % (per_x / R) == 0) {
        L.C = per_x / R;
        L.row0 = x * R;
        L.r = j / L.C;
        L.c = j % L.C;
        L.count = band / per_x;
      }
    }
  } else {
    L.first = b;
    L.stride = G;
    L.count = b < T ? (T - b + G - 1) / G : 0;
  }
  return L;
}

// Weight formats of the ring.
constexpr int kWInt8 = 0;          // int8 codes, used as loaded
constexpr int kWPacked4 = 1;       // 4-bit codes two per byte, unpacked x16 in LDS
constexpr int kWMasked8 = 2;       // int8 codes, TASQ mask applied in LDS
constexpr int kWPacked4Masked = 3; // 4-bit codes, unpacked and masked in LDS

// Bytes of one ring slot: the activation fragment pairs of the 4 waves, the
// NB int8 weight fragment images, and (packed 4-bit weights) the NB packed
// fragments as loaded.
template <bool A4, int WX, int NB>
struct Slot {
  static constexpr int kAFrag = A4 ? 1024 : 2048;  // one activation fragment pair
  static constexpr int kA = 4 * 2 * kAFrag;        // 4 waves x 2 fragments
  static constexpr int kW = NB * 2048;
  static constexpr int kStage = (WX == kWPacked4 || WX == kWPacked4Masked) ? NB * 1024 : 0;
  static constexpr int kBytes = kA + kW + kStage;
};

// Weight-scale ring: 4 tiles x branches (1 or 2) x 256 floats.
template <bool KS>
struct ScaleRing {
  static constexpr int kBranches = KS ? 2 : 1;
  static constexpr int kFloats = 4 * kBranches * 256;
};

// The work of one wave. Wave w moves weight fragments w and w + 4; XI >= 0:
// it also moves DMA instruction XI of fragment 8, which waves 0 and 1 share
// for int8 weights (one instruction each) and wave 0 moves for packed ones.
// (A compile-time XI keeps every LDS address of the wave's transform
// provably apart from the DMAs in flight; with a run-time index the compiler
// waits for all of them.)
template <bool A4, bool SYM, bool CFG, int WX, bool KS, int NB, int XI>
__device__ __forceinline__ void gemm_wave(const GemmArgs& g, int wave, int lane, uint8_t* st0,
                                          uint8_t* st1, uint8_t* st2, float* sring) {
  using SL = Slot<A4, WX, NB>;
  constexpr bool W4 = WX == kWPacked4 || WX == kWPacked4Masked;
  constexpr bool MASK = WX == kWMasked8 || WX == kWPacked4Masked;
  constexpr int NP = SYM ? 1 : 2;                    // accumulator planes
  constexpr int SHIFT = (A4 ? 4 : 0) + (W4 ? 4 : 0);  // undo the x16 unpacks
  constexpr int BN = 16 * NB;
  constexpr int RPT = CFG ? 64 : 128;    // output rows per tile
  constexpr int kALoads = A4 ? 1 : 2;    // DMA instructions per activation fragment pair
  constexpr int kWLoads = W4 ? 1 : 2;    // DMA instructions per weight fragment
  constexpr int kOpsA = 2 * kALoads;
  constexpr bool XW = XI >= 0;
  constexpr int kOpsW = 2 * kWLoads + (XW ? 1 : 0);
  constexpr int kOps = kOpsA + kOpsW;    // vector-memory instructions per step and wave
  constexpr int kSR = ScaleRing<KS>::kBranches;
  static_assert(NB >= 8 && NB <= 9, "weight fragments per tile");
  uint8_t* const slots[kStages] = {st0, st1, st2};

  const int nks = KS ? g.nks : 1;
  const int ct = (g.N + BN - 1) / BN;
  const int T = (((CFG ? g.Mh : g.M) + RPT - 1) / RPT) * ct;
  const TileList tl = my_tiles(T, ct);
  if (tl.count == 0) return;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)((int64_t)g.M * g.lda));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.W, (uint32_t)((int64_t)g.N * g.ldw));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.w_scales, (uint32_t)(nks * g.N) * 4u);

  auto coords = [&](int ti, int& m0, int& n0) __attribute__((always_inline)) {
    const int t = tl.at(ti);
    const int tr = t / ct;
    m0 = tr * RPT;
    n0 = (t - tr * ct) * BN;
  };
  // Global row of row i (0..15) of this wave's activation fragment fi: with
  // CFG, fragment 0 holds conditional rows and fragment 1 their partners.
  auto a_row = [&](int m0, int fi, int i, bool& ok) __attribute__((always_inline)) {
    if constexpr (CFG) {
      const int crow = m0 + 16 * wave + i;
      ok = crow < g.Mh;
      return crow + fi * g.Mh;
    } else {
      const int r = m0 + 32 * wave + 16 * fi + i;
      ok = r < g.M;
      return r;
    }
  };
  // Steps of branch j (a multiple of the ring depth) and its K range (j is
  // 0 or 1; selected, not indexed: an array of the kernel's arguments
  // indexed at run time would go through scratch).
  auto ksteps = [&](int j) __attribute__((always_inline)) {
    return KS && j ? g.ksteps[1] : g.ksteps[0];
  };
  auto kbeg = [&](int j) __attribute__((always_inline)) { return KS && j ? g.kofs[1] : 0; };
  auto kend = [&](int j) __attribute__((always_inline)) {
    return KS && !j ? g.kofs[1] : g.K;
  };

  const int i16 = lane & 15;
  const int q4 = lane >> 4;

  // ---- load streams: one cursor (tile, branch, step) per operand, both
  // two to three steps ahead of the MFMAs (the step s of the stream goes
  // into ring slot s % 3). Entering a tile, wave 0 also moves the tile's
  // 16*NB weight scales of every branch into entry ti % 4 of a small LDS
  // ring (16 bytes per lane; columns past N read as 0); the tile's folds
  // and epilogue read them there. Entry ti % 4 is refilled for tile ti + 4
  // at least one step after the epilogue of tile ti.
  int w_ti = 0, w_j = 0, w_k = 0, a_ti = 0, a_j = 0, a_k = 0;
  unsigned wv[kOpsW], av[2][2];
  // Weight DMA instruction o of this wave: fragment and instruction index.
  auto w_frag = [&](int o) __attribute__((always_inline)) {
    return o < 2 * kWLoads ? wave + 4 * (o / kWLoads) : 8;
  };
  auto w_inst = [&](int o) __attribute__((always_inline)) {
    return o < 2 * kWLoads ? o % kWLoads : XI;
  };
  auto w_enter = [&](int ti) __attribute__((always_inline)) {
    int m0, n0;
    coords(ti, m0, n0);
    if (wave == 0) {
      const unsigned v = 16u * (unsigned)lane < 4u * (unsigned)BN ? 16u * (unsigned)lane : kOOB;
      for (int j = 0; j < nks; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_void*)(sring + ((ti & 3) * kSR + j) * 256), 16, v,
            4u * (unsigned)(j * g.N + n0), 0, 0);
    }
#pragma unroll
    for (int o = 0; o < kOpsW; ++o) {
      const int f = w_frag(o), i = w_inst(o);
      if constexpr (W4) {
        const int n = n0 + 16 * f + (lane >> 2);
        wv[o] = n < g.N ? (unsigned)n * (unsigned)g.ldw + 16u * (unsigned)(lane & 3) : kOOB;
      } else {
        const int n = n0 + 16 * f + WFrag::dma_row(i, lane);
        wv[o] = n < g.N ? (unsigned)n * (unsigned)g.ldw + 16u * (unsigned)WFrag::dma_chunk(i, lane)
                        : kOOB;
      }
    }
  };
  auto a_enter = [&](int ti) __attribute__((always_inline)) {
    int m0, n0;
    coords(ti, m0, n0);
#pragma unroll
    for (int fi = 0; fi < 2; ++fi)
#pragma unroll
      for (int i = 0; i < kALoads; ++i) {
        const int row = A4 ? PFrag::dma_row(i, lane) : WFrag::dma_row(i, lane);
        const int chunk = A4 ? PFrag::dma_chunk(i, lane) : WFrag::dma_chunk(i, lane);
        bool ok;
        const int r = a_row(m0, fi, row, ok);
        av[fi][i] = ok ? (unsigned)r * (unsigned)g.lda + 16u * (unsigned)chunk : kOOB;
      }
  };
  // One DMA instruction of each stream's current step (chunks past the end
  // of the branch read zeros): weight instruction o of this wave;
  // activation fragment fi of this wave, instruction i.
  auto w_dst = [&](uint8_t* slot, int o) __attribute__((always_inline)) {
    if constexpr (W4)
      return slot + SL::kA + SL::kW + w_frag(o) * 1024;
    else
      return slot + SL::kA + w_frag(o) * 2048 + w_inst(o) * 1024;
  };
  auto w_op = [&](uint8_t* slot, int o) __attribute__((always_inline)) {
    const int k0 = kbeg(w_j) + w_k * BK;
    const int ke = kend(w_j);
    unsigned v = wv[o];
    if constexpr (W4) {
      if (k0 + BK > ke && k0 + 32 * (lane & 3) >= ke) v = kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)w_dst(slot, o), 16, v,
                                               (unsigned)k0 / 2u, 0, 0);
    } else {
      if (k0 + BK > ke && k0 + 16 * WFrag::dma_chunk(w_inst(o), lane) >= ke) v = kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)w_dst(slot, o), 16, v,
                                               (unsigned)k0, 0, 0);
    }
  };
  auto a_op = [&](uint8_t* slot, int fi, int i) __attribute__((always_inline)) {
    const int k0 = kbeg(a_j) + a_k * BK;
    const int ke = kend(a_j);
    unsigned v = av[fi][i];
    const int chunk = A4 ? PFrag::dma_chunk(i, lane) : WFrag::dma_chunk(i, lane);
    if (k0 + BK > ke && k0 + (A4 ? 32 : 16) * chunk >= ke) v = kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ra, (lds_void*)(slot + (2 * wave + fi) * SL::kAFrag + i * 1024), 16, v,
        (unsigned)k0 / (A4 ? 2u : 1u), 0, 0);
  };
  auto w_advance = [&]() __attribute__((always_inline)) {
    if (++w_k < ksteps(w_j)) return;
    w_k = 0;
    if (KS && ++w_j < nks) return;
    w_j = 0;
    if (++w_ti < tl.count) {
      w_enter(w_ti);
    } else {
#pragma unroll
      for (int o = 0; o < kOpsW; ++o) wv[o] = kOOB;
    }
  };
  auto a_advance = [&]() __attribute__((always_inline)) {
    if (++a_k < ksteps(a_j)) return;
    a_k = 0;
    if (KS && ++a_j < nks) return;
    a_j = 0;
    if (++a_ti < tl.count) {
      a_enter(a_ti);
    } else {
#pragma unroll
      for (int fi = 0; fi < 2; ++fi)
#pragma unroll
        for (int i = 0; i < kALoads; ++i) av[fi][i] = kOOB;
    }
  };
  // Load o of a step (of kOps): weights and activations alternate while
  // both have loads left.
  auto load_op = [&](uint8_t* slot, int o) __attribute__((always_inline)) {
    constexpr int kMin = kOpsW < kOpsA ? kOpsW : kOpsA;
    if (o < 2 * kMin) {
      if (o % 2 == 0)
        w_op(slot, o / 2);
      else
        a_op(slot, (o / 2) / kALoads, (o / 2) % kALoads);
    } else {
      const int k = kMin + (o - 2 * kMin);
      if (kOpsW > kOpsA)
        w_op(slot, k);
      else
        a_op(slot, k / kALoads, k % kALoads);
    }
  };
  auto issue_all = [&](uint8_t* slot) __attribute__((always_inline)) {
#pragma unroll
    for (int o = 0; o < kOps; ++o) load_op(slot, o);
    w_advance();
    a_advance();
  };

  // ---- weight transform: unit t = weight DMA instruction t of this wave
  // (16 bytes per lane), read back by the lane that loaded it, transformed,
  // and written as int8 image bytes.
  constexpr int kTUnits = WX == kWInt8 ? 0 : kOpsW;
  uint32_t mlut = 0, mkeep = 0xFFFFFFFFu;
  if constexpr (MASK) {
    const int kk = g.w_lsb_k + (W4 ? 4 : 0);  // x16 codes: k + 4 low bits
    mlut = ((1u << kk) - 1u) << 8;
    mkeep = 0x01010101u * (0xFFu & ~((1u << kk) - 1u));
  }
  auto t_src = [&](const uint8_t* slot, int t) __attribute__((always_inline)) {
    return (const v4u*)w_dst(const_cast<uint8_t*>(slot), t);
  };
  // Output dwords of input dword d of a unit: 2 (unpacked) or 1.
  constexpr int kOutPer = W4 ? 2 : 1;
  v4u tin[kTUnits > 0 ? kTUnits : 1];
  uint32_t tout[kTUnits > 0 ? kTUnits : 1][4 * kOutPer];
  auto t_dword = [&](int t, int d) __attribute__((always_inline)) {
    const uint32_t x = tin[t][d];
    if constexpr (W4) {
      unpack4_x16(x, tout[t][2 * d], tout[t][2 * d + 1]);
      if constexpr (MASK) {
        tout[t][2 * d] = trunc_mag4(tout[t][2 * d], mlut, mkeep);
        tout[t][2 * d + 1] = trunc_mag4(tout[t][2 * d + 1], mlut, mkeep);
      }
    } else {
      tout[t][d] = trunc_mag4(x, mlut, mkeep);
    }
  };
  auto t_write = [&](uint8_t* slot, int t) __attribute__((always_inline)) {
    if constexpr (W4) {
      // lane p holds elements 32 (p%4) .. +31 of row p/4: image chunks
      // 2 (p%4) and 2 (p%4) + 1 of that row
      uint8_t* img = slot + SL::kA + w_frag(t) * 2048;
      const int r = lane >> 2, c = 2 * (lane & 3);
      *reinterpret_cast<v4u*>(img + WFrag::at(r, c)) =
          v4u{tout[t][0], tout[t][1], tout[t][2], tout[t][3]};
      *reinterpret_cast<v4u*>(img + WFrag::at(r, c + 1)) =
          v4u{tout[t][4], tout[t][5], tout[t][6], tout[t][7]};
    } else {
      *reinterpret_cast<v4u*>(w_dst(slot, t) + lane * 16) =
          v4u{tout[t][0], tout[t][1], tout[t][2], tout[t][3]};
    }
  };
  // Spread over a half step: every unit read after the first weight
  // fragment's MFMAs; its 4 input dwords transformed a few at a time
  // after fragments 1 .. NB-1 (the VALU work interleaves with the MFMAs
  // instead of stalling them); a unit written once its last dword is done.
  auto xform = [&](uint8_t* slot, int jj) __attribute__((always_inline)) {
    if constexpr (kTUnits > 0) {
      constexpr int D = 4 * kTUnits;
      if (jj == 0) {
#pragma unroll
        for (int t = 0; t < kTUnits; ++t) tin[t] = *(t_src(slot, t) + lane);
      } else {
        const int lo = D * (jj - 1) / (NB - 1), hi = D * jj / (NB - 1);
#pragma unroll
        for (int d = 0; d < D; ++d)
          if (d >= lo && d < hi) {
            t_dword(d / 4, d % 4);
            if (d % 4 == 3) t_write(slot, d / 4);
          }
      }
    }
  };
  auto xform_all = [&](uint8_t* slot) __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) xform(slot, jj);
  };

  // ---- operands ----
  const int rw0 = WFrag::read_off(lane, 0), rw1 = WFrag::read_off(lane, 1);
  const int ra0 = A4 ? PFrag::read_off(lane, 0) : rw0, ra1 = A4 ? PFrag::read_off(lane, 1) : rw1;
  typedef typename std::conditional<A4, v2u, v4u>::type araw;
  auto a_read = [&](const uint8_t* slot, int fi, int h) __attribute__((always_inline)) {
    return *reinterpret_cast<const araw*>(slot + (2 * wave + fi) * SL::kAFrag + (h ? ra1 : ra0));
  };
  auto operand = [&](const araw& r) __attribute__((always_inline)) {
    v4i o;
    if constexpr (A4) {
      uint32_t a, b, c, e;
      unpack4_x16(r.x, a, b);
      unpack4_x16(r.y, c, e);
      o[0] = (int)a;
      o[1] = (int)b;
      o[2] = (int)c;
      o[3] = (int)e;
    } else {
      o[0] = (int)r.x;
      o[1] = (int)r.y;
      o[2] = (int)r.z;
      o[3] = (int)r.w;
    }
    return o;
  };
  // The weight fragments of the half step being computed; each fragment's
  // registers are refilled with the next half's fragment right after its
  // last MFMA.
  v4i WB[NB];
  auto read_wb = [&](const uint8_t* slot, int h) __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < NB; ++jj)
      WB[jj] = *reinterpret_cast<const v4i*>(slot + SL::kA + jj * 2048 + (h ? rw1 : rw0));
  };
  // MFMA operands of one half step: the codes of both activation fragments
  // and (DualScale) their non-negative planes.
  struct Opnd {
    v4i x[2], xp[2];
  };
  Opnd OP[2];
  auto prep = [&](Opnd& o, int fi, const araw& r) __attribute__((always_inline)) {
    o.x[fi] = operand(r);
    if constexpr (!SYM) o.xp[fi] = positive(o.x[fi]);
  };

  // DUAL: acc[0] = sum pos(c) w, acc[1] = sum c w (acc- = acc[1] - acc[0]).
  v4i acc[NP][2][NB];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int fi = 0; fi < 2; ++fi)
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) acc[p][fi][jj] = v4i{0, 0, 0, 0};
  };
  // Keep the accumulators in AGPRs across steps (an empty asm statement that
  // takes and returns them in AGPRs): the loop then carries them where the
  // MFMAs read and write them, with no copies.
  auto pin_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int fi = 0; fi < 2; ++fi)
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) asm volatile("" : "+a"(acc[p][fi][jj]));
  };

  // One half step: per weight fragment jj, its MFMAs with both activation
  // fragments (full codes and, DualScale, the non-negative plane), then the
  // read that refills its registers with fragment jj of the next half (from
  // `wslot`, half `nh`); the next half's activation fragments are read from
  // `aslot` after the first fragment and prepared after the third; hook(jj)
  // (a load of a later step, a piece of the weight transform, or nothing)
  // runs after fragment jj. Scheduling barriers keep this order.
  auto compute_half = [&](const Opnd& op, Opnd& on, const uint8_t* aslot, const uint8_t* wslot,
                          int nh, auto&& hook) __attribute__((always_inline)) {
    araw an[2];
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) {
#pragma unroll
      for (int fi = 0; fi < 2; ++fi)
        acc[NP - 1][fi][jj] = mfma(op.x[fi], WB[jj], acc[NP - 1][fi][jj]);
      if constexpr (!SYM) {
#pragma unroll
        for (int fi = 0; fi < 2; ++fi) acc[0][fi][jj] = mfma(op.xp[fi], WB[jj], acc[0][fi][jj]);
      }
      WB[jj] = *reinterpret_cast<const v4i*>(wslot + SL::kA + jj * 2048 + (nh ? rw1 : rw0));
      if (jj == 0) {
        an[0] = a_read(aslot, 0, nh);
        an[1] = a_read(aslot, 1, nh);
      }
      if (jj == 2) prep(on, 0, an[0]);
      if (jj == 3) prep(on, 1, an[1]);
      hook(jj);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int rsub = q4 * 4;
  // Activation scales of both branches, loaded once before the load stream
  // starts (a load here waits on every DMA in flight: vmcnt counts in order).
  const float asc[4] = {g.act_scales[0], g.act_scales[1], KS ? g.act_scales[2] : 0.0f,
                        KS ? g.act_scales[3] : 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(asc[i]));  // consumed here, not in a tile
  auto sp_of = [&](int j) __attribute__((always_inline)) { return KS && j ? asc[2] : asc[0]; };
  auto sn_of = [&](int j) __attribute__((always_inline)) { return KS && j ? asc[3] : asc[1]; };

  // Accumulator element r of slot (p, fi, jj), read out of its AGPR.
  auto acc_at = [&](int p, int fi, int jj, int r) __attribute__((always_inline)) {
    int v;
    const v4i a = acc[p][fi][jj];
    switch (r) {
      case 0: asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a.x)); break;
      case 1: asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a.y)); break;
      case 2: asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a.z)); break;
      default: asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a.w)); break;
    }
    return v;
  };
  auto accs = [&](int fi, int jj, int r, int& ap, int& an) __attribute__((always_inline)) {
    const int a0 = acc_at(0, fi, jj, r);
    ap = a0 >> SHIFT;
    if constexpr (SYM)
      an = 0;
    else
      an = (acc_at(NP - 1, fi, jj, r) - a0) >> SHIFT;
  };
  // The epilogue part of branch j for accumulator element (fi, jj, r).
  auto ypart = [&](const float* sw, float sp, float sn, int fi, int jj, int r)
      __attribute__((always_inline)) {
    int ap, an;
    accs(fi, jj, r, ap, an);
    return epi_part<SYM>(ap, an, sp, sn, sw[jj]);
  };
  auto load_sw = [&](int ti, int j, float* sw) __attribute__((always_inline)) {
    static_assert(NB == 9, "scale reads");
    lds_read9_stride16(sring + ((ti & 3) * kSR + j) * 256 + i16, sw);
  };
  auto dump = [&](int m0, const unsigned* coff, int j) __attribute__((always_inline)) {
    // accumulator dump (testing aid): planes (acc+, acc-) of branch j in [2 nks, M, N]
    const int64_t plane = (int64_t)g.M * g.N;
#pragma unroll
    for (int fi = 0; fi < 2; ++fi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bool ok;
        const int grow = a_row(m0, fi, rsub + r, ok);
        if (!ok) continue;
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
          if (coff[jj] == kOOB) continue;
          const int64_t e = (int64_t)grow * g.N + (coff[jj] >> 2);
          int ap, an;
          accs(fi, jj, r, ap, an);
          g.dbg[2 * j * plane + e] = ap;
          g.dbg[(2 * j + 1) * plane + e] = an;
        }
      }
  };
  auto col_offsets = [&](int n0, unsigned* coff) __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) {
      const int col = n0 + 16 * jj + i16;
      coff[jj] = col < g.N ? 4u * (unsigned)col : kOOB;
    }
  };

  // Input branches (two): fp32 sums of the first branch's epilogue parts,
  // kept in AGPRs beside the accumulators (the VGPRs hold the operand
  // pipeline), pinned there like the accumulators.
  constexpr int kYS = KS ? 2 * NB * 4 : 1;
  float ysum[kYS];
  auto pin_ys = [&]() __attribute__((always_inline)) {
    if constexpr (KS) {
#pragma unroll
      for (int i = 0; i < kYS; ++i) asm volatile("" : "+a"(ysum[i]));
    }
  };
  auto ys_get = [&](int i) __attribute__((always_inline)) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(ysum[i]));
    return v;
  };
  auto ys_set = [&](int i, float v) __attribute__((always_inline)) {
    asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(ysum[i]) : "v"(v));
  };
  if constexpr (KS) {
#pragma unroll
    for (int i = 0; i < kYS; ++i) ys_set(i, 0.0f);
  }
  // End of the first input branch j = 0 of tile ti: its epilogue parts
  // start the sums; the caller restarts the accumulators.
  auto fold = [&](int ti, int j) __attribute__((always_inline)) {
    if constexpr (KS) {
      float sw[NB];
      load_sw(ti, j, sw);
      const float spj = sp_of(j), snj = sn_of(j);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int fi = 0; fi < 2; ++fi)
#pragma unroll
          for (int jj = 0; jj < NB; ++jj) {
            const int i = (fi * NB + jj) * 4 + r;
            const float y = ypart(sw, spj, snj, fi, jj, r);
            ys_set(i, y);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (g.dbg) {
        int m0, n0;
        coords(ti, m0, n0);
        unsigned coff[NB];
        col_offsets(n0, coff);
        dump(m0, coff, j);
      }
    }
  };

  // Tile epilogue (after the last branch j): y = (branch sums) * 1/B, then
  // CFG; outputs go out through range-checked buffer stores (rows past the
  // end and columns past N are dropped by the range check), one accumulator
  // row at a time so the working set stays small.
  auto epilogue = [&](int ti, int j) __attribute__((always_inline)) {
    int m0, n0;
    coords(ti, m0, n0);
    float sw[NB];
    unsigned coff[NB];
    load_sw(ti, j, sw);
    col_offsets(n0, coff);
    const float spj = sp_of(j), snj = sn_of(j);
    auto yout = [&](int fi, int jj, int r) __attribute__((always_inline)) {
      float y = ypart(sw, spj, snj, fi, jj, r);
      if constexpr (KS) y = __fadd_rn(ys_get((fi * NB + jj) * 4 + r), y);
      return __fmul_rn(y, g.inv_b);
    };
    const int rows_here = min(RPT, (CFG ? g.Mh : g.M) - m0);
    const __amdgpu_buffer_rsrc_t ry =
        make_rsrc(g.Y + (int64_t)m0 * g.N, (uint32_t)rows_here * (uint32_t)g.N * 4u);
    const unsigned rowb = (unsigned)g.N * 4u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (CFG) {
        const unsigned ro = (unsigned)(16 * wave + rsub + r) * rowb;
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
          const float yc = yout(0, jj, r);
          const float yu = yout(1, jj, r);
          const float d = __fsub_rn(yc, yu);
          const float t = __fmul_rn(g.guidance, d);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(__fadd_rn(yu, t)), ry,
                                                ro + coff[jj], 0, 0);
        }
      } else {
#pragma unroll
        for (int fi = 0; fi < 2; ++fi) {
          const unsigned ro = (unsigned)(32 * wave + 16 * fi + rsub + r) * rowb;
#pragma unroll
          for (int jj = 0; jj < NB; ++jj)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yout(fi, jj, r)), ry,
                                                  ro + coff[jj], 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (g.dbg) dump(m0, coff, j);
  };

  // Prologue: steps 0..2 of both streams in flight; step 0 landed (and
  // transformed), half 0 of its weights read and of its activations
  // prepared.
  w_enter(0);
  a_enter(0);
  issue_all(slots[0]);
  issue_all(slots[1]);
  issue_all(slots[2]);
  wait_vmcnt<2 * kOps>();
  if constexpr (kTUnits > 0) {
    xform_all(slots[0]);
    wait_lgkm0();
  }
  __builtin_amdgcn_s_barrier();
  read_wb(slots[0], 0);
  prep(OP[0], 0, a_read(slots[0], 0, 0));
  prep(OP[0], 1, a_read(slots[0], 1, 0));

  // Loads of one step spread over a half step, one per weight fragment.
  const int last = NB - 1 < kOps - 1 ? NB - 1 : kOps - 1;
  auto spread = [&](uint8_t* slot, int jj) __attribute__((always_inline)) {
    if (jj < last) {
      load_op(slot, jj);
    } else if (jj == last) {
      for (int o = jj; o < kOps; ++o) load_op(slot, o);
      w_advance();
      a_advance();
    }
  };
  // One step s (u = s % 3): half 0 (its weights and prepared activations in
  // registers; half 1 of slot u read and prepared meanwhile); then wait for
  // this wave's LDS accesses, and barrier (step s+1 visible everywhere; slot
  // u no longer read by anyone); then half 1, while half 0 of step s+1 is
  // read and prepared and the loads of step s+3 go into slot u one per
  // weight fragment (unless ISSUE is false: the caller issues them after
  // the tile epilogue). This wave's loads of step s+1 are waited for before
  // the barrier; with a weight transform, already before half 0, which then
  // transforms them.
  auto step = [&](auto uc, auto issuec) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    constexpr int un = (u + 1) % kStages;
    constexpr bool ISSUE = decltype(issuec)::value;
    if constexpr (kTUnits > 0) {
      wait_vmcnt<kOps>();
      compute_half(OP[0], OP[1], slots[u], slots[u], 1, [&](int jj) { xform(slots[un], jj); });
    } else {
      compute_half(OP[0], OP[1], slots[u], slots[u], 1, [](int) {});
      wait_vmcnt<kOps>();
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    if constexpr (ISSUE)
      compute_half(OP[1], OP[0], slots[un], slots[un], 0, [&](int jj) { spread(slots[u], jj); });
    else
      compute_half(OP[1], OP[0], slots[un], slots[un], 0, [](int) {});
  };

  // The steps of branch j but its last ring cycle, from a fresh start of
  // the accumulators.
  auto branch_body = [&](int j) __attribute__((always_inline)) {
    zero_acc();
    pin_acc();
    pin_ys();
    const int P = ksteps(j);
    for (int kb = 0; kb + kStages < P; kb += kStages) {
      step(IC<0>{}, std::true_type{});
      step(IC<1>{}, std::true_type{});
      step(IC<2>{}, std::true_type{});
      pin_acc();
      pin_ys();
    }
    step(IC<0>{}, std::true_type{});
    step(IC<1>{}, std::true_type{});
  };
  for (int ti = 0; ti < tl.count; ++ti) {
    if constexpr (KS) {
      // two input branches: the first is folded (a run-time loop of folds
      // keeps more values live than the register file holds)
      branch_body(0);
      step(IC<2>{}, std::true_type{});
      fold(ti, 0);
    }
    branch_body(nks - 1);
    step(IC<2>{}, std::false_type{});
    epilogue(ti, nks - 1);
    issue_all(slots[2]);
  }
}

template <bool A4, bool SYM, bool CFG, int WX, bool KS, int NB>
__global__ __launch_bounds__(kThreads, 1) void k2_gemm1(GemmArgs g) {
  constexpr int kStage = Slot<A4, WX, NB>::kBytes;
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st2[kStage];
  __shared__ __attribute__((aligned(16))) float sring[ScaleRing<KS>::kFloats];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  // fragment 8 (NB = 9): waves 0 and 1 one instruction each (int8 weights),
  // wave 0 (packed weights, one instruction per fragment)
  static_assert(NB == 9, "wave roles");
  constexpr int kXW = (WX == kWPacked4 || WX == kWPacked4Masked) ? 1 : 2;
  if (wave == 0)
    gemm_wave<A4, SYM, CFG, WX, KS, NB, 0>(g, wave, lane, st0, st1, st2, sring);
  else if (kXW == 2 && wave == 1)
    gemm_wave<A4, SYM, CFG, WX, KS, NB, kXW == 2 ? 1 : -1>(g, wave, lane, st0, st1, st2, sring);
  else
    gemm_wave<A4, SYM, CFG, WX, KS, NB, -1>(g, wave, lane, st0, st1, st2, sring);
}

constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices] = {};

hipError_t device_cus(int& cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached && g_cus[dev] > 0) {
    cus = g_cus[dev];
    return hipSuccess;
  }
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && cached) g_cus[dev] = cus;
  return e;
}

template <bool A4, bool SYM, bool CFG, int WX, bool KS>
hipError_t run(const GemmArgs& g, hipStream_t s) {
  constexpr int NB = 9;
  const int rpt = CFG ? 64 : 128;
  const int T = (((CFG ? g.Mh : g.M) + rpt - 1) / rpt) * ((g.N + 16 * NB - 1) / (16 * NB));
  int cus = 0;
  const hipError_t e = device_cus(cus);
  if (e != hipSuccess) return e;
  const int G = T < cus ? T : cus;
  hipLaunchKernelGGL((k2_gemm1<A4, SYM, CFG, WX, KS, NB>), dim3(G), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

template <bool CFG, int WX>
hipError_t run_ks(const GemmArgs& g, hipStream_t s) {
  constexpr bool A4 = QL_G1_A4 != 0, SYM = QL_G1_SYM != 0;
  if (g.nks > 1) return run<A4, SYM, CFG, WX, true>(g, s);
  return run<A4, SYM, CFG, WX, false>(g, s);
}

template <bool CFG>
hipError_t run_wx(const GemmArgs& g, int w4, hipStream_t s) {
  if (w4) return g.w_lsb_k > 0 ? run_ks<CFG, kWPacked4Masked>(g, s) : run_ks<CFG, kWPacked4>(g, s);
  if (g.w_lsb_k > 0) return run_ks<CFG, kWMasked8>(g, s);
  return run_ks<CFG, kWInt8>(g, s);
}

}  // namespace

#define QL_G1_CAT2(a, b) launch_gemm1_a##a##_s##b
#define QL_G1_CAT(a, b) QL_G1_CAT2(a, b)

hipError_t QL_G1_CAT(QL_G1_A4, QL_G1_SYM)(const GemmArgs& g, int cfg, int w4, hipStream_t s) {
  if (g.nks < 1 || g.nks > 2) return hipErrorNotSupported;
  return cfg ? run_wx<true>(g, w4, s) : run_wx<false>(g, w4, s);
}

}  // namespace ql
