// K2 for HQ-DM's single Hadamard (hi/lo weight planes), SegLinear inputs of
// 3 or 4 branches, and the W8A8 DualScale CFG layers with 144-column tiles
// at any TASQ weight depth (where it measured faster than k_gemm1.hip). Integer
// GEMM of the activation codes against the weight codes on the int8 matrix
// cores of gfx950, both DualScale polarity planes in one kernel, with the
// fp32 epilogue (scales, Hadamard normalisation, CFG combine) fused.
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
//  * Output tile 128 rows x (16*NB) columns, NB = 9 (144 columns) when it
//    divides N: the DiT-XL/2 widths 1152, 3456, 4608 are 8, 24, 32 x 144, so
//    at M = 4096 (CFG pairs) the tile counts are exact multiples of 256 CUs.
//  * 8 waves per workgroup (2 per SIMD, so one wave's waits overlap the
//    other's MFMAs): wave w owns 32 rows (row band w % 4) and one of two
//    column groups (w / 4) of ceil(NB/2) / floor(NB/2) fragments; the two
//    waves sharing a SIMD carry NB fragments together.
//  * Both operands go HBM -> LDS by buffer_load ... lds (no VGPR staging)
//    into a ring of 4 steps of 128 K, 4 steps ahead of the MFMAs; each
//    fragment pair is loaded once per workgroup by one wave. The DMA lanes
//    read whole 128-byte lines (coalesced) and the LDS image is XOR-swizzled
//    so that the MFMA operand reads are bank-conflict free.
//  * Persistent workgroups: each one walks its tiles as one continuous
//    stream of K-steps, so the loads of the next tile overlap the epilogue of
//    the current one. Workgroups (whose id mod 8 is their XCD) get bands of
//    consecutive tiles that share rows in that XCD's L2.
//  * Every out-of-range row or K-chunk is read as zero by the buffer range
//    check, so ragged M, N and K need no special path.
//  * 4-bit activation codes stay packed through memory and LDS and are
//    unpacked on the way into the MFMA, each code multiplied by 16 (nibble
//    placed in the high half of its byte: two ANDs, a shift, two byte
//    permutes); accumulators are shifted back exactly in the epilogue.
//    4-bit weight codes arrive expanded to one int8 per code (plans served
//    here store them so).
//  * CFG pairing: a row band is 16 conditional rows and their 16
//    unconditional partners (fragments 0 and 1), so a lane holds both
//    accumulators of a pair in the same register slot.
//  * Single Hadamard (HQ-DM explainer 2.1, activations rotated only): the
//    plan's weight rows hold hi and lo int8 planes of H W_int^T in adjacent
//    16-row fragments; the symmetric kernel multiplies both and the epilogue
//    combines each pair exactly in fp64 (epilogue_hs). Its tiles are 128 or
//    192 weight rows (NB = 8 or 12; 192 uses all 160 KB of LDS with 8-bit
//    activations).
//  * TASQ weight depth (TASQ explainer 2: one stored buffer, low magnitude
//    bits dropped per stage and layer): the stored codes reach LDS by DMA and
//    each wave masks the 16-byte units its own DMA brought in, in place, two
//    steps ahead of the MFMAs; the step barrier publishes them.
//  * Input branches (SegQuant explainer 2.A, input segmentation): when the
//    K loop crosses a branch end, the branch's epilogue part is folded into
//    fp32 partial sums held in a per-thread workspace slice and the
//    accumulators restart (fold, epilogue_ks).
#include <type_traits>

#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
template <int V>
using IC = std::integral_constant<int, V>;

constexpr int kThreads = kGemmThreads;
constexpr int BK = 128;                 // K elements per ring stage
constexpr int kStages = 4;              // ring depth (= unroll of the step loop)
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

// LDS image of a fragment pair (16 rows x 128 K, the two 16 x 64 MFMA
// operands of one step) and the DMA that fills it.
//
// int8 (2 KB, two DMAs of 1 KB): DMA lane p of instruction i loads row
// r = 8i + p/8, 16-byte chunk (p%8) ^ ((r/2)%8) of the row's 128 bytes, so
// every 8 consecutive lanes read one whole 128-byte line (coalesced); lane
// p's bytes land at i*1024 + p*16. MFMA lane l of half h (row l%16, chunk
// 4h + l/16) finds its 16 bytes at the same swizzled position; the 16 lanes
// read together hit 16 distinct 16-byte bank groups.
//
// packed 4-bit (1 KB, one DMA): DMA lane p loads row p/4, 16-byte chunk
// (p%4) ^ ((p/16)%4) of the row's 64 bytes; MFMA lane l of half h reads the
// 8 bytes of element group 4h + l/16 (8-byte half of one of those chunks).
template <bool P4>
struct Frag {
  uint32_t d[P4 ? 2 : 4];
};

template <bool P4>
struct FragIO {
  static constexpr int kBytes = P4 ? 1024 : 2048;  // fragment pair
  static constexpr int kLoads = P4 ? 1 : 2;        // DMA instructions per pair
  // Row (0..15) and 16-byte chunk that lane p of DMA instruction i loads.
  __device__ static __forceinline__ int dma_row(int i, int p) {
    return P4 ? (p >> 2) : (8 * i + (p >> 3));
  }
  __device__ static __forceinline__ int dma_chunk(int i, int p) {
    const int r = dma_row(i, p);
    return P4 ? ((p & 3) ^ ((r >> 2) & 3)) : ((p & 7) ^ ((r >> 1) & 7));
  }
  // K elements covered by one 16-byte chunk.
  static constexpr int kChunkElems = P4 ? 32 : 16;
  // Where MFMA lane l finds half h of its operand pair inside the image.
  __device__ static __forceinline__ int read_off(int l, int h) {
    const int r = l & 15;
    if constexpr (P4) {
      const int e = 4 * h + (l >> 4);  // 8-byte element group of the row
      return (4 * r + ((e >> 1) ^ ((r >> 2) & 3))) * 16 + (e & 1) * 8;
    } else {
      const int c = 4 * h + (l >> 4);
      return (r >> 3) * 1024 + (8 * (r & 7) + (c ^ ((r >> 1) & 7))) * 16;
    }
  }
  // One DMA instruction of the pair into LDS at `dst` (wave-uniform).
  __device__ static __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, uint8_t* dst, unsigned voff,
                                             unsigned soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, soff, 0, 0);
  }
  __device__ static __forceinline__ void read(Frag<P4>& f, const uint8_t* img, int roff) {
    if constexpr (P4) {
      const uint2 v = *reinterpret_cast<const uint2*>(img + roff);
      f.d[0] = v.x;
      f.d[1] = v.y;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(img + roff);
      f.d[0] = v.x;
      f.d[1] = v.y;
      f.d[2] = v.z;
      f.d[3] = v.w;
    }
  }
};

template <bool A4, int NB>
struct Layout {
  static constexpr int kNB0 = (NB + 1) / 2;  // weight fragments of column group 0
  static constexpr int kNB1 = NB / 2;        // weight fragments of column group 1
  static constexpr int kAFrags = 8;          // 128 rows = 8 fragment pairs
  static constexpr int kABytes = kAFrags * FragIO<A4>::kBytes;
  static constexpr int kStage = kABytes + NB * FragIO<false>::kBytes;
  // DMA: wave w moves activation pair w and weight pair w, and waves
  // w < NB - 8 also weight pair w + 8.
  static_assert(NB >= 8 && NB <= 16, "fragment distribution");
  static constexpr int kOpsLow = FragIO<A4>::kLoads + 2 * FragIO<false>::kLoads;  // waves < NB-8
  static constexpr int kOpsHigh = FragIO<A4>::kLoads + FragIO<false>::kLoads;     // the others
};

// MFMA operand (16 int8 in natural K order) from raw fragment data.
template <bool P4>
__device__ __forceinline__ v4i operand(const Frag<P4>& f) {
  v4i o;
  if constexpr (P4) {
    uint32_t a, b, c, e;
    unpack4_x16(f.d[0], a, b);
    unpack4_x16(f.d[1], c, e);
    o[0] = (int)a;
    o[1] = (int)b;
    o[2] = (int)c;
    o[3] = (int)e;
  } else {
    o[0] = (int)f.d[0];
    o[1] = (int)f.d[1];
    o[2] = (int)f.d[2];
    o[3] = (int)f.d[3];
  }
  return o;
}

// Non-negative polarity plane of an operand (negative bytes zeroed).
__device__ __forceinline__ v4i positive(v4i c) {
  v4i p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = (int)pos_plane((uint32_t)c[i]);
  return p;
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
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
// (workgroup id mod 8) owns a band of consecutive tiles. When that band is
// R whole tile rows and its per_x workgroups divide into R rows of C
// columns, the workgroups run the band as successive R x C blocks (all R
// rows, C columns at a time): the concurrent tiles of an XCD then share R
// activation row panels and C weight column panels in its L2, instead of
// streaming every weight column panel once per row. Otherwise tiles are
// taken in row-major order within the band, or strided over the grid.
struct TileList {
  int first, stride, count;
  int ct, C;  // grouped order: tile columns, block width (C = 0: linear order)
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

// lgkmcnt-only wait (vmcnt / expcnt left at their maxima), gfx9 encoding.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// Instruction-mix masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;

// Issue order of one step's straight-line body: the activation-fragment
// groups (half h, pair fi) each run their NBW MFMAs on the full codes, with
// the polarity split / unpack VALU work of that group slotted between them,
// then the NBW MFMAs on the non-negative plane with the next step's LDS
// reads slotted between them. MFMAs never wait behind a burst of reads or
// VALU work, and the LDS traffic spreads over the whole step.
template <int MASK, int COUNT>
__device__ __forceinline__ void sched_group() {
  if constexpr (COUNT > 0) __builtin_amdgcn_sched_group_barrier(MASK, COUNT, 0);
}

// NBW MFMAs, each followed by VPER VALU instructions and, for the first NR of
// them, one LDS read.
template <int JJ, int NBW, int VPER, int NR>
__device__ __forceinline__ void sched_mfmas() {
  if constexpr (JJ < NBW) {
    sched_group<kSchedMfma, 1>();
    sched_group<kSchedValu, VPER>();
    sched_group<kSchedDsRead, (JJ < NR ? 1 : 0)>();
    sched_mfmas<JJ + 1, NBW, VPER, NR>();
  }
}

template <int GR, int NBW, int NREADS, int VPER, int VPER2, bool DUAL>
__device__ __forceinline__ void sched_groups() {
  if constexpr (GR < 4) {
    constexpr int nr = NREADS * (GR + 1) / 4 - NREADS * GR / 4;
    if constexpr (DUAL) {
      sched_mfmas<0, NBW, VPER, 0>();
      sched_mfmas<0, NBW, VPER2, nr>();
    } else {
      sched_mfmas<0, NBW, VPER, nr>();
    }
    sched_group<kSchedDsRead, (nr > NBW ? nr - NBW : 0)>();
    sched_groups<GR + 1, NBW, NREADS, VPER, VPER2, DUAL>();
  }
}

// VALU2_PER_GROUP: further VALU work slotted between the non-negative-plane
// MFMAs (the weight transform of a later step); NWRITES LDS writes close the
// step.
template <int NBW, int NREADS, int VALU_PER_GROUP, bool DUAL, int VALU2_PER_GROUP = 0,
          int NWRITES = 0>
__device__ __forceinline__ void schedule_step() {
  sched_groups<0, NBW, NREADS, (VALU_PER_GROUP + NBW - 1) / NBW,
               (VALU2_PER_GROUP + NBW - 1) / NBW, DUAL>();
  sched_group<kSchedDsWrite, NWRITES>();
}

// n (4, 5 or 6) floats at p, p + 16, ... (LDS), read in one asm block that
// waits for them itself. The scale ring is written by DMA, and the compiler,
// unable to tell which DMA wrote it, would otherwise wait for every load in
// flight before a plain LDS read of it; the ring entry read here was written
// steps earlier and published by the step barriers since.
template <int N>
__device__ __forceinline__ void lds_read_stride16(const float* p, float* v) {
  static_assert(N >= 4 && N <= 6, "scale reads");
  const uint32_t a = (uint32_t)reinterpret_cast<uintptr_t>(p);  // LDS offset of a shared pointer
  if constexpr (N == 4) {
    asm volatile(
        "ds_read_b32 %0, %4\n\tds_read_b32 %1, %4 offset:64\n\t"
        "ds_read_b32 %2, %4 offset:128\n\tds_read_b32 %3, %4 offset:192\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a)
        : "memory");
  } else if constexpr (N == 5) {
    asm volatile(
        "ds_read_b32 %0, %5\n\tds_read_b32 %1, %5 offset:64\n\t"
        "ds_read_b32 %2, %5 offset:128\n\tds_read_b32 %3, %5 offset:192\n\t"
        "ds_read_b32 %4, %5 offset:256\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4])
        : "v"(a)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b32 %0, %6\n\tds_read_b32 %1, %6 offset:64\n\t"
        "ds_read_b32 %2, %6 offset:128\n\tds_read_b32 %3, %6 offset:192\n\t"
        "ds_read_b32 %4, %6 offset:256\n\tds_read_b32 %5, %6 offset:320\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5])
        : "v"(a)
        : "memory");
  }
}

// Plain tiles (no single Hadamard, no input branches) take their weight
// scales from a ring of kScaleRing tile entries of 256 floats in LDS.
constexpr int kScaleRing = 8;

// The work of one wave. CG (column group) fixes at compile time how many
// weight fragments the wave multiplies and TW whether it also moves weight
// pair w + 8, so a step's body has no branches and every step issues the
// same number of loads: the compiler can then prove from the explicit
// waits below that each LDS read finds its data landed.
template <bool A4, bool SYM, bool CFG, bool HS, bool KS, int NB, int CG, bool TW, bool MK, bool DBG>
__device__ __forceinline__ void gemm_wave(const GemmArgs& g, int wave, int lane, uint8_t* st0,
                                          uint8_t* st1, uint8_t* st2, uint8_t* st3,
                                          float* sring) {
  using Lay = Layout<A4, NB>;
  using IA = FragIO<A4>;
  using IW = FragIO<false>;  // weights are int8 codes (4-bit ones expanded by the plan)
  constexpr int NP = SYM ? 1 : 2;                     // accumulator planes
  constexpr int SHIFT = A4 ? 4 : 0;  // undo the x16 unpack of 4-bit activations
  constexpr int BN = 16 * NB;
  constexpr int NBW = CG ? Lay::kNB1 : Lay::kNB0;     // weight fragments of this wave
  constexpr int J0 = CG ? Lay::kNB0 : 0;              // first weight fragment of this wave
  constexpr int RPT = CFG ? 64 : 128;                 // output rows per tile
  uint8_t* const slots[kStages] = {st0, st1, st2, st3};

  const int band = wave & 3;  // row band: 32 rows of the tile

  const int ct = (g.N + BN - 1) / BN;
  const int T = (((CFG ? g.Mh : g.M) + RPT - 1) / RPT) * ct;
  const TileList tl = my_tiles(T, ct);
  if (tl.count == 0) return;

  const int nk = (g.K + BK - 1) / BK;
  const int total = tl.count * nk;  // steps of this workgroup's stream

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)((int64_t)g.M * g.lda));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.W, (uint32_t)((int64_t)g.N * g.ldw));
  constexpr bool kRing = !HS && !KS;  // weight scales through the LDS ring
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.w_scales, (uint32_t)g.Nout * 4u);

  auto coords = [&](int ti, int& m0, int& n0) __attribute__((always_inline)) {
    const int t = tl.at(ti);
    const int tr = t / ct;
    m0 = tr * RPT;
    n0 = (t - tr * ct) * BN;
  };

  // Global row of row i (0..15) of activation pair f (0..7) of a tile: pair f
  // belongs to row band f/2; with CFG, pair 2b holds 16 conditional rows and
  // 2b+1 their unconditional partners.
  auto a_row = [&](int m0, int f, int i, bool& ok) __attribute__((always_inline)) {
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

  // Load stream position (kStages steps ahead of the MFMAs) and this lane's
  // DMA offsets for the stream's tile; the K offset of a step goes into the
  // scalar operand of the loads.
  int iss_ti = 0, iss_k = 0;
  unsigned av[IA::kLoads], wv[2][IW::kLoads];
  // Entering a tile (kStages steps ahead of its MFMAs, so at most kStages
  // tiles ahead of the epilogue that reads the entry), wave 0 also moves the
  // tile's 16*NB weight scales into entry ti % kScaleRing of the scale ring
  // (16 bytes per lane; columns past N read as 0).
  auto enter_tile = [&](int ti) __attribute__((always_inline)) {
    int m0, n0;
    coords(ti, m0, n0);
    if constexpr (kRing) {
      static_assert(kScaleRing > kStages, "scale ring entries outlive the stream's lead");
      if (wave == 0) {
        const unsigned v = 16u * (unsigned)lane < 4u * (unsigned)BN ? 16u * (unsigned)lane : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_void*)(sring + (ti % kScaleRing) * 256), 16, v, 4u * (unsigned)n0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < IA::kLoads; ++i) {
      bool ok;
      const int r = a_row(m0, wave, IA::dma_row(i, lane), ok);
      av[i] = ok ? (unsigned)r * (unsigned)g.lda + 16u * (unsigned)IA::dma_chunk(i, lane) : kOOB;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < IW::kLoads; ++i) {
        const int n = n0 + 16 * (wave + 8 * q) + IW::dma_row(i, lane);
        wv[q][i] = n < g.N ? (unsigned)n * (unsigned)g.ldw + 16u * (unsigned)IW::dma_chunk(i, lane)
                           : kOOB;
      }
  };

  // Issue the stream's next step into `slot`. Past the end of the stream
  // the same loads are issued with out-of-range offsets (they write zeros
  // into slots nothing reads), so every step issues the same loads.
  auto issue = [&](uint8_t* slot) __attribute__((always_inline)) {
    const int k0 = iss_k * BK;
    const unsigned sa = (unsigned)k0 / (A4 ? 2u : 1u);
    const unsigned sw = (unsigned)k0;
    const bool ragged = k0 + BK > g.K;  // chunks past K must read zeros
#pragma unroll
    for (int i = 0; i < IA::kLoads; ++i) {
      unsigned v = av[i];
      if (ragged && k0 + IA::kChunkElems * IA::dma_chunk(i, lane) >= g.K) v = kOOB;
      IA::dma(ra, slot + wave * IA::kBytes + i * 1024, v, sa);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (q == 0 || TW) {
#pragma unroll
        for (int i = 0; i < IW::kLoads; ++i) {
          unsigned v = wv[q][i];
          if (ragged && k0 + IW::kChunkElems * IW::dma_chunk(i, lane) >= g.K) v = kOOB;
          IW::dma(rw, slot + Lay::kABytes + (wave + 8 * q) * IW::kBytes + i * 1024, v, sw);
        }
      }
    }
    if (++iss_k == nk) {
      iss_k = 0;
      if (++iss_ti < tl.count) {
        enter_tile(iss_ti);
      } else {
#pragma unroll
        for (int i = 0; i < IA::kLoads; ++i) av[i] = kOOB;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int i = 0; i < IW::kLoads; ++i) wv[q][i] = kOOB;
      }
    }
  };

  // Wait until at most n of this wave's issued steps are still in flight.
  auto wait_steps = [&](auto nc) __attribute__((always_inline)) {
    constexpr int n = decltype(nc)::value;
    wait_vmcnt<n * (TW ? Lay::kOpsLow : Lay::kOpsHigh)>();
  };

  // TASQ weight depth (MK): the weight bytes this wave's DMA brought into a
  // slot (16 per lane per DMA instruction), read back by the lane that
  // loaded them, magnitude-masked in place (trunc_mag4) and published by the
  // next step barrier; each weight byte is masked once per workgroup. The
  // masked step is two steps ahead of the MFMAs (its loads are waited for
  // one step earlier than without the mask), so no extra barrier is needed.
  // (Splitting the wave that also moves pair 8's share over the other SIMDs
  // measured 1-1.5 % slower.)
  constexpr int kTUnits = MK ? (TW ? 2 : 1) * IW::kLoads : 0;
  uint32_t mlut = 0, mkeep = 0xFFFFFFFFu;
  if constexpr (MK) {
    const int kk = g.w_lsb_k;
    mlut = ((1u << kk) - 1u) << 8;
    mkeep = 0x01010101u * (0xFFu & ~((1u << kk) - 1u));
  }
  // Unit t: DMA instruction t % 2 of weight pair wave + 8 (t / 2).
  auto mask_unit = [&](uint8_t* slot, int t) __attribute__((always_inline)) {
    const int q = t / IW::kLoads, i = t % IW::kLoads;
    v4u* p = reinterpret_cast<v4u*>(slot + Lay::kABytes + (wave + 8 * q) * IW::kBytes + i * 1024 +
                                    lane * 16);
    const v4u v = *p;
    *p = v4u{trunc_mag4(v.x, mlut, mkeep), trunc_mag4(v.y, mlut, mkeep),
             trunc_mag4(v.z, mlut, mkeep), trunc_mag4(v.w, mlut, mkeep)};
  };
  auto mask_slot = [&](uint8_t* slot) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kTUnits; ++t) mask_unit(slot, t);
  };

  int roff_a[2], roff_w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    roff_a[h] = IA::read_off(lane, h);
    roff_w[h] = IW::read_off(lane, h);
  }

  struct Frags {
    Frag<A4> a[2][2];    // [pair of the band][half]
    Frag<false> w[NBW][2];  // [fragment slot][half]
  };
  Frags F[2];
  auto read_all = [&](Frags& f, const uint8_t* slot) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int fi = 0; fi < 2; ++fi)
        IA::read(f.a[fi][h], slot + (2 * band + fi) * IA::kBytes, roff_a[h]);
#pragma unroll
      for (int jj = 0; jj < NBW; ++jj)
        IW::read(f.w[jj][h], slot + Lay::kABytes + (J0 + jj) * IW::kBytes, roff_w[h]);
    }
  };

  // DUAL: acc[0] = sum pos(c) w, acc[1] = sum c w (acc- = acc[1] - acc[0]).
  v4i acc[NP][2][NBW];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int fi = 0; fi < 2; ++fi)
#pragma unroll
        for (int jj = 0; jj < NBW; ++jj) acc[p][fi][jj] = v4i{0, 0, 0, 0};
  };

  // Step s's MFMAs on `f` plus the reads of step s+1's fragments into `n`,
  // issued in the interleaved order of schedule_step.
  auto compute = [&](const Frags& f, Frags& n, const uint8_t* nslot,
                     uint8_t* tslot) __attribute__((always_inline)) {
    mask_slot(tslot);
    read_all(n, nslot);
    v4i b[NBW][2];
#pragma unroll
    for (int jj = 0; jj < NBW; ++jj)
#pragma unroll
      for (int h = 0; h < 2; ++h) b[jj][h] = operand<false>(f.w[jj][h]);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int fi = 0; fi < 2; ++fi) {
        const v4i a = operand<A4>(f.a[fi][h]);
#pragma unroll
        for (int jj = 0; jj < NBW; ++jj) acc[NP - 1][fi][jj] = mfma(a, b[jj][h], acc[NP - 1][fi][jj]);
        if constexpr (!SYM) {
          const v4i ap = positive(a);
#pragma unroll
          for (int jj = 0; jj < NBW; ++jj) acc[0][fi][jj] = mfma(ap, b[jj][h], acc[0][fi][jj]);
        }
      }
    constexpr int kReads = 4 + 2 * NBW + kTUnits;
    constexpr int kValu = (SYM ? 0 : 12) + (A4 ? 10 : 0);
    schedule_step<NBW, kReads, kValu, !SYM, (20 * kTUnits + 3) / 4, kTUnits>();
  };

  // Scales of the last input branch (the only one without input branches).
  const int jl = KS ? g.nks - 1 : 0;
  const float sp = g.act_scales[2 * jl];
  const float sn = g.act_scales[2 * jl + 1];
  const int i16 = lane & 15;
  const int rsub = (lane >> 4) * 4;
  // Input branches: the fp32 sum of the finished branches' epilogue parts
  // per output lives in this thread's slice of the plan's workspace (slot s
  // of the thread at [block][s][thread]), written at each branch end and read
  // back (from L2) by the next branch end or by the tile epilogue. Also the
  // current branch and the K-step at which it ends.
  static_assert(!KS || 2 * NBW * 4 <= kYSlots, "partial-sum slots");
  // Buffer accesses: the workgroup's block in the descriptor, the thread in
  // one vector offset, the slot in the scalar offset (no per-slot addresses).
  const __amdgpu_buffer_rsrc_t ryw =
      make_rsrc(KS ? g.ypart_ws + (int64_t)blockIdx.x * kYSlots * kThreads : g.Y,
                KS ? (uint32_t)(kYSlots * kThreads * 4) : 0u);
  const unsigned ytid = 4u * threadIdx.x;
  auto yoff = [&](int fi, int jj, int r) __attribute__((always_inline)) {
    return (unsigned)(((fi * NBW + jj) * 4 + r) * kThreads * 4);
  };
  // Loads bypass the L1 (glc): the slot was last written by this thread.
  auto yload = [&](int fi, int jj, int r) __attribute__((always_inline)) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ryw, ytid, yoff(fi, jj, r), 1));
  };
  auto ystore = [&](int fi, int jj, int r, float v) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ryw, ytid, yoff(fi, jj, r), 0);
  };
  int cur_seg = 0;
  int seg_end = KS ? g.ks_end[0] : 0;

  // (acc+, acc-) of accumulator slot (fi, jj, r), shifted back to code units.
  auto accs = [&](int fi, int jj, int r, int& ap, int& an) __attribute__((always_inline)) {
    ap = acc[0][fi][jj][r] >> SHIFT;
    if constexpr (SYM)
      an = 0;
    else
      an = (acc[NP - 1][fi][jj][r] - acc[0][fi][jj][r]) >> SHIFT;
  };

  // Tile epilogue. The scales of the tile's columns are loaded first and
  // waited for once; the outputs then go out through range-checked buffer
  // stores (rows past the end and columns past N are dropped by the range
  // check), so no store waits on another and there are no per-element
  // branches.
  // Accumulator dump (testing aid): planes 2j and 2j + 1 of [2 * nks, M, N]
  // hold (acc+, acc-) of input branch j.
  auto dump_acc = [&](int m0, const unsigned (&coff)[NBW], int j) __attribute__((always_inline)) {
    const int64_t plane = (int64_t)g.M * g.N;
#pragma unroll
    for (int fi = 0; fi < 2; ++fi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bool ok;
        const int grow = a_row(m0, 2 * band + fi, rsub + r, ok);
        if (!ok) continue;
#pragma unroll
        for (int jj = 0; jj < NBW; ++jj) {
          if (coff[jj] == kOOB) continue;
          const int64_t e = (int64_t)grow * g.N + (coff[jj] >> 2);
          int ap, an;
          accs(fi, jj, r, ap, an);
          g.dbg[2 * j * plane + e] = ap;
          g.dbg[(2 * j + 1) * plane + e] = an;
        }
      }
  };

  // End of input branch cur_seg of a tile: add its epilogue part (before
  // 1/B) to the partial sums (fp32, branch order) in the workspace; the
  // caller restarts the accumulators. The scale loads and the stores drain
  // before the K loop goes on, so the next reload finds the sums in L2.
  auto fold = [&](int ti) __attribute__((always_inline)) {
    int m0, n0;
    coords(ti, m0, n0);
    const int j = cur_seg;
    const float spj = g.act_scales[2 * j];
    const float snj = g.act_scales[2 * j + 1];
    float swj[NBW];
    unsigned coff[NBW];
#pragma unroll
    for (int jj = 0; jj < NBW; ++jj) {
      const int col = n0 + 16 * (J0 + jj) + i16;
      swj[jj] = g.w_scales[(int64_t)j * g.Nout + min(col, g.N - 1)];
      coff[jj] = col < g.N ? 4u * (unsigned)col : kOOB;
    }
#pragma unroll
    for (int jj = 0; jj < NBW; ++jj) asm volatile("" ::"v"(swj[jj]));
    // One accumulator row r at a time (8 partial sums in flight), so the
    // reloads do not all occupy registers at once.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float old[2][NBW];
#pragma unroll
      for (int fi = 0; fi < 2; ++fi)
#pragma unroll
        for (int jj = 0; jj < NBW; ++jj) old[fi][jj] = j > 0 ? yload(fi, jj, r) : 0.0f;
#pragma unroll
      for (int fi = 0; fi < 2; ++fi)
#pragma unroll
        for (int jj = 0; jj < NBW; ++jj) {
          int ap, an;
          accs(fi, jj, r, ap, an);
          float y = epi_part<SYM>(ap, an, spj, snj, swj[jj]);
          if (j > 0) y = __fadd_rn(old[fi][jj], y);
          if constexpr (KS) ystore(fi, jj, r, y);
        }
      asm volatile("" ::: "memory");
    }
    if constexpr (DBG) {
      if (g.dbg) dump_acc(m0, coff, j);
    }
    wait_vmcnt<0>();
  };

  // Single Hadamard: fragments (J0 + 2p, J0 + 2p + 1) hold the hi and lo
  // planes of the same 16 output channels; the exact sum 128 * hi + lo is
  // formed in fp64 (|sum| < 2^53) and rounded once to fp32.
  auto epilogue_hs = [&](int ti) __attribute__((always_inline)) {
    static_assert(!HS || (SYM && NBW % 2 == 0 && J0 % 2 == 0), "hi/lo fragment pairs");
    constexpr int NPR = NBW / 2;
    int m0, n0;
    coords(ti, m0, n0);
    float sw[NPR];
    unsigned coff[NPR];
#pragma unroll
    for (int p = 0; p < NPR; ++p) {
      const int col = n0 / 2 + 8 * J0 + 16 * p + i16;
      sw[p] = g.w_scales[min(col, g.Nout - 1)];
      coff[p] = col < g.Nout ? 4u * (unsigned)col : kOOB;
    }
#pragma unroll
    for (int p = 0; p < NPR; ++p) asm volatile("" ::"v"(sw[p]));
    const int rows_here = min(RPT, (CFG ? g.Mh : g.M) - m0);
    const __amdgpu_buffer_rsrc_t ry =
        make_rsrc(g.Y + (int64_t)m0 * g.Nout, (uint32_t)rows_here * (uint32_t)g.Nout * 4u);
    const unsigned rowb = (unsigned)g.Nout * 4u;
    auto value = [&](int fi, int p, int r) __attribute__((always_inline)) {
      const int hi = acc[0][fi][2 * p][r] >> SHIFT;
      const int lo = acc[0][fi][2 * p + 1][r] >> SHIFT;
      const double e = __dadd_rn(__dmul_rn((double)hi, 128.0), (double)lo);
      const float a = __double2float_rn(e);
      return __fmul_rn(a, sp);
    };
    auto out = [&](float a, int p) __attribute__((always_inline)) {
      return __fmul_rn(__fmul_rn(a, sw[p]), g.inv_b);
    };
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (CFG) {
        const unsigned ro = (unsigned)(16 * band + rsub + r) * rowb;
#pragma unroll
        for (int p = 0; p < NPR; ++p) {
          const float yc = out(value(0, p, r), p);
          const float yu = out(value(1, p, r), p);
          const float d = __fsub_rn(yc, yu);
          const float t = __fmul_rn(g.guidance, d);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(__fadd_rn(yu, t)), ry,
                                                ro + coff[p], 0, 0);
        }
      } else {
#pragma unroll
        for (int fi = 0; fi < 2; ++fi) {
          const unsigned ro = (unsigned)(16 * (2 * band + fi) + rsub + r) * rowb;
#pragma unroll
          for (int p = 0; p < NPR; ++p)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out(value(fi, p, r), p)), ry,
                                                  ro + coff[p], 0, 0);
        }
      }
    }
    if (g.dbg) {  // accumulator dump (testing aid): hi and lo plane sums
      const int64_t plane = (int64_t)g.M * g.Nout;
#pragma unroll
      for (int fi = 0; fi < 2; ++fi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bool ok;
          const int grow = a_row(m0, 2 * band + fi, rsub + r, ok);
          if (!ok) continue;
#pragma unroll
          for (int p = 0; p < NPR; ++p) {
            if (coff[p] == kOOB) continue;
            const int64_t e = (int64_t)grow * g.Nout + (coff[p] >> 2);
            g.dbg[e] = acc[0][fi][2 * p][r] >> SHIFT;
            g.dbg[plane + e] = acc[0][fi][2 * p + 1][r] >> SHIFT;
          }
        }
    }
    wait_vmcnt<0>();
  };

  auto epilogue = [&](int ti) __attribute__((always_inline)) {
    int m0, n0;
    coords(ti, m0, n0);
    float sw[NBW];
    unsigned coff[NBW];  // byte offset of this lane's column in a row, or out of range
    lds_read_stride16<NBW>(sring + (ti % kScaleRing) * 256 + 16 * J0 + i16, sw);
#pragma unroll
    for (int jj = 0; jj < NBW; ++jj) {
      const int col = n0 + 16 * (J0 + jj) + i16;
      coff[jj] = col < g.N ? 4u * (unsigned)col : kOOB;
    }
    auto yout = [&](int fi, int jj, int r) __attribute__((always_inline)) {
      int ap, an;
      accs(fi, jj, r, ap, an);
      // plain tiles carry no rotation: the launcher admits them with
      // 1/B = 1 only, so the exact multiply by 1/B is left out
      return epi_part<SYM>(ap, an, sp, sn, sw[jj]);
    };
    const int rows_here = min(RPT, (CFG ? g.Mh : g.M) - m0);
    const __amdgpu_buffer_rsrc_t ry =
        make_rsrc(g.Y + (int64_t)m0 * g.N, (uint32_t)rows_here * (uint32_t)g.N * 4u);
    const unsigned rowb = (unsigned)g.N * 4u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (CFG) {
        const unsigned ro = (unsigned)(16 * band + rsub + r) * rowb;
#pragma unroll
        for (int jj = 0; jj < NBW; ++jj) {
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
          const unsigned ro = (unsigned)(16 * (2 * band + fi) + rsub + r) * rowb;
#pragma unroll
          for (int jj = 0; jj < NBW; ++jj)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yout(fi, jj, r)), ry,
                                                  ro + coff[jj], 0, 0);
        }
      }
    }
    if (g.dbg) dump_acc(m0, coff, jl);
    // Let the stores complete here, while no load is in flight: pending
    // stores would otherwise leave the compiler unable to account the loads
    // of the next steps, and it would drain the whole load stream later.
    wait_vmcnt<0>();
  };

  // Tile epilogue with input branches: the last branch is folded like the
  // others (its sum now complete in the workspace), then the sums are read
  // back a row at a time, scaled by 1/B, combined for CFG and stored; the
  // accumulators are no longer live by then.
  auto epilogue_ks = [&](int ti) __attribute__((always_inline)) {
    fold(ti);
    int m0, n0;
    coords(ti, m0, n0);
    unsigned coff[NBW];
#pragma unroll
    for (int jj = 0; jj < NBW; ++jj) {
      const int col = n0 + 16 * (J0 + jj) + i16;
      coff[jj] = col < g.N ? 4u * (unsigned)col : kOOB;
    }
    const int rows_here = min(RPT, (CFG ? g.Mh : g.M) - m0);
    const __amdgpu_buffer_rsrc_t ry =
        make_rsrc(g.Y + (int64_t)m0 * g.N, (uint32_t)rows_here * (uint32_t)g.N * 4u);
    const unsigned rowb = (unsigned)g.N * 4u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float y[2][NBW];
#pragma unroll
      for (int fi = 0; fi < 2; ++fi)
#pragma unroll
        for (int jj = 0; jj < NBW; ++jj) y[fi][jj] = __fmul_rn(yload(fi, jj, r), g.inv_b);
      if constexpr (CFG) {
        const unsigned ro = (unsigned)(16 * band + rsub + r) * rowb;
#pragma unroll
        for (int jj = 0; jj < NBW; ++jj) {
          const float d = __fsub_rn(y[0][jj], y[1][jj]);
          const float t = __fmul_rn(g.guidance, d);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(__fadd_rn(y[1][jj], t)), ry,
                                                ro + coff[jj], 0, 0);
        }
      } else {
#pragma unroll
        for (int fi = 0; fi < 2; ++fi) {
          const unsigned ro = (unsigned)(16 * (2 * band + fi) + rsub + r) * rowb;
#pragma unroll
          for (int jj = 0; jj < NBW; ++jj)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y[fi][jj]), ry,
                                                  ro + coff[jj], 0, 0);
        }
      }
      asm volatile("" ::: "memory");
    }
    wait_vmcnt<0>();
  };

  int cmp_ti = 0, cmp_k = 0;  // compute position

  // One step: wait for step s+1 (this wave's DMA) and for this wave's reads
  // of step s (so its slot is free), barrier (step s+1 visible to all, slot
  // of step s free everywhere), refill that slot with step s+4, then run
  // step s's MFMAs interleaved with the reads of step s+1's fragments.
  // Returns true when step s ends a tile. u = s % kStages is a compile-time
  // constant at every call site.
  auto step = [&](int s, auto uc) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    wait_steps(IC<MK ? 1 : 2>{});
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    issue(slots[u]);
    // (on the last step this reads a stale slot; the values are never used;
    // the masked slot holds step s+2, issued like every step)
    compute(F[u & 1], F[(u + 1) & 1], slots[(u + 1) % kStages], slots[(u + 2) % kStages]);
    return ++cmp_k == nk;
  };

  // prologue: steps 0 .. 3 in flight, step 0 landed and read
  enter_tile(0);
  issue(slots[0]);
  issue(slots[1]);
  issue(slots[2]);
  issue(slots[3]);
  if constexpr (MK) {
    wait_steps(IC<2>{});  // steps 0 and 1 landed: mask this wave's bytes of them
    mask_slot(slots[0]);
    mask_slot(slots[1]);
    wait_lgkm0();
  } else {
    wait_steps(IC<3>{});
  }
  __builtin_amdgcn_s_barrier();
  read_all(F[0], slots[0]);
  zero_acc();

  // The ring cycle is unrolled by its depth so that slots and fragment
  // buffers are static.
  auto step_epi = [&](int s, auto uc) __attribute__((always_inline)) {
    if (step(s, uc)) {
      if constexpr (HS)
        epilogue_hs(cmp_ti);
      else if constexpr (KS)
        epilogue_ks(cmp_ti);
      else
        epilogue(cmp_ti);
      zero_acc();
      cmp_k = 0;
      ++cmp_ti;
      if constexpr (KS) {
        cur_seg = 0;
        seg_end = g.ks_end[0];
      }
    } else if constexpr (KS) {
      if (cmp_k == seg_end) {
        fold(cmp_ti);
        zero_acc();
        ++cur_seg;
        // entries past the last branch hold a step count no tile reaches
        seg_end = cur_seg == 1 ? g.ks_end[1] : cur_seg == 2 ? g.ks_end[2] : g.ks_end[3];
      }
    }
  };
  int sb = 0;
  for (; sb + kStages <= total; sb += kStages) {
    step_epi(sb + 0, IC<0>{});
    step_epi(sb + 1, IC<1>{});
    step_epi(sb + 2, IC<2>{});
    step_epi(sb + 3, IC<3>{});
  }
  if (sb + 0 < total) step_epi(sb + 0, IC<0>{});
  if (sb + 1 < total) step_epi(sb + 1, IC<1>{});
  if (sb + 2 < total) step_epi(sb + 2, IC<2>{});
}

template <bool A4, bool SYM, bool CFG, bool HS, bool KS, int NB, bool MK, bool DBG>
__global__ __launch_bounds__(kThreads, 1) void k2_gemm(GemmArgs g) {
  using Lay = Layout<A4, NB>;
  // One LDS object per ring stage: the compiler tracks DMA -> LDS writes per
  // object, so a fragment read waits only for the DMA of its own stage.
  __shared__ __attribute__((aligned(16))) uint8_t st0[Lay::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[Lay::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st2[Lay::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st3[Lay::kStage];
  static_assert(kStages == 4, "one LDS object per stage");
  // weight-scale ring of the plain tiles (single-Hadamard tiles use all of LDS)
  __shared__ __attribute__((aligned(16))) float sring[(HS || KS) ? 4 : kScaleRing * 256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  // waves w < NB - 8 also move weight pair w + 8; with NB <= 12 those are
  // all column-group-0 waves
  static_assert(NB >= 8 && NB <= 12, "wave roles");
  if (wave < NB - 8)
    gemm_wave<A4, SYM, CFG, HS, KS, NB, 0, true, MK, DBG>(g, wave, lane, st0, st1, st2, st3, sring);
  else if (wave < 4)
    gemm_wave<A4, SYM, CFG, HS, KS, NB, 0, false, MK, DBG>(g, wave, lane, st0, st1, st2, st3, sring);
  else
    gemm_wave<A4, SYM, CFG, HS, KS, NB, 1, false, MK, DBG>(g, wave, lane, st0, st1, st2, st3, sring);
}

// Compute units per device, queried on the first launch there. The grid
// never exceeds the current device's count (a plan's partial-sum workspace
// is sized by the same count).
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

template <bool A4, bool SYM, bool CFG, bool HS, bool KS, int NB, bool MK = false, bool DBG = false>
hipError_t run(const GemmArgs& g, hipStream_t s) {
  const int rpt = CFG ? 64 : 128;
  const int T = (((CFG ? g.Mh : g.M) + rpt - 1) / rpt) * ((g.N + 16 * NB - 1) / (16 * NB));
  int cus = 0;
  const hipError_t e = device_cus(cus);
  if (e != hipSuccess) return e;
  const int G = T < cus ? T : cus;
  hipLaunchKernelGGL((k2_gemm<A4, SYM, CFG, HS, KS, NB, MK, DBG>), dim3(G), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

// Whether 192-column tiles (NB = 12) beat tiles of 16 * nb columns: they
// read fewer LDS bytes per product, and win unless they need more rounds of
// tiles over the compute units, counted in tile-width units (ties go wide).
hipError_t wide_tiles(const GemmArgs& g, int cfg, int nb, bool& wide) {
  int cus = 0;
  const hipError_t e = device_cus(cus);
  if (e != hipSuccess) return e;
  const long rows = ((cfg ? g.Mh : g.M) + (cfg ? 63 : 127)) / (cfg ? 64 : 128);
  const long tn = rows * ((g.N + 16 * nb - 1) / (16 * nb)), t12 = rows * ((g.N + 191) / 192);
  wide = ((t12 + cus - 1) / cus) * 12 <= ((tn + cus - 1) / cus) * nb;
  return hipSuccess;
}

template <bool A4>
hipError_t run_mode(const GemmArgs& g, int sym, int cfg, int hs, hipStream_t s) {
  // Single Hadamard: symmetric codes, 128 or 192 weight rows (64 or 96
  // channels) per tile, so that every wave holds whole hi/lo pairs. The
  // wider tile reads fewer LDS bytes per product; it is taken unless it
  // needs more rounds of tiles over the compute units (in tile-width units).
  if (hs) {
    if (!sym || g.nks > 1) return hipErrorInvalidValue;
    bool wide = false;
    const hipError_t e = wide_tiles(g, cfg, 8, wide);
    if (e != hipSuccess) return e;
    if (wide)
      return cfg ? run<A4, true, true, true, false, 12>(g, s)
                 : run<A4, true, false, true, false, 12>(g, s);
    return cfg ? run<A4, true, true, true, false, 8>(g, s)
               : run<A4, true, false, true, false, 8>(g, s);
  }
  // Three or four input branches: 128-column tiles (the partial sums take
  // 32 registers). The per-branch accumulator dump (a testing aid) lives in
  // an instantiation of its own: its address arithmetic at every branch end
  // would push the DualScale kernels past the register file (spills).
  if (g.nks > 2) {
    if (g.dbg) {
      if (sym)
        return cfg ? run<A4, true, true, false, true, 8, false, true>(g, s)
                   : run<A4, true, false, false, true, 8, false, true>(g, s);
      return cfg ? run<A4, false, true, false, true, 8, false, true>(g, s)
                 : run<A4, false, false, false, true, 8, false, true>(g, s);
    }
    if (sym)
      return cfg ? run<A4, true, true, false, true, 8>(g, s)
                 : run<A4, true, false, false, true, 8>(g, s);
    return cfg ? run<A4, false, true, false, true, 8>(g, s)
               : run<A4, false, false, false, true, 8>(g, s);
  }
  // int8 weights at any TASQ depth, 8-bit DualScale activations, CFG,
  // 144-column tiles, no rotation (the DiT-XL/2 W8A8 layers): this kernel
  // measured 2-6 % faster than k_gemm1.hip there. Every other plan runs
  // k_gemm1.hip.
  if (!A4 && !sym && cfg && g.nks == 1 && g.N % 144 == 0 && g.inv_b == 1.0f)
    return g.w_lsb_k > 0 ? run<false, false, true, false, false, 9, true>(g, s)
                         : run<false, false, true, false, false, 9>(g, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, int a4, int sym, int cfg, int hs, hipStream_t s) {
  return a4 ? run_mode<true>(g, sym, cfg, hs, s) : run_mode<false>(g, sym, cfg, hs, s);
}

}  // namespace ql
