// K2: integer GEMM of the activation codes against the weight codes on the
// int8 matrix cores of gfx950, both DualScale polarity planes in one kernel,
// with the fp32 epilogue (scales, Hadamard normalisation, CFG combine) fused.
//
// Method (pages): SegQuant explainer 2.B -- X is split into its
// non-negative and negative parts, each multiplied by the weight codes, the
// two products run side by side in one batched kernel and their rescaled
// results are summed in the epilogue; "Closing the Null Space" explainer,
// problem statement -- guided output uncond + w (cond - uncond).
//
// Design for CDNA4:
//  * v_mfma_i32_16x16x64_i8: a wave multiplies a 16x64 code fragment by a
//    64x16 weight fragment per instruction. Each A fragment is split on the
//    fly into its two polarity planes (byte sign masks), and both planes are
//    multiplied by the same weight fragment into two accumulator sets -- the
//    batch-2 GEMM shares every W tile it loads.
//  * Workgroup tile 128 x 128 outputs, 4 waves of 64 x 64, K step 64 bytes,
//    double-buffered LDS (rows padded to 80 bytes so the 16-byte fragment
//    reads of 16 consecutive rows hit distinct banks).
//  * 4-bit codes are unpacked to int8 on the way into LDS, each code
//    multiplied by 16 (nibble moved to the high half of its byte) so the
//    unpack is two ANDs, a shift and two byte permutes; the accumulators are
//    shifted back exactly (every product is a multiple of 16 or 256).
//  * CFG pairing: a workgroup owns 64 conditional rows m0.. and their 64
//    unconditional partners m0 + M/2.. ; within a wave, fragments 0,1 are
//    conditional and 2,3 the partners, so a lane holds both accumulators of
//    a pair in the same register slot and combines them without LDS.
#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;       // K elements (bytes of int8) per step
constexpr int LDS_ROW = 80;  // bytes per LDS row (64 + 16 pad)
constexpr int TILE_BYTES = BM * LDS_ROW;

struct RowMap {
  // Global row of local tile row lr, and whether it exists.
  int m0;
  int M, Mh;
  template <bool CFG>
  __device__ __forceinline__ int row(int lr, bool& valid) const {
    if constexpr (CFG) {
      const int g = lr >> 6, q = (lr >> 5) & 1, o = lr & 31;
      const int crow = m0 + g * 32 + o;
      valid = crow < Mh;
      return crow + q * Mh;
    } else {
      const int r = m0 + lr;
      valid = r < M;
      return r;
    }
  }
};

// Global -> registers for one K step of a 128-row operand tile.
// int8 operand: 2 chunks of 16 bytes per thread; int4: 1 chunk of 16 packed bytes.
template <bool P4>
struct TileLoad {
  uint4 v[P4 ? 1 : 2];
};

template <bool P4>
__device__ __forceinline__ void load_tile(TileLoad<P4>& t, const uint8_t* base, const int64_t* roff,
                                          const bool* rvalid, int k0, int K, int tid) {
  if constexpr (P4) {
    const int c = tid & 1;
    const int kk = k0 + c * 32;
    const bool ok = rvalid[0] && kk < K;
    t.v[0] = ok ? *reinterpret_cast<const uint4*>(base + roff[0] + kk / 2) : make_uint4(0, 0, 0, 0);
  } else {
    const int c = tid & 3;
    const int kk = k0 + c * 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool ok = rvalid[h] && kk < K;
      t.v[h] = ok ? *reinterpret_cast<const uint4*>(base + roff[h] + kk) : make_uint4(0, 0, 0, 0);
    }
  }
}

template <bool P4>
__device__ __forceinline__ void store_tile(const TileLoad<P4>& t, uint8_t* lds, int tid) {
  if constexpr (P4) {
    const int lr = tid >> 1, c = tid & 1;
    uint4 lo, hi;
    unpack4_x16(t.v[0].x, lo.x, lo.y);
    unpack4_x16(t.v[0].y, lo.z, lo.w);
    unpack4_x16(t.v[0].z, hi.x, hi.y);
    unpack4_x16(t.v[0].w, hi.z, hi.w);
    uint8_t* p = lds + lr * LDS_ROW + c * 32;
    *reinterpret_cast<uint4*>(p) = lo;
    *reinterpret_cast<uint4*>(p + 16) = hi;
  } else {
    const int c = tid & 3;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lr = (tid >> 2) + h * 64;
      *reinterpret_cast<uint4*>(lds + lr * LDS_ROW + c * 16) = t.v[h];
    }
  }
}

__device__ __forceinline__ v4i as_v4i(uint4 u) {
  v4i r;
  r[0] = (int)u.x;
  r[1] = (int)u.y;
  r[2] = (int)u.z;
  r[3] = (int)u.w;
  return r;
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// y from the two accumulators, in the documented order, no contraction.
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

template <bool A4, bool W4, bool SYM, bool CFG, bool DBG>
__global__ __launch_bounds__(kThreads, 2) void k2_gemm(GemmArgs g) {
  constexpr int NP = SYM ? 1 : 2;  // accumulator planes
  constexpr int SHIFT = (A4 ? 4 : 0) + (W4 ? 4 : 0);
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][TILE_BYTES];  // [buf][A/W]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tn = blockIdx.x, tm = blockIdx.y;
  const int n0 = tn * BN;
  RowMap rm{CFG ? tm * 64 : tm * BM, g.M, g.Mh};

  // Rows this thread loads for A and W.
  int64_t aoff[2], woff[2];
  bool aval[2], wval[2];
  {
    const int nrow = A4 ? 1 : 2;
    for (int h = 0; h < nrow; ++h) {
      const int lr = A4 ? (tid >> 1) : ((tid >> 2) + h * 64);
      bool v;
      const int r = rm.row<CFG>(lr, v);
      aval[h] = v;
      aoff[h] = v ? (int64_t)r * g.lda : 0;
    }
    const int nw = W4 ? 1 : 2;
    for (int h = 0; h < nw; ++h) {
      const int lr = W4 ? (tid >> 1) : ((tid >> 2) + h * 64);
      const int n = n0 + lr;
      wval[h] = n < g.N;
      woff[h] = wval[h] ? (int64_t)n * g.ldw : 0;
    }
  }

  v4i acc[NP][4][4];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[p][i][j] = v4i{0, 0, 0, 0};

  TileLoad<A4> ta;
  TileLoad<W4> tw;
  const int nk = (g.K + BK - 1) / BK;
  load_tile<A4>(ta, g.A, aoff, aval, 0, g.K, tid);
  load_tile<W4>(tw, g.W, woff, wval, 0, g.K, tid);
  store_tile<A4>(ta, smem[0][0], tid);
  store_tile<W4>(tw, smem[0][1], tid);
  __syncthreads();

  const int frow = lane & 15;
  const int fk = (lane >> 4) * 16;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_tile<A4>(ta, g.A, aoff, aval, (kt + 1) * BK, g.K, tid);
      load_tile<W4>(tw, g.W, woff, wval, (kt + 1) * BK, g.K, tid);
    }
    const uint8_t* As = smem[cur][0];
    const uint8_t* Ws = smem[cur][1];
    v4i b[4];
#pragma unroll
    for (int nj = 0; nj < 4; ++nj)
      b[nj] = as_v4i(*reinterpret_cast<const uint4*>(Ws + (wn * 64 + nj * 16 + frow) * LDS_ROW + fk));
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const uint4 a = *reinterpret_cast<const uint4*>(As + (wm * 64 + mi * 16 + frow) * LDS_ROW + fk);
      if constexpr (SYM) {
        const v4i av = as_v4i(a);
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) acc[0][mi][nj] = mfma(av, b[nj], acc[0][mi][nj]);
      } else {
        uint4 ap, an;
        split_polarity(a.x, ap.x, an.x);
        split_polarity(a.y, ap.y, an.y);
        split_polarity(a.z, ap.z, an.z);
        split_polarity(a.w, ap.w, an.w);
        const v4i vp = as_v4i(ap), vn = as_v4i(an);
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
          acc[0][mi][nj] = mfma(vp, b[nj], acc[0][mi][nj]);
          acc[1][mi][nj] = mfma(vn, b[nj], acc[1][mi][nj]);
        }
      }
    }
    if (kt + 1 < nk) {
      store_tile<A4>(ta, smem[cur ^ 1][0], tid);
      store_tile<W4>(tw, smem[cur ^ 1][1], tid);
    }
    __syncthreads();
  }

  // ---- epilogue ----
  const float sp = g.act_scales[0];
  const float sn = g.act_scales[1];
  float sw[4];
  int col[4];
#pragma unroll
  for (int nj = 0; nj < 4; ++nj) {
    col[nj] = n0 + wn * 64 + nj * 16 + (lane & 15);
    sw[nj] = col[nj] < g.N ? g.w_scales[col[nj]] : 0.0f;
  }
  const int rsub = (lane >> 4) * 4;

  if constexpr (DBG) {
    const int64_t plane = (int64_t)g.M * g.N;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bool v;
        const int grow = rm.row<CFG>(wm * 64 + mi * 16 + rsub + r, v);
        if (!v) continue;
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
          if (col[nj] >= g.N) continue;
          const int64_t e = (int64_t)grow * g.N + col[nj];
          g.dbg[e] = acc[0][mi][nj][r] >> SHIFT;
          g.dbg[plane + e] = SYM ? 0 : (acc[NP - 1][mi][nj][r] >> SHIFT);
        }
      }
  }

  if constexpr (CFG) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int crow = rm.m0 + wm * 32 + mi * 16 + rsub + r;
        if (crow >= g.Mh) continue;
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
          if (col[nj] >= g.N) continue;
          const float yc = epi<SYM>(acc[0][mi][nj][r] >> SHIFT, acc[NP - 1][mi][nj][r] >> SHIFT,
                                    sp, sn, sw[nj], g.inv_b);
          const float yu = epi<SYM>(acc[0][mi + 2][nj][r] >> SHIFT,
                                    acc[NP - 1][mi + 2][nj][r] >> SHIFT, sp, sn, sw[nj], g.inv_b);
          const float d = __fsub_rn(yc, yu);
          const float t = __fmul_rn(g.guidance, d);
          g.Y[(int64_t)crow * g.N + col[nj]] = __fadd_rn(yu, t);
        }
      }
  } else {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int grow = rm.m0 + wm * 64 + mi * 16 + rsub + r;
        if (grow >= g.M) continue;
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
          if (col[nj] >= g.N) continue;
          g.Y[(int64_t)grow * g.N + col[nj]] =
              epi<SYM>(acc[0][mi][nj][r] >> SHIFT, acc[NP - 1][mi][nj][r] >> SHIFT, sp, sn,
                       sw[nj], g.inv_b);
        }
      }
  }
}

template <bool A4, bool W4, bool SYM, bool CFG>
hipError_t run(const GemmArgs& g, hipStream_t s) {
  const int rows = CFG ? g.Mh : g.M;
  const int rt = CFG ? (rows + 63) / 64 : (rows + BM - 1) / BM;
  const dim3 grid((g.N + BN - 1) / BN, rt);
  if (g.dbg)
    hipLaunchKernelGGL((k2_gemm<A4, W4, SYM, CFG, true>), grid, dim3(kThreads), 0, s, g);
  else
    hipLaunchKernelGGL((k2_gemm<A4, W4, SYM, CFG, false>), grid, dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

template <bool A4, bool W4>
hipError_t run_mode(const GemmArgs& g, int sym, int cfg, hipStream_t s) {
  if (sym) return cfg ? run<A4, W4, true, true>(g, s) : run<A4, W4, true, false>(g, s);
  return cfg ? run<A4, W4, false, true>(g, s) : run<A4, W4, false, false>(g, s);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, int a4, int w4, int sym, int cfg, hipStream_t s) {
  if (a4) return w4 ? run_mode<true, true>(g, sym, cfg, s) : run_mode<true, false>(g, sym, cfg, s);
  return w4 ? run_mode<false, true>(g, sym, cfg, s) : run_mode<false, false>(g, sym, cfg, s);
}

}  // namespace ql
