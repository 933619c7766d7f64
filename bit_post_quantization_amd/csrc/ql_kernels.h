// Internal interface between the C ABI (qlinear_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

// Reduction workspace of one plan: per-block partial maxima written by the
// max-reduce kernel and read by the quantize kernel of the same call (stream
// order makes them visible; nothing needs clearing between calls).
constexpr int kMaxReduceBlocks = 1024;
constexpr int kMaxKSeg = 4;  // input branches (SegLinear input segmentation)
// Grid exchange of the one-pass quantizer. Workgroup b writes its partial
// maxima of input branch j as word[2j][b] = (sequence number << 32) | bits
// (the maximum) and word[2j+1][b] (the most negative value's magnitude);
// workgroup 0 waits for every word of the grid to carry the call's number,
// folds them, and writes the maxima of each branch the same way into
// result[2j], result[2j+1], which the other workgroups wait for. 64-bit
// words are written and read whole, so a tag and its value arrive together
// and no fence is needed; nothing is reset between calls. Zero at allocation
// (sequence numbers start at 1).
struct GridSync {
  uint64_t word[2 * kMaxKSeg][kMaxReduceBlocks];
  uint64_t result[2 * kMaxKSeg];
  uint32_t fallbacks;  // workgroups that stopped waiting and scanned X themselves
  uint32_t pad[47];
};
static_assert(sizeof(GridSync) % 256 == 0, "exchange words keep their alignment");
struct ReduceWs {
  // per branch: bits of max(+0, max x), max(+0, -min x)
  uint32_t part[kMaxKSeg][2][kMaxReduceBlocks];
  GridSync sync;
};

struct QuantArgs {
  const void* X;
  int64_t nunits;            // number of 4-element units (M*K/4)
  void* codes;
  float* act_scales;         // out [2 * nks]
  const float* static_scales;// in [2 * nks] or nullptr
  ReduceWs* ws;
  int reduce_blocks;         // partials written by the reduce kernel
  float qa;
  int keep_mask;             // ~((1 << lsb_k) - 1)
  int sym;
  int nks;                   // input branches (1: one scale pair for the tensor)
  int k_units;               // K / 4
  int ks_units[kMaxKSeg];    // branch starts in units (k_j / 4); unused ones = k_units
  uint32_t seq;              // call sequence number (one-pass quantizer's barrier), >= 1
};

struct GemmArgs {
  const uint8_t* A;          // activation codes: int8 [M,K] or packed [M,K/2]
  const uint8_t* W;          // weight codes: int8 [N,K], or 4-bit packed [N,K/2]
  const float* act_scales;   // [2 * nks]
  const float* w_scales;     // [nks * Nout]
  float* Y;                  // [M,N] or [M/2,N]
  int32_t* dbg;              // [2,M,N] or nullptr
  int M, N, K;               // N: weight rows (2 * roundup(Nout, 16) for single Hadamard)
  int Nout;                  // output columns (N except for single Hadamard)
  int Mh;                    // M/2 with CFG pairing
  int64_t lda, ldw;          // bytes per row of A / W
  float guidance;
  float inv_b;               // 1/B (rotation) or 1
  int nks;                   // input branches (1: none)
  int ks_end[kMaxKSeg];      // K-step (of 128) at which each branch but the last ends
  float* ypart_ws;           // input branches: kYSlots * kGemmThreads floats per workgroup
  int kofs[kMaxKSeg + 1];    // branch j covers K columns [kofs[j], kofs[j+1])
  int ksteps[kMaxKSeg];      // 128-column steps of branch j, rounded up to a multiple of 3
  int w_lsb_k;               // TASQ: low magnitude bits cleared from every weight code
};

// GEMM workgroup size and the per-thread partial-sum slots of a GEMM with
// input branches; the workspace holds one block per workgroup (at most one
// workgroup per compute unit).
constexpr int kGemmThreads = 512;
constexpr int kYSlots = 32;
inline size_t gemm_ypart_bytes(int cus) {
  return (size_t)cus * kYSlots * kGemmThreads * sizeof(float);
}

// K1: activation quantization. Returns the launch status.
hipError_t launch_quantize(const QuantArgs& a, int x_bf16, int hadamard_block, int a4,
                           hipStream_t s);

// K1 with input branches: launch_quantize handles a.nks > 1 too.
// K2 for single-Hadamard weight planes (requires sym).
hipError_t launch_gemm(const GemmArgs& g, int a4, int sym, int cfg, int hs, hipStream_t s);
// K2 for every other plan (k_gemm1.hip, one object per activation width and
// scale mode). w4: 4-bit weights packed two per byte.
hipError_t launch_gemm1_a0_s0(const GemmArgs& g, int cfg, int w4, hipStream_t s);
hipError_t launch_gemm1_a0_s1(const GemmArgs& g, int cfg, int w4, hipStream_t s);
hipError_t launch_gemm1_a1_s0(const GemmArgs& g, int cfg, int w4, hipStream_t s);
hipError_t launch_gemm1_a1_s1(const GemmArgs& g, int cfg, int w4, hipStream_t s);
inline hipError_t launch_gemm1(const GemmArgs& g, int a4, int sym, int cfg, int w4,
                               hipStream_t s) {
  if (a4) return sym ? launch_gemm1_a1_s1(g, cfg, w4, s) : launch_gemm1_a1_s0(g, cfg, w4, s);
  return sym ? launch_gemm1_a0_s1(g, cfg, w4, s) : launch_gemm1_a0_s0(g, cfg, w4, s);
}

// Measurement aid: the int8 MFMA ceiling microkernel (one workgroup of
// 256 * waves_per_simd threads per block, blocks = compute units).
hipError_t launch_probe_mfma(const void* ops, int iters, int waves_per_simd, int blocks, int* sink,
                             hipStream_t s);

// K3: standalone CFG combine.
hipError_t launch_cfg_combine(const float* Y, int64_t half_elems, float w, float* out,
                              hipStream_t s);

// K0: plan kernels.
hipError_t launch_rotate_rows(float* W, int64_t nunits, int hadamard_block, hipStream_t s);
// Max |W[n, c0 .. c0+cw)| per row (row stride K).
hipError_t launch_row_absmax(const float* W, int N, int K, int c0, int cw, uint32_t* rowmax,
                             hipStream_t s);
hipError_t launch_weight_scales(const uint32_t* rowmax, int N, int mode, const int32_t* seg,
                                int nseg, float qw, float* sw, hipStream_t s);
// Codes of the columns [c0, c0 + cw) of W (row stride K) with the scales sw[N].
hipError_t launch_quantize_weights(const float* W, const float* sw, int N, int K, int c0, int cw,
                                   float qw, uint8_t* out, hipStream_t s);
// Single-Hadamard weight planes: out has 2 * roundup(N, 16) rows of K bytes
// (hi / lo interleaved per 16 channels; rows past N must be zeroed by the
// caller). K % 4 == 0 and K % hadamard_block == 0.
hipError_t launch_fwht_split(const uint8_t* codes, int N, int K, int hadamard_block, uint8_t* out,
                             hipStream_t s);
// 4-bit codes (int8 in [-8, 7], n % 16 == 0, 16-byte aligned) packed two
// per byte: element 2i in the low nibble of byte i.
hipError_t launch_pack4(const uint8_t* codes, int64_t n, uint8_t* packed, hipStream_t s);
// Packed 4-bit codes back to int8, the k (0..3) low magnitude bits cleared.
hipError_t launch_unpack4(const uint8_t* packed, int64_t n, int k, uint8_t* codes, hipStream_t s);
// Weight codes with the k low magnitude bits cleared (nbytes % 16 == 0,
// 16-byte aligned), and a copy of the nsw weight scales.
hipError_t launch_truncate_weights(const uint8_t* in, int64_t nbytes, int k, uint8_t* out,
                                   const float* sw_in, float* sw_out, int nsw, hipStream_t s);

}  // namespace ql
