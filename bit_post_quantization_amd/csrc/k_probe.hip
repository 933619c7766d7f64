// Measurement aid, not a step of the method: the int8 matrix-core rate the
// device sustains, the measured ceiling beside the GEMM's spec-peak
// roofline. The int8 GEMM's step structure, memory pipeline and epilogue are
// all absent here: only v_mfma_i32_16x16x64_i8 on register operands.
//
// Every wave loads the same 16 operand fragments (8 activation-side, 8
// weight-side; lane l holds 16 bytes of each) and issues 16 MFMAs per
// iteration into 16 independent accumulators. Successive MFMAs take
// different operand pairs, so with random bytes the multiplier inputs switch
// on every instruction (the power draw of real data), and with constant
// bytes they do not. Each thread finally writes the wrapped int32 sum of its
// 64 accumulator registers, which keeps every product live and lets a test
// check the whole computation against a host-side sum.
#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kProbeFrags = 8;  // operand fragments per side
constexpr int kProbeAcc = 16;   // independent accumulators per wave

template <int WPS>
__global__ __launch_bounds__(256 * WPS, 1) void k_probe_mfma(const v4i* __restrict__ ops, int iters,
                                                          int* __restrict__ sink) {
  const int lane = threadIdx.x & (kWave - 1);
  v4i a[kProbeFrags], b[kProbeFrags];
#pragma unroll
  for (int f = 0; f < kProbeFrags; ++f) {
    a[f] = ops[f * kWave + lane];
    b[f] = ops[(kProbeFrags + f) * kWave + lane];
  }
  v4i acc[kProbeAcc];
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j) acc[j] = v4i{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j)
      acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j % kProbeFrags],
                                                     b[(j + j / kProbeFrags) % kProbeFrags],
                                                     acc[j], 0, 0, 0);
  }
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j)
    s += (uint32_t)acc[j][0] + (uint32_t)acc[j][1] + (uint32_t)acc[j][2] + (uint32_t)acc[j][3];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = (int)s;
}

}  // namespace

hipError_t launch_probe_mfma(const void* ops, int iters, int waves_per_simd, int blocks, int* sink,
                             hipStream_t s) {
  const v4i* o = reinterpret_cast<const v4i*>(ops);
  if (waves_per_simd == 1)
    hipLaunchKernelGGL(k_probe_mfma<1>, dim3(blocks), dim3(256), 0, s, o, iters, sink);
  else
    hipLaunchKernelGGL(k_probe_mfma<2>, dim3(blocks), dim3(512), 0, s, o, iters, sink);
  return hipGetLastError();
}

}  // namespace ql
