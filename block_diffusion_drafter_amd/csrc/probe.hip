// Measurement aid: a loop that keeps every matrix core of the chip busy with
// bf16 MFMAs and nothing else, so a projection's MFMA rate can be reported
// against what this chip sustains under full load (its clock drops below the
// nominal one when all CUs multiply), beside the datasheet peak.
#include "common.h"
#include "internal.h"

namespace dflash {

namespace {

constexpr int kProbeThreads = 512;  // 8 waves: two per SIMD
constexpr int kProbeChains = 8;     // independent accumulators per wave (covers the MFMA latency)

// Each wave issues iters x kProbeChains v_mfma_f32_16x16x32_bf16 on operands
// with varied, nonzero bits (an all-zero operand draws less power, which
// would let the clock stay higher than under a real GEMM). Every wave's lane
// 0 stores one sum of its accumulators so the loop cannot be dropped.
__global__ __launch_bounds__(kProbeThreads) void mfma_loop_kernel(int iters, float* sink) {
  const unsigned gid = blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = gid * 2654435761u + 0x9E3779B9u;
  u32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // xorshift32; two bf16 per word in [-1, -0.5] U [0.5, 1]: sign and mantissa random
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    a[i] = (x & 0x807F807Fu) | 0x3F003F00u;
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    b[i] = (x & 0x807F807Fu) | 0x3F003F00u;
  }
  f32x4 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = mfma_frag<bf16>(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if ((threadIdx.x & 63) == 0) sink[gid >> 6] = s;
}

}  // namespace

}  // namespace dflash

using namespace dflash;

extern "C" int32_t dflash_probe_mfma_bf16(int32_t n_workgroups, int32_t iters, float* sink,
                                          double* flops, void* stream) {
  if (n_workgroups < 1 || iters < 1) return DFLASH_ERR_SHAPE;
  if (!sink) return DFLASH_ERR_NULL;
  if (flops)
    *flops = (double)n_workgroups * (kProbeThreads / 64) * (double)iters * kProbeChains * 16.0 *
             16.0 * 32.0 * 2.0;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(n_workgroups), dim3(kProbeThreads), 0,
                     (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}
