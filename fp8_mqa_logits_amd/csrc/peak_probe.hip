// Sustained fp8 MFMA throughput on this device, for the roofline report.  Not a
// step of the indexer: it gives the measured peak that the logits kernel's
// MFMA rate is set against, next to the published 5.0 PFLOP/s dense fp8 figure.
//
// Each wave issues back-to-back v_mfma_f32_16x16x128_f8f6f4 on kProbeChains
// independent accumulators (enough to cover the MFMA result latency), with
// operands held in registers, so nothing but the matrix pipe and the issue
// slot is exercised.  One MFMA is 2 * 16 * 16 * 128 = 65536 flops.
//
// A second probe runs the logits kernels' own per-fragment core (eight MFMAs,
// then ReLU, head weights and the cross-lane head reduction) on register
// operands with no memory traffic: at the logits kernel's occupancy its rate is
// the ceiling that the exact epilogue leaves to the kernel.

#include "device_common.hpp"
#include "launch.hpp"
#include "mqa_core.hpp"

#include <fp8idx.h>

namespace fp8idx {

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  // e4m3fn codes 0x30..0x37 (0.5 .. 0.9375): finite, so sums stay finite
  const int bytes = 0x30 + (lane & 7);
  const int word = bytes * 0x01010101;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = word;
    b[i] = word ^ (i << 24);
  }
  v4f acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) acc[j] = mfma_fp8_16x16x128(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kProbeThreads) void logits_core_probe_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  // e4m3fn codes 0x30..0x3f (0.5 .. 0.9375 and 1.0 .. 1.875): finite scores; weights of both signs
  QFrags qf;
#pragma unroll
  for (int qi = 0; qi < 4; ++qi)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 8; ++i) qf.a[qi][t][i] = (0x30 + ((lane + 5 * qi + 3 * t + i) & 15)) * 0x01010101;
#pragma unroll
      for (int i = 0; i < 4; ++i) qf.w[qi][t][i] = ((lane + i + qi + t) & 1) ? 0.25f + 0.01f * (4 * qi + i) : -0.125f;
    }
  v8i b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (0x38 + ((lane + 3 * i) & 7)) * 0x01010101;
  float acc = 0.f;
  for (int it = 0; it < iters; ++it) {
    b[0] ^= it & 7;   // a new B operand every fragment, as a key tile would give
    acc += fragment_logit(qf, b);
  }
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

hipError_t launch_logits_core_probe(int blocks, int iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(logits_core_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s, iters, out);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int blocks, int iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s, iters, out);
  return hipGetLastError();
}

}  // namespace fp8idx
