// Achievable-peak microkernels: the measured ceilings the roofline fractions
// are read against, next to the vendor peaks.
//  * hbm_read_kernel: every 16-byte word of a buffer much larger than the
//    memory-side cache read once (grid-stride, 16 B per lane per load);
//  * mfma_loop_kernel: each wave keeps 8 independent 16x16x32 fp16 MFMA
//    accumulator chains busy from registers (no memory traffic).
// Both write a value derived from what they computed, so nothing is elided.
#pragma once
#include "mfma.h"

namespace dllm {

__global__ __launch_bounds__(256) void hbm_read_kernel(const Frag16* p, size_t n16, unsigned* sink) {
  unsigned acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += 4 * stride) {
    Frag16 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t j = i + u * stride;
      v[u] = j < n16 ? __builtin_nontemporal_load(p + j) : Frag16{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // practically never; keeps the loads live
}

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* sink) {
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (f16_t)(0.001f * (float)((threadIdx.x + e) & 7));
    b[e] = (f16_t)(0.002f * (float)((threadIdx.x * 3 + e) & 7));
  }
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == 1234.5f) sink[0] = s;
}

}  // namespace dllm
