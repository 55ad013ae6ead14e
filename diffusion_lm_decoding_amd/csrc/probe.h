// Achievable-peak microkernels: the measured ceilings the roofline fractions
// are read against, next to the vendor peaks.
//  * hbm_read_kernel: every 16-byte word of a buffer much larger than the
//    memory-side cache read once, in contiguous 32 KiB chunks per workgroup;
//  * mfma_loop_kernel: each wave keeps 4 independent 32x32x16 fp16 MFMA
//    accumulator chains busy from registers (no memory traffic).
// Both write a value derived from what they computed, so nothing is elided.
#pragma once
#include "mfma.h"

namespace dllm {

// Each workgroup reads 256 x 8 consecutive 16-byte words per iteration (8 KiB
// per wave-load group in flight), grid-striding over the buffer.
__global__ __launch_bounds__(256) void hbm_read_kernel(const Frag16* p, size_t n16, unsigned* sink) {
  constexpr int U = 8;
  unsigned acc = 0;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  for (size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x; i + 256 * (U - 1) < n16; i += stride) {
    Frag16 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + 256 * u);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // practically never; keeps the loads live
}

// 4 independent 32x32x16 fp16 accumulator chains per wave (on MI355X this
// form sustains close to the dense peak; 16x16x32 chains stay well below it).
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* sink) {
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (f16_t)(0.001f * (float)((threadIdx.x + e) & 7));
    b[e] = (f16_t)(0.002f * (float)((threadIdx.x * 3 + e) & 7));
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) s += acc[c][0] + acc[c][5] + acc[c][10] + acc[c][15];
  if (s == 1234.5f) sink[0] = s;
}

}  // namespace dllm
