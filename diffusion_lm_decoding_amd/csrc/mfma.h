// MFMA traits and the packed operand layout shared by every kernel.
//
// All matrix operands (weights and activations) live in HBM in "fragment
// order": a matrix with R rows and K columns is cut into tiles of 32 rows x KF
// columns; each tile is 64 lanes x 16 bytes, and lane l's 16 bytes are
// exactly what lane l of a 32x32 MFMA needs for that tile.  A wave therefore
// loads one operand tile with a single fully coalesced 1 KiB access.
//
//   bf16: one v_mfma_f32_32x32x16_bf16 per tile, KF = 16.
//         element (i, k) -> lane i + 32*(k/8), slot k%8.
//   f32 : four v_mfma_f32_32x32x2_f32 per tile, KF = 8.
//         element (i, k) -> lane i + 32*(k%2), slot k/2.
//
// The same map is used for the A operand (rows = output features) and the B
// operand (rows = tokens), so C[i][j] = sum_k A[i][k] B[j][k].  The 32x32 fp32
// result of lane l, register r sits at row i = 8*(r/4) + 4*(l/32) + r%4,
// column j = l%32 (checked on gfx950 against a host reference).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace dllm {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef uint16_t bf16_t;  // bf16 bit pattern in memory

typedef uint32_t Frag16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// round to nearest even (inputs are finite or propagate NaN as NaN)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct Mfma;

template <> struct Mfma<bf16_t> {
  static constexpr int KF = 16;   // k per 16-byte fragment
  static constexpr int E = 8;     // elements per lane per fragment
  __device__ static __forceinline__ int lane_of(int i, int k) { return i + 32 * (k >> 3); }
  __device__ static __forceinline__ int slot_of(int, int k) { return k & 7; }
  __host__ __device__ static constexpr int k_of(int lane, int slot) { return 8 * (lane >> 5) + slot; }
  __device__ static __forceinline__ f32x16 mma(const Frag16& a, const Frag16& b, f32x16 c) {
    bf16x8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ bf16_t store_cvt(float v) { return f32_to_bf16(v); }
};

template <> struct Mfma<float> {
  static constexpr int KF = 8;
  static constexpr int E = 4;
  __device__ static __forceinline__ int lane_of(int i, int k) { return i + 32 * (k & 1); }
  __device__ static __forceinline__ int slot_of(int, int k) { return k >> 1; }
  __host__ __device__ static constexpr int k_of(int lane, int slot) { return 2 * slot + (lane >> 5); }
  __device__ static __forceinline__ f32x16 mma(const Frag16& a, const Frag16& b, f32x16 c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ float store_cvt(float v) { return v; }
};

// Element offset of (row, k) in a packed matrix with K columns (K % KF == 0).
template <typename T>
__device__ __forceinline__ size_t packed_off(int row, int k, int K) {
  constexpr int KF = Mfma<T>::KF, E = Mfma<T>::E;
  size_t tile = static_cast<size_t>(row >> 5) * (K / KF) + (k / KF);
  int kk = k % KF;
  return (tile * 64 + Mfma<T>::lane_of(row & 31, kk)) * E + Mfma<T>::slot_of(row & 31, kk);
}

// Row i (0..31) and column j of accumulator register r of lane l.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

}  // namespace dllm
