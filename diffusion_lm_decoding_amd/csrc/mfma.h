// MFMA traits and the packed operand layout shared by every kernel.
//
// Projection operands (weights and activations) live in HBM in "fragment
// order": a matrix with R rows and K columns is cut into tiles of 16 rows x KF
// columns; each tile is 64 lanes x 16 bytes, and lane l's 16 bytes are exactly
// what lane l of a 16x16 MFMA needs for that tile, so a wave loads one operand
// tile with a single fully coalesced 1 KiB access.
//
//   bf16: one v_mfma_f32_16x16x32_bf16 per tile, KF = 32.
//         element (i, k) -> lane i + 16*(k/8), slot k%8.
//   f32 : four v_mfma_f32_16x16x4_f32 per tile, KF = 16.
//         element (i, k) -> lane i + 16*(k%4), slot k/4.
//
// The same map is used for the A operand (rows = output features) and the B
// operand (rows = tokens), so C[i][j] = sum_k A[i][k] B[j][k]; the 16x16 fp32
// result of lane l, register r sits at row i = 4*(l/16) + r, column j = l%16.
//
// Attention uses the 32x32 shapes (Mfma32): v_mfma_f32_32x32x16_bf16 with
// element (i, k) at lane i + 32*(k/8), slot k%8, and v_mfma_f32_32x32x2_f32
// (four per 16-byte fragment) with (i, k) at lane i + 32*(k%2), slot k/2; the
// 32x32 result of lane l, register r sits at row 8*(r/4) + 4*(l/32) + r%4,
// column l%32.  All four lane maps were checked on gfx950 against a host
// reference.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dllm {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint16_t bf16_t;  // bf16 bit pattern in memory
typedef uint32_t Frag16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// round to nearest even; NaN stays NaN
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

typedef _Float16 f16_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// element load / round-to-nearest-even store; bits() is the 16-bit pattern
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  __device__ static __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ bf16_t cvt(float v) { return f32_to_bf16(v); }
  __device__ static __forceinline__ uint32_t bits(float v) { return f32_to_bf16(v); }
};
template <> struct Elem<f16_t> {
  __device__ static __forceinline__ float load(const f16_t* p) { return (float)*p; }
  __device__ static __forceinline__ f16_t cvt(float v) { return (f16_t)v; }
  __device__ static __forceinline__ uint32_t bits(float v) { return __builtin_bit_cast(uint16_t, (f16_t)v); }
};
template <> struct Elem<float> {
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ float cvt(float v) { return v; }
};

// ---- 16x16 shapes: projections -------------------------------------------
template <typename T> struct Mfma16;

template <> struct Mfma16<bf16_t> {
  static constexpr int KF = 32;
  static constexpr int E = 8;
  __host__ __device__ static constexpr int lane_of(int i, int k) { return i + 16 * (k >> 3); }
  __host__ __device__ static constexpr int slot_of(int k) { return k & 7; }
  __device__ static __forceinline__ f32x4 mma(const Frag16& a, const Frag16& b, f32x4 c) {
    bf16x8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
  }
};

template <> struct Mfma16<f16_t> {
  static constexpr int KF = 32;
  static constexpr int E = 8;
  __host__ __device__ static constexpr int lane_of(int i, int k) { return i + 16 * (k >> 3); }
  __host__ __device__ static constexpr int slot_of(int k) { return k & 7; }
  __device__ static __forceinline__ f32x4 mma(const Frag16& a, const Frag16& b, f32x4 c) {
    f16x8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, c, 0, 0, 0);
  }
};

template <> struct Mfma16<float> {
  static constexpr int KF = 16;
  static constexpr int E = 4;
  __host__ __device__ static constexpr int lane_of(int i, int k) { return i + 16 * (k & 3); }
  __host__ __device__ static constexpr int slot_of(int k) { return k >> 2; }
  __device__ static __forceinline__ f32x4 mma(const Frag16& a, const Frag16& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
};

// Element offset of (row, k) in a packed matrix with K columns (K % KF == 0).
template <typename T>
__device__ __forceinline__ size_t packed_off(int row, int k, int K) {
  constexpr int KF = Mfma16<T>::KF, E = Mfma16<T>::E;
  const size_t tile = static_cast<size_t>(row >> 4) * (K / KF) + (k / KF);
  const int kk = k % KF;
  return (tile * 64 + Mfma16<T>::lane_of(row & 15, kk)) * E + Mfma16<T>::slot_of(kk);
}

// Row of accumulator register r of lane l in a 16x16 result.
__device__ __forceinline__ int acc16_row(int r, int lane) { return 4 * (lane >> 4) + r; }

// ---- 32x32 shapes: attention ----------------------------------------------
template <typename T> struct Mfma32;

template <> struct Mfma32<bf16_t> {
  static constexpr int KF = 16;
  __device__ static __forceinline__ f32x16 mma(const Frag16& a, const Frag16& b, f32x16 c) {
    bf16x8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
  }
};

template <> struct Mfma32<f16_t> {
  static constexpr int KF = 16;
  __device__ static __forceinline__ f32x16 mma(const Frag16& a, const Frag16& b, f32x16 c) {
    f16x8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c, 0, 0, 0);
  }
};

template <> struct Mfma32<float> {
  static constexpr int KF = 8;
  __device__ static __forceinline__ f32x16 mma(const Frag16& a, const Frag16& b, f32x16 c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
};

__device__ __forceinline__ int acc32_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

}  // namespace dllm
