// Attention softmax(Q K^T / sqrt(dh)) V over the layer's KV cache.
//
// The fresh K/V of the rows being recomputed were already written into their
// cache rows by the Q/K/V epilogue, so the keys of every query are one
// contiguous range [0, limit) of the cache: prefix, fresh block and suffix are
// read in place and no concatenated copy exists.  limit is the canvas length
// for the refresh-style modes and the end of the query's block for block
// diffusion (prompt queries: the prompt length).
//
// One workgroup owns (sequence, head, 32 queries) and a contiguous share of the
// key tiles; its 4 waves take alternate 32-key tiles.  Per tile a wave computes
// S^T = K Q^T with MFMA (keys on rows, the 32 queries on columns: lane l owns
// query l%32), updates an online softmax in log2 units, and multiplies P V with
// MFMA while P stays in registers: the V^T fragment is read with the key
// permutation that matches the accumulator layout of S^T.  Wave states are
// merged in LDS, key shares through a workspace read back in share order by
// the last-arriving workgroup; the merge order is fixed.
//
// Cache layouts: K [batch][H][seq_pad][dh] (head dims in the rotary pair order
// of the projection), V^T [batch][H][dh][seq_pad].
#pragma once
#include "gemm.h"

namespace dllm {

constexpr int kMaxAttnSplits = 8;   // key shares per (sequence, head, 32 queries)

struct AttnArgs {
  const void* q;      // T [rows][d]
  const void* kc;     // T, layer base
  const void* vt;     // T, layer base
  void* out;          // T packed [rows][d]
  RowGeom g;
  int H, d, seq_pad;
  int N, P, blk, block_causal;
  int qblocks, splits;
  float scale_log2;
  float* ws;          // key-share partials when splits > 1
};

__device__ __forceinline__ int attn_limit(const AttnArgs& a, int pos) {
  if (!a.block_causal) return a.N;
  if (pos < a.P) return a.P;
  return a.P + ((pos - a.P) / a.blk + 1) * a.blk;
}

template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int KF = Mfma32<T>::KF;
  constexpr int NQF = DH / KF;   // fragments along dh
  constexpr int ND = DH / 32;    // output d-tiles
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hf = lane >> 5;
  const int wg = blockIdx.x, split = blockIdx.y;
  const int qb = wg % a.qblocks, bh = wg / a.qblocks;
  const int h = bh % a.H, b = bh / a.H;

  const int irow = qb * 32 + (lane & 31);
  const bool valid = irow < a.g.nr;
  const int m = b * a.g.nr + (valid ? irow : 0);
  const int pos = a.g.row_start + (valid ? irow : 0);
  const int limit = valid ? attn_limit(a, pos) : 0;
  const int last = min(a.g.nr, qb * 32 + 32) - 1;
  const int kmax = attn_limit(a, a.g.row_start + last);
  const int ntile = (kmax + 31) / 32;
  const int t0 = (int)((long)ntile * split / a.splits), t1 = (int)((long)ntile * (split + 1) / a.splits);

  const T* q = static_cast<const T*>(a.q);
  const T* kc = static_cast<const T*>(a.kc) + ((size_t)b * a.H + h) * a.seq_pad * DH;
  const T* vt = static_cast<const T*>(a.vt) + ((size_t)b * a.H + h) * DH * a.seq_pad;

  Frag16 qf[NQF];
#pragma unroll
  for (int c = 0; c < NQF; ++c) {
    const T* src = q + (size_t)m * a.d + h * DH + c * KF;
    if constexpr (sizeof(T) == 2) {
      qf[c] = *reinterpret_cast<const Frag16*>(src + 8 * hf);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[c][e] = __float_as_uint(reinterpret_cast<const float*>(src)[2 * e + hf]);
    }
  }

  float mrun = -INFINITY, lrun = 0.f;
  f32x16 o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;

  for (int t = t0 + wave; t < t1; t += 4) {
    const int kb = t * 32;
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const T* krow = kc + (size_t)(kb + (lane & 31)) * DH;
    // 16-bit types: the tile's K and V fragments are requested together, so the
    // V latency hides behind the QK^T products and the softmax
    Frag16 kf[NQF];
    Frag16 vf[ND][2];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c = 0; c < NQF; ++c) kf[c] = *reinterpret_cast<const Frag16*>(krow + c * KF + 8 * hf);
#pragma unroll
      for (int i = 0; i < ND; ++i) {
        const T* vrow = vt + (size_t)(i * 32 + (lane & 31)) * a.seq_pad + kb + 4 * hf;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 16 * c);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 * c + 8);
          vf[i][c] = Frag16{lo.x, lo.y, hi.x, hi.y};
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < NQF; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) kf[c][e] = __float_as_uint(reinterpret_cast<const float*>(krow)[c * KF + 2 * e + hf]);
    }
#pragma unroll
    for (int c = 0; c < NQF; ++c) s = Mfma32<T>::mma(kf[c], qf[c], s);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + acc32_row(r, lane);
      s[r] = key < limit ? s[r] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mrun, mx);
    const float msafe = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = exp2f(mrun - msafe);
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = exp2f(s[r] - msafe);
      psum += s[r];
    }
    psum += __shfl_xor(psum, 32);
    lrun = lrun * alpha + psum;
    mrun = mnew;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;

    // P V: the accumulator register r of S^T holds key kb + acc32_row(r, lane)
    if constexpr (sizeof(T) == 2) {
      Frag16 pf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pf[c][e] = Elem<T>::bits(s[8 * c + 2 * e]) | (Elem<T>::bits(s[8 * c + 2 * e + 1]) << 16);
#pragma unroll
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c) o[i] = Mfma32<T>::mma(vf[i][c], pf[c], o[i]);
    } else {
#pragma unroll
      for (int i = 0; i < ND; ++i) {
        const float* vrow = reinterpret_cast<const float*>(vt) + (size_t)(i * 32 + (lane & 31)) * a.seq_pad + kb + 4 * hf;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const Frag16 vf = *reinterpret_cast<const Frag16*>(vrow + 8 * u);
          Frag16 pf;
#pragma unroll
          for (int e = 0; e < 4; ++e) pf[e] = __float_as_uint(s[4 * u + e]);
          o[i] = Mfma32<T>::mma(vf, pf, o[i]);
        }
      }
    }
  }

  // merge the four waves (fixed order 0, 1, 2, 3)
  __shared__ float sm_m[4][64], sm_l[4][64];
  __shared__ float sm_o[3][ND][16][64];
  sm_m[wave][lane] = mrun;
  sm_l[wave][lane] = lrun;
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) sm_o[wave - 1][i][r][lane] = o[i][r];
  }
  __syncthreads();
  if (wave != 0) return;
  float M = mrun;
#pragma unroll
  for (int w = 1; w < 4; ++w) M = fmaxf(M, sm_m[w][lane]);
  const float Ms = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  {
    const float f0 = exp2f(mrun - Ms);
    L = lrun * f0;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= f0;
  }
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const float f = exp2f(sm_m[w][lane] - Ms);
    L += sm_l[w][lane] * f;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] += sm_o[w - 1][i][r][lane] * f;
  }

  if (a.splits > 1) {
    const size_t rec = (size_t)(ND * 16 + 2) * 64;
    float* dst = a.ws + ((size_t)split * gridDim.x + wg) * rec;
    dst[lane] = M;
    dst[64 + lane] = L;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[128 + (i * 16 + r) * 64 + lane] = o[i][r];
    return;  // attn_merge_kernel combines the key shares
  }

  if (!valid) return;
  const float inv = 1.0f / L;
  T* out = static_cast<T*>(a.out);
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      out[packed_off<T>(m, h * DH + i * 32 + acc32_row(r, lane), a.d)] = Elem<T>::cvt(o[i][r] * inv);
}

// Combine the key shares of a split attention launch in share order (one wave
// per (sequence, head, 32 queries)); launched after attn_kernel on the same
// stream, so every share is complete.
// 256 threads: thread t handles accumulator lane t%64 and the registers
// (i, r) with (16 i + r) % 4 == t/64.
template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int nwg) {
  constexpr int ND = DH / 32;
  constexpr int PER = ND * 16 / 4;
  const int lane = threadIdx.x & 63, part = threadIdx.x >> 6, wg = blockIdx.x;
  const int qb = wg % a.qblocks, bh = wg / a.qblocks;
  const int h = bh % a.H, b = bh / a.H;
  const int irow = qb * 32 + (lane & 31);
  if (irow >= a.g.nr) return;
  const int m = b * a.g.nr + irow;
  const size_t rec = (size_t)(ND * 16 + 2) * 64;
  const float* base = a.ws + (size_t)wg * rec;
  const size_t sstride = (size_t)nwg * rec;
  // every load is issued before the first use (splits <= kMaxAttnSplits)
  float mv[kMaxAttnSplits], lv[kMaxAttnSplits], ov[kMaxAttnSplits][PER];
#pragma unroll
  for (int sp = 0; sp < kMaxAttnSplits; ++sp) {
    const bool on = sp < a.splits;
    const float* src = base + sp * sstride;
    mv[sp] = on ? src[lane] : -INFINITY;
    lv[sp] = on ? src[64 + lane] : 0.f;
#pragma unroll
    for (int q = 0; q < PER; ++q) ov[sp][q] = on ? src[128 + (4 * q + part) * 64 + lane] : 0.f;
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxAttnSplits; ++sp) M = fmaxf(M, mv[sp]);
  const float Mz = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  float o[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) o[q] = 0.f;
#pragma unroll
  for (int sp = 0; sp < kMaxAttnSplits; ++sp) {
    const float f = sp < a.splits ? exp2f(mv[sp] - Mz) : 0.f;
    L += lv[sp] * f;
#pragma unroll
    for (int q = 0; q < PER; ++q) o[q] += ov[sp][q] * f;
  }
  const float inv = 1.0f / L;
  T* out = static_cast<T*>(a.out);
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int ir = 4 * q + part, i = ir / 16, r = ir % 16;
    out[packed_off<T>(m, h * DH + i * 32 + acc32_row(r, lane), a.d)] = Elem<T>::cvt(o[q] * inv);
  }
}

}  // namespace dllm
