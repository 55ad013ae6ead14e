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
// key tiles (shares spread short batches over all CUs); its NW waves take the
// 32-key tiles round-robin.  Per tile a wave computes S^T = K Q^T with MFMA (keys on rows,
// the 32 queries on columns: lane l owns query l%32), updates an online
// softmax in log2 units, and multiplies P V with MFMA while P stays in
// registers: the V^T fragment holds the keys in the order that matches the
// accumulator layout of S^T.  The wave states are merged pairwise in LDS (a
// fixed binary tree).
//
// With several key shares each workgroup writes its state to a workspace and
// attn_merge_kernel, launched next on the same stream, combines the shares in
// share order.  (Letting the
// last-arriving workgroup combine them instead needs an agent-scope
// release/acquire pair per workgroup, i.e. an L2 write-back and invalidate on
// every XCD; measured slower on MI355X than the second launch.)  Every merge
// order is fixed, so results are run-to-run identical.
//
// Cache layouts: K [batch][H][seq_pad][dh] (head dims in the rotary pair order
// of the projection), V^T [batch][H][dh][seq_pad] with, for 16-bit types, the
// keys of each 32-key tile in the order given by vt_col (gemm.h).
#pragma once
#include "gemm.h"

namespace dllm {

constexpr int kMaxAttnSplits = 16;  // key shares per (sequence, head, 32 queries)

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

// Online-softmax states (m, l, o) of the same queries over disjoint keys:
// (m1, l1, o1) <- their combination.
template <int ND>
__device__ __forceinline__ void attn_combine(float& m1, float& l1, f32x16 (&o1)[ND], float m2, float l2,
                                             const float (*o2)[16][64], int lane) {
  const float M = fmaxf(m1, m2);
  const float Ms = M == -INFINITY ? 0.f : M;
  const float f1 = exp2f(m1 - Ms), f2 = exp2f(m2 - Ms);
  l1 = l1 * f1 + l2 * f2;
  m1 = M;
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o1[i][r] = o1[i][r] * f1 + o2[i][r][lane] * f2;
}

// Which rows, keys and key tiles a workgroup covers.
struct AttnWork {
  int lane, wave, hf, wg, split, h, b;
  int m, limit;   // this lane's query row and its key limit
  bool valid;
  int t0, t1;     // key tiles [t0, t1) of this share
  // key share split_ of splits_ (blockIdx.y of a.splits by default)
  __device__ AttnWork(const AttnArgs& a) : AttnWork(a, blockIdx.y, a.splits) {}
  __device__ AttnWork(const AttnArgs& a, int split_, int splits_) {
    lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    hf = lane >> 5;
    wg = blockIdx.x;
    split = split_;
    const int qb = wg % a.qblocks, bh = wg / a.qblocks;
    h = bh % a.H;
    b = bh / a.H;
    const int irow = qb * 32 + (lane & 31);
    valid = irow < a.g.nr;
    m = b * a.g.nr + (valid ? irow : 0);
    limit = valid ? attn_limit(a, a.g.row_start + irow) : 0;
    const int last = min(a.g.nr, qb * 32 + 32) - 1;
    const int ntile = (attn_limit(a, a.g.row_start + last) + 31) / 32;
    t0 = (int)((long)ntile * split / splits_);
    t1 = (int)((long)ntile * (split + 1) / splits_);
  }
};

// S^T = K Q^T for one 32-key tile, online-softmax update, o += P V over ND
// 32-dim output tiles.  kf: K fragments of the tile; for 16-bit types vf holds
// the V^T fragments (d-tile i, key half c) in vt_col order.
template <typename T, int DH, int ND = DH / 32>
__device__ __forceinline__ void attn_tile16(const Frag16 (&qf)[DH / 16], const Frag16 (&kf)[DH / 16],
                                            const Frag16 (&vf)[ND][2], int kb, int limit, float scale_log2,
                                            float& mrun, float& lrun, f32x16 (&o)[ND], int lane) {
  constexpr int NQF = DH / 16;
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
  for (int c = 0; c < NQF; ++c) s = Mfma32<T>::mma(kf[c], qf[c], s);
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = kb + acc32_row(r, lane);
    s[r] = key < limit ? s[r] * scale_log2 : -INFINITY;
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
  // accumulator register r of S^T holds key kb + acc32_row(r, lane)
  Frag16 pf[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) pf[c][e] = Elem<T>::bits(s[8 * c + 2 * e]) | (Elem<T>::bits(s[8 * c + 2 * e + 1]) << 16);
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c) o[i] = Mfma32<T>::mma(vf[i][c], pf[c], o[i]);
}

// Merge the NW wave states (tree in LDS, lds: >= (NW/2) * (2 + 16 ND) * 64
// floats, free on entry), then wave 0 writes the normalised output dims
// [d0, d0 + 32 ND) of the head or, with several key shares (ND = DH/32), the
// share's state to the workspace.
template <typename T, int DH, int NW, int ND = DH / 32>
__device__ __forceinline__ void attn_finish(const AttnArgs& a, const AttnWork& w, float mrun, float lrun,
                                            f32x16 (&o)[ND], float* lds, int d0 = 0) {
  const int lane = w.lane, wave = w.wave;
  if constexpr (NW > 1) {
    float (*sm_m)[64] = reinterpret_cast<float (*)[64]>(lds);
    float (*sm_l)[64] = reinterpret_cast<float (*)[64]>(lds + (NW / 2) * 64);
    float (*sm_o)[ND][16][64] = reinterpret_cast<float (*)[ND][16][64]>(lds + NW * 64);
#pragma unroll
    for (int half = NW / 2; half >= 1; half /= 2) {
      if (wave >= half && wave < 2 * half) {
        const int sl = wave - half;
        sm_m[sl][lane] = mrun;
        sm_l[sl][lane] = lrun;
#pragma unroll
        for (int i = 0; i < ND; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) sm_o[sl][i][r][lane] = o[i][r];
      }
      __syncthreads();
      if (wave < half) attn_combine<ND>(mrun, lrun, o, sm_m[wave][lane], sm_l[wave][lane], sm_o[wave], lane);
      if (half > 1) __syncthreads();
    }
  }
  if (wave != 0) return;
  if (a.splits > 1) {
    // share record: m[64], l[64], then o as [i][r / 4][lane][r % 4] so each
    // lane stores (and the merge loads) four accumulator registers at once
    const size_t rec = (size_t)(ND * 16 + 2) * 64;
    float* dst = a.ws + ((size_t)w.split * gridDim.x + w.wg) * rec;
    dst[lane] = mrun;
    dst[64 + lane] = lrun;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<f32x4*>(dst + 128 + ((i * 4 + r4) * 64 + lane) * 4) =
            f32x4{o[i][4 * r4], o[i][4 * r4 + 1], o[i][4 * r4 + 2], o[i][4 * r4 + 3]};
    return;  // attn_merge_kernel combines the key shares
  }
  if (!w.valid) return;
  const float inv = 1.0f / lrun;
  T* out = static_cast<T*>(a.out);
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      out[packed_off<T>(w.m, w.h * DH + d0 + i * 32 + acc32_row(r, lane), a.d)] = Elem<T>::cvt(o[i][r] * inv);
}

template <int NW, int DH, int ND = DH / 32>
constexpr int attn_merge_floats() { return (NW / 2) * (2 + 16 * ND) * 64; }

// Fragments are loaded into registers per tile: with the key shares spread
// over all CUs each wave holds about one tile, so a deeper copy pipeline has
// nothing to hide (an LDS-ring variant that streams a whole head through one
// workgroup measured no faster on MI355X: one CU cannot keep enough bytes in
// flight to cover the memory latency at this little compute per tile).
template <typename T, int DH, int NW>
__global__ __launch_bounds__(64 * NW) void attn_kernel(AttnArgs a) {
  constexpr int KF = Mfma32<T>::KF;
  constexpr int NQF = DH / KF;
  constexpr int ND = DH / 32;
  __shared__ float lds[attn_merge_floats<NW, DH>() > 0 ? attn_merge_floats<NW, DH>() : 1];
  const AttnWork w(a);
  const int lane = w.lane, hf = w.hf;
  const T* q = static_cast<const T*>(a.q);
  const T* kc = static_cast<const T*>(a.kc) + ((size_t)w.b * a.H + w.h) * a.seq_pad * DH;
  const T* vt = static_cast<const T*>(a.vt) + ((size_t)w.b * a.H + w.h) * DH * a.seq_pad;

  Frag16 qf[NQF];
#pragma unroll
  for (int c = 0; c < NQF; ++c) {
    const T* src = q + (size_t)w.m * a.d + w.h * DH + c * KF;
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

  for (int t = w.t0 + w.wave; t < w.t1; t += NW) {
    const int kb = t * 32;
    const T* krow = kc + (size_t)(kb + (lane & 31)) * DH;
    if constexpr (sizeof(T) == 2) {
      // the tile's K and V^T fragments are requested together (vt_col order:
      // fragment (i, c) is 16 contiguous bytes)
      Frag16 kf[NQF], vf[ND][2];
#pragma unroll
      for (int c = 0; c < NQF; ++c) kf[c] = *reinterpret_cast<const Frag16*>(krow + c * KF + 8 * hf);
#pragma unroll
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          vf[i][c] = *reinterpret_cast<const Frag16*>(vt + (size_t)(i * 32 + (lane & 31)) * a.seq_pad + kb +
                                                      (2 * c + hf) * 8);
      attn_tile16<T, DH>(qf, kf, vf, kb, w.limit, a.scale_log2, mrun, lrun, o, lane);
    } else {
      const float* kr = reinterpret_cast<const float*>(krow);
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int c = 0; c < NQF; ++c) {
        Frag16 kf;
#pragma unroll
        for (int e = 0; e < 4; ++e) kf[e] = __float_as_uint(kr[c * KF + 2 * e + hf]);
        s = Mfma32<T>::mma(kf, qf[c], s);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + acc32_row(r, lane);
        s[r] = key < w.limit ? s[r] * a.scale_log2 : -INFINITY;
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
      for (int i = 0; i < ND; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
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
  attn_finish<T, DH, NW>(a, w, mrun, lrun, o, lds);
}

// Few (sequence, head, 32-query) blocks (block steps of small batches;
// 16-bit caches): instead of key shares combined by a second launch, grid.y
// cuts the head's output dims into DH / (32 ND) slices.  Each workgroup runs
// the online softmax over every key tile (the scores are recomputed per
// slice: 8 MFMAs a tile, little next to the loads) and accumulates P V for
// its ND 32-dim output tiles only, so it writes final outputs and no merge
// kernel follows.  Its NW waves take the key tiles round-robin, requesting
// the next tile's fragments before the current tile's math, and are merged
// by the LDS tree.  With ND = DH / 32 (one slice: the whole head) it also
// serves a full round of blocks that needs no key shares (batch >= 8 steps).
template <typename T, int DH, int NW, int ND>
__global__ __launch_bounds__(64 * NW) void attn_dslice_kernel(AttnArgs a) {
  static_assert(sizeof(T) == 2, "16-bit caches");
  constexpr int NQF = DH / 16;
  __shared__ float lds[attn_merge_floats<NW, DH, ND>() > 0 ? attn_merge_floats<NW, DH, ND>() : 1];
  const AttnWork w(a, 0, 1);
  const int lane = w.lane, hf = w.hf;
  const int d0 = blockIdx.y * ND * 32;
  const T* q = static_cast<const T*>(a.q);
  const T* kc = static_cast<const T*>(a.kc) + ((size_t)w.b * a.H + w.h) * a.seq_pad * DH;
  const T* vt = static_cast<const T*>(a.vt) + ((size_t)w.b * a.H + w.h) * DH * a.seq_pad + (size_t)d0 * a.seq_pad;
  Frag16 qf[NQF];
#pragma unroll
  for (int c = 0; c < NQF; ++c) qf[c] = *reinterpret_cast<const Frag16*>(q + (size_t)w.m * a.d + w.h * DH + c * 16 + 8 * hf);
  float mrun = -INFINITY, lrun = 0.f;
  f32x16 o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  auto load = [&](int t, Frag16 (&kf)[NQF], Frag16 (&vf)[ND][2]) {
    const int kb = t * 32;
    const T* krow = kc + (size_t)(kb + (lane & 31)) * DH;
#pragma unroll
    for (int c = 0; c < NQF; ++c) kf[c] = *reinterpret_cast<const Frag16*>(krow + c * 16 + 8 * hf);
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        vf[i][c] = *reinterpret_cast<const Frag16*>(vt + (size_t)(i * 32 + (lane & 31)) * a.seq_pad + kb + (2 * c + hf) * 8);
  };
  Frag16 ka[NQF], va[ND][2], kb2[NQF], vb[ND][2];
  int t = w.t0 + w.wave;
  if (t < w.t1) load(t, ka, va);
  for (; t < w.t1; t += 2 * NW) {
    const bool second = t + NW < w.t1;
    if (second) load(t + NW, kb2, vb);
    attn_tile16<T, DH, ND>(qf, ka, va, t * 32, w.limit, a.scale_log2, mrun, lrun, o, lane);
    if (second) {
      if (t + 2 * NW < w.t1) load(t + 2 * NW, ka, va);
      attn_tile16<T, DH, ND>(qf, kb2, vb, (t + NW) * 32, w.limit, a.scale_log2, mrun, lrun, o, lane);
    }
  }
  attn_finish<T, DH, NW, ND>(a, w, mrun, lrun, o, lds, d0);
}

// Many query rows (cache passes, block-diffusion steps; 16-bit caches): a
// workgroup owns NW consecutive 32-query blocks of one (sequence, head), one
// per wave, and streams the key tiles its last block attends through an
// S-stage LDS ring filled by the DMA path, so each tile is read from memory
// once for 32 NW queries.  Every wave runs the online softmax of its own
// queries over every tile (keys past a query's limit are masked), and
// writes its normalised output; no key shares.
template <typename T, int DH, int NW, int S>
__global__ __launch_bounds__(64 * NW) void attn_wide_kernel(AttnArgs a) {
  static_assert(sizeof(T) == 2, "16-bit caches");
  constexpr int NQF = DH / 16, ND = DH / 32;
  constexpr int FR = NQF + 2 * ND;   // fragments per 32-key tile: K then V^T
  constexpr int LW = FR / NW;
  static_assert(FR % NW == 0, "tile fragments split evenly over the waves");
  __shared__ Frag16 ring[S][FR][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5;
  const int qgroups = (a.qblocks + NW - 1) / NW;
  const int qg = blockIdx.x % qgroups, bh = blockIdx.x / qgroups;
  const int h = bh % a.H, b = bh / a.H;
  const int qb = qg * NW + wave;                       // this wave's query block
  const int irow = qb * 32 + (lane & 31);
  const bool valid = irow < a.g.nr;
  const int m = b * a.g.nr + (valid ? irow : 0);
  const int limit = valid ? attn_limit(a, a.g.row_start + irow) : 0;
  // the workgroup's key tiles: what its last valid query row attends
  const int last = min(a.g.nr, qg * NW * 32 + NW * 32) - 1;
  const int nt = (attn_limit(a, a.g.row_start + last) + 31) / 32;
  const T* kc = static_cast<const T*>(a.kc) + ((size_t)b * a.H + h) * a.seq_pad * DH;
  const T* vt = static_cast<const T*>(a.vt) + ((size_t)b * a.H + h) * DH * a.seq_pad;

  // tile t's copies into ring slot `slot`; tiles past the workgroup's last
  // copy that tile again (valid memory, never used), so every loop body
  // issues the same copies and every wait below is a constant
  auto issue = [&](int t, int slot) __attribute__((always_inline)) {
    const int kb = min(t, nt - 1) * 32;
#pragma unroll
    for (int q = 0; q < LW; ++q) {
      const int f = wave + q * NW;
      const T* src;
      if (f < NQF) {
        src = kc + (size_t)(kb + (lane & 31)) * DH + f * 16 + 8 * hf;
      } else {
        const int g = f - NQF, i = g >> 1, c = g & 1;
        src = vt + (size_t)(i * 32 + (lane & 31)) * a.seq_pad + kb + (2 * c + hf) * 8;
      }
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)&ring[slot][f][0], 16, 0, 0);
    }
  };
  // the queries first: the wait for a tile's copies then covers them too
  Frag16 qf[NQF];
  const T* qrow = static_cast<const T*>(a.q) + (size_t)m * a.d + h * DH + 8 * hf;
#pragma unroll
  for (int c = 0; c < NQF; ++c) qf[c] = *reinterpret_cast<const Frag16*>(qrow + c * 16);
  float mrun = -INFINITY, lrun = 0.f;
  f32x16 o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  static_assert(S % 2 == 0 && S >= 2, "ring of an even number of tiles");
  auto read = [&](int slot, Frag16 (&k)[NQF], Frag16 (&v)[ND][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NQF; ++c) k[c] = ring[slot][c][lane];
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c) v[i][c] = ring[slot][NQF + 2 * i + c][lane];
  };
  // Ring slots are compile-time constants (S tiles per loop body): with a
  // run-time slot index the compiler waits for every copy in flight before
  // each LDS read.  One barrier per tile.
  // DB (4 waves, whose registers hold two tiles): tile t computes from one
  // register set while tile t + 1 is read into the other; S tiles in flight.
  // Otherwise one register set: a tile is read after the barrier that makes
  // it visible; S - 1 tiles in flight.
  constexpr bool DB = NW == 4;
  int t = 0;
  if constexpr (DB) {
    static_for<0, S>([&](auto t_c) { issue(decltype(t_c)::value, decltype(t_c)::value); });
    Frag16 kf[2][NQF], vf[2][ND][2];
    wait_vmcnt<(S - 1) * LW>();   // the queries and tile 0 have landed
    __builtin_amdgcn_s_barrier();
    read(0, kf[0], vf[0]);
    auto tile = [&](int tt, auto slot_c) __attribute__((always_inline)) {
      constexpr int slot = decltype(slot_c)::value, cur = slot % 2, nxt = 1 - cur;
      // tile tt + 1 landed (S - 2 later tiles in flight) and every wave has
      // read tile tt into registers: its slot takes tile tt + S
      wait_vmcnt<(S - 2) * LW>();
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
      issue(tt + S, slot);
      read((slot + 1) % S, kf[nxt], vf[nxt]);
      attn_tile16<T, DH>(qf, kf[cur], vf[cur], tt * 32, limit, a.scale_log2, mrun, lrun, o, lane);
    };
    for (; t + S <= nt; t += S)
      static_for<0, S>([&](auto i_c) __attribute__((always_inline)) { tile(t + decltype(i_c)::value, i_c); });
    static_for<0, S>([&](auto i_c) __attribute__((always_inline)) {
      if (t + decltype(i_c)::value < nt) tile(t + decltype(i_c)::value, i_c);
    });
  } else {
    static_for<0, S - 1>([&](auto t_c) { issue(decltype(t_c)::value, decltype(t_c)::value); });
    Frag16 kf[NQF], vf[ND][2];
    auto tile = [&](int tt, auto slot_c) __attribute__((always_inline)) {
      constexpr int slot = decltype(slot_c)::value;
      // tile tt landed (S - 2 later tiles in flight) and every wave has read
      // tile tt - 1: its slot takes tile tt + S - 1
      wait_vmcnt<(S - 2) * LW>();
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
      issue(tt + S - 1, (slot + S - 1) % S);
      read(slot, kf, vf);
      attn_tile16<T, DH>(qf, kf, vf, tt * 32, limit, a.scale_log2, mrun, lrun, o, lane);
    };
    for (; t + S <= nt; t += S)
      static_for<0, S>([&](auto i_c) __attribute__((always_inline)) { tile(t + decltype(i_c)::value, i_c); });
    static_for<0, S>([&](auto i_c) __attribute__((always_inline)) {
      if (t + decltype(i_c)::value < nt) tile(t + decltype(i_c)::value, i_c);
    });
  }
  wait_vmcnt<0>();   // the copies past the end
  if (!valid) return;
  const float inv = 1.0f / lrun;
  T* out = static_cast<T*>(a.out);
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      out[packed_off<T>(m, h * DH + i * 32 + acc32_row(r, lane), a.d)] = Elem<T>::cvt(o[i][r] * inv);
}

// Combine the key shares of a split attention launch in share order; launched
// after attn_kernel on the same stream, so every share is complete.  Grid
// (sequence x head x 32-query block, output d-tile of 32): wave w of the 4
// handles accumulator registers 4w .. 4w+3 of that d-tile, one 16-byte load
// per share, so each thread issues all of its loads (3 per share) before the
// first use.  MAXS >= a.splits bounds the unrolled share loop (sized at
// compile time: a larger bound costs registers and issue slots, 4.1 -> 5.7 us
// per launch on MI355X going from 16 to 32 at 8 shares).
template <typename T, int DH, int MAXS>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int nwg) {
  static_assert(MAXS <= kMaxAttnSplits, "share bound");
  const int lane = threadIdx.x & 63, part = threadIdx.x >> 6;
  const int wg = blockIdx.x, i = blockIdx.y;
  const int qb = wg % a.qblocks, bh = wg / a.qblocks;
  const int h = bh % a.H, b = bh / a.H;
  const int irow = qb * 32 + (lane & 31);
  if (irow >= a.g.nr) return;
  const int m = b * a.g.nr + irow;
  const size_t rec = (size_t)(DH / 32 * 16 + 2) * 64;
  const float* base = a.ws + (size_t)wg * rec;
  const size_t sstride = (size_t)nwg * rec;
  float mv[MAXS], lv[MAXS];
  f32x4 ov[MAXS];
#pragma unroll
  for (int sp = 0; sp < MAXS; ++sp) {
    const bool on = sp < a.splits;
    const float* src = base + sp * sstride;
    mv[sp] = on ? src[lane] : -INFINITY;
    lv[sp] = on ? src[64 + lane] : 0.f;
    ov[sp] = on ? *reinterpret_cast<const f32x4*>(src + 128 + ((i * 4 + part) * 64 + lane) * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < MAXS; ++sp) M = fmaxf(M, mv[sp]);
  const float Mz = M == -INFINITY ? 0.f : M;
  float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < MAXS; ++sp) {
    const float f = sp < a.splits ? exp2f(mv[sp] - Mz) : 0.f;
    L += lv[sp] * f;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] += ov[sp][q] * f;
  }
  const float inv = 1.0f / L;
  T* out = static_cast<T*>(a.out);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    out[packed_off<T>(m, h * DH + i * 32 + acc32_row(4 * part + q, lane), a.d)] = Elem<T>::cvt(o[q] * inv);
}

}  // namespace dllm
