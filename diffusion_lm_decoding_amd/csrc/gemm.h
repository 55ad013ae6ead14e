// Projection GEMM  Y[m][n] = sum_k X[m][k] W[n][k]  on MFMA, with fused
// epilogues.  X and W are packed (mfma.h).  One workgroup (4 waves) owns one
// 32-column n-tile, MT 32-row m-tiles and one slice of K; its 4 waves split
// the slice four ways and stream their weight fragments straight from HBM
// (each weight byte is read once per m-group), adding into MT 32x32 fp32
// accumulators.  Partial sums are combined in a fixed order: waves through
// LDS, K-slices through a workspace that the last-arriving workgroup of the
// tile reads back in slice order (a ticket counter decides who is last; the
// order of arrival never changes the result).
#pragma once
#include "mfma.h"

namespace dllm {

struct RowGeom {
  int M;          // rows of this forward = batch * nr
  int nr;         // rows per sequence
  int row_start;  // canvas position of each sequence's first row
};

// ---------------------------------------------------------------------------
// epilogues: called once per (n-tile, m-tile) with the finished accumulator
// ---------------------------------------------------------------------------

// Q/K/V projection: rotary embedding on q and k (the packed weight rows of
// each head are ordered so that dims (j, j + dh/2) are adjacent output
// columns 2j, 2j+1), q to a row buffer, k and v into the layer's cache rows.
template <typename T>
struct EpiQKV {
  RowGeom g;
  int d, dh, H, seq_pad;
  T* q;             // [rows][d], per-head permuted dims
  T* kc;            // [batch][H][seq_pad][dh], permuted dims
  T* vt;            // [batch][H][dh][seq_pad], natural dims
  const float* cs;  // [seq][dh/2] cos
  const float* sn;  // [seq][dh/2] sin
  __device__ void operator()(int nt, int mt, const f32x16& acc, int lane) const {
    const int m = mt * 32 + (lane & 31);
    if (m >= g.M) return;
    const int b = m / g.nr;
    const int pos = g.row_start + m % g.nr;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int n0 = nt * 32 + 8 * q4 + 4 * (lane >> 5);
      float v[4] = {acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]};
      const int region = n0 / d, nn = n0 % d, h = nn / dh, p = nn % dh;
      if (region < 2) {
#pragma unroll
        for (int t = 0; t < 4; t += 2) {
          const int j = (p + t) >> 1;
          const float c = cs[pos * (dh / 2) + j], s = sn[pos * (dh / 2) + j];
          const float e = v[t], o = v[t + 1];
          v[t] = e * c - o * s;
          v[t + 1] = o * c + e * s;
        }
        T* dst = region == 0 ? q + (size_t)m * d + nn
                             : kc + (((size_t)b * H + h) * seq_pad + pos) * dh + p;
#pragma unroll
        for (int t = 0; t < 4; ++t) dst[t] = Mfma<T>::store_cvt(v[t]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          vt[(((size_t)b * H + h) * dh + p + t) * seq_pad + pos] = Mfma<T>::store_cvt(v[t]);
      }
    }
  }
};

// Residual update x[m][n] += y (fp32 residual stream).
struct EpiResidual {
  int M, ld;
  float* x;
  __device__ void operator()(int nt, int mt, const f32x16& acc, int lane) const {
    const int m = mt * 32 + (lane & 31);
    if (m >= M) return;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int n0 = nt * 32 + 8 * q4 + 4 * (lane >> 5);
      float4* p = reinterpret_cast<float4*>(x + (size_t)m * ld + n0);
      float4 r = *p;
      r.x += acc[4 * q4];
      r.y += acc[4 * q4 + 1];
      r.z += acc[4 * q4 + 2];
      r.w += acc[4 * q4 + 3];
      *p = r;
    }
  }
};

// SwiGLU: packed rows 2i / 2i+1 are gate row i / up row i, so each lane holds
// (g_i, u_i, g_{i+1}, u_{i+1}); a_i = silu(g_i) * u_i goes to the packed input
// of the down projection.
template <typename T>
struct EpiSwiGLU {
  int M, F;
  T* a;  // packed [rows][F]
  __device__ void operator()(int nt, int mt, const f32x16& acc, int lane) const {
    const int m = mt * 32 + (lane & 31);
    if (m >= M) return;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int n0 = nt * 32 + 8 * q4 + 4 * (lane >> 5);
#pragma unroll
      for (int t = 0; t < 4; t += 2) {
        const float gt = acc[4 * q4 + t], up = acc[4 * q4 + t + 1];
        const float s = gt / (1.0f + expf(-gt));
        a[packed_off<T>(m, (n0 + t) >> 1, F)] = Mfma<T>::store_cvt(s * up);
      }
    }
  }
};

// LM head: planted bias, mask_id excluded, then per (vocab tile, row) the
// running (max, argmax, sum exp(l - max)) that the merge kernel combines.
// Ties keep the lowest vocabulary index.  Logits never leave registers unless
// a debug buffer is given.
struct EpiLMHead {
  int M;                  // head rows = batch * block_len
  int blk;                // block_len
  int gen_len, gen_off;   // row m -> bias index (m/blk)*gen_len + gen_off + m%blk
  const int* target;      // may be null
  const float* alpha;
  int mask_id, vocab;
  float* pmax;            // [n_tiles][M]
  float* psum;
  int* parg;
  float* dbg;             // [M][vocab] or null
  __device__ void operator()(int nt, int mt, const f32x16& acc, int lane) const {
    const int m = mt * 32 + (lane & 31);
    const bool valid = m < M;
    int tgt = -1;
    float al = 0.f;
    if (valid && target) {
      const int bi = (m / blk) * gen_len + gen_off + m % blk;
      tgt = target[bi];
      al = alpha[bi];
    }
    float v[16];
    float mx = -INFINITY;
    int am = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int voc = nt * 32 + acc_row(r, lane);
      float x = acc[r];
      if (voc == tgt) x += al;
      if (voc == mask_id) x = -INFINITY;
      v[r] = x;
      if (x > mx) { mx = x; am = voc; }
      if (valid && dbg) dbg[(size_t)m * vocab + voc] = x;
    }
    const float omx = __shfl_xor(mx, 32);
    const int oam = __shfl_xor(am, 32);
    if (omx > mx || (omx == mx && oam < am)) { mx = omx; am = oam; }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += expf(v[r] - mx);
    // fixed order: lower half-lane first
    const float os = __shfl_xor(s, 32);
    s = (lane < 32) ? s + os : os + s;
    if (valid && lane < 32) {
      pmax[(size_t)nt * M + m] = mx;
      psum[(size_t)nt * M + m] = s;
      parg[(size_t)nt * M + m] = am;
    }
  }
};

// ---------------------------------------------------------------------------
// kernel
// ---------------------------------------------------------------------------
struct GemmArgs {
  const Frag16* X;      // packed [m_tiles*32][K]
  const Frag16* W;      // packed [n_tiles*32][K]
  int KT;               // k fragments
  int n_tiles, m_tiles;
  int m_groups;         // ceil(m_tiles / MT)
  int splits;
  float* ws;            // splits * n_tiles * m_groups * MT * 1024 floats
  unsigned* counters;   // n_tiles * m_groups, zero on entry, zero on exit
};

// Workgroup id -> (n-tile, m-group, split) with the m-groups of one n-tile on
// the same XCD (workgroup i runs on XCD i % 8), so their shared weight tiles
// are fetched into one L2.
__device__ __forceinline__ int xcd_remap(int hw, int total) {
  const int per = total / 8, rem = total % 8, x = hw % 8, slot = hw / 8;
  if (hw >= per * 8) return hw;          // ragged tail keeps its id
  (void)rem;
  return x * per + slot;
}

template <typename T, int MT, class Epi>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs a, Epi epi) {
  constexpr int U = 4;  // k fragments in flight per wave per batch
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int total = gridDim.x;
  const int lin = xcd_remap(blockIdx.x, total);
  const int s = lin % a.splits;
  const int rest = lin / a.splits;
  const int mg = rest % a.m_groups;
  const int nt = rest / a.m_groups;
  const int mt0 = mg * MT;
  const int nmt = min(MT, a.m_tiles - mt0);

  const int k0 = (int)((long)a.KT * s / a.splits), k1 = (int)((long)a.KT * (s + 1) / a.splits);
  const int len = k1 - k0;
  const int a0 = k0 + len * wave / 4, a1 = k0 + len * (wave + 1) / 4;

  f32x16 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  const Frag16* wp = a.W + (size_t)nt * a.KT * 64 + lane;
  const Frag16* xp = a.X + (size_t)mt0 * a.KT * 64 + lane;
  int kt = a0;
  for (; kt + U <= a1; kt += U) {
    Frag16 wf[U], xf[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) wf[u] = __builtin_nontemporal_load(&wp[(size_t)(kt + u) * 64]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MT; ++i)
        if (i < nmt) xf[u][i] = xp[((size_t)i * a.KT + kt + u) * 64];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MT; ++i)
        if (i < nmt) acc[i] = Mfma<T>::mma(wf[u], xf[u][i], acc[i]);
  }
  for (; kt < a1; ++kt) {
    const Frag16 wf = __builtin_nontemporal_load(&wp[(size_t)kt * 64]);
#pragma unroll
    for (int i = 0; i < MT; ++i)
      if (i < nmt) acc[i] = Mfma<T>::mma(wf, xp[((size_t)i * a.KT + kt) * 64], acc[i]);
  }

  // waves 1..3 -> LDS; wave 0 adds them in order
  __shared__ float red[3][MT][16][64];
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave - 1][i][r][lane] = acc[i][r];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] += red[w][i][r][lane];
  }

  if (a.splits == 1) {
    if (wave == 0)
      for (int i = 0; i < nmt; ++i) epi(nt, mt0 + i, acc[i], lane);
    return;
  }

  const size_t tile_id = (size_t)nt * a.m_groups + mg;
  if (wave == 0) {
    float* dst = a.ws + ((size_t)s * a.n_tiles * a.m_groups + tile_id) * MT * 1024;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(i * 16 + r) * 64 + lane] = acc[i][r];
  }
  __threadfence();
  __syncthreads();
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    const unsigned t = atomicAdd(&a.counters[tile_id], 1u);
    s_last = (t == (unsigned)a.splits - 1);
    if (s_last) atomicExch(&a.counters[tile_id], 0u);
  }
  __syncthreads();
  if (!s_last || wave != 0) return;
  __threadfence();
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  for (int sp = 0; sp < a.splits; ++sp) {
    const float* src = a.ws + ((size_t)sp * a.n_tiles * a.m_groups + tile_id) * MT * 1024;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] += src[(i * 16 + r) * 64 + lane];
  }
  for (int i = 0; i < nmt; ++i) epi(nt, mt0 + i, acc[i], lane);
}

}  // namespace dllm
