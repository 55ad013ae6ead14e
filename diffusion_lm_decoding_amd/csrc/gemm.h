// Projection GEMM  Y[m][n] = sum_k X[m][k] W[n][k]  on 16x16 MFMA with fused
// epilogues; X and W are packed (mfma.h).  No workgroup ever waits for or
// reads another's partial sums, so results are bitwise reproducible and no
// device-scope fence is needed.
//
//  * gemm_skinny_kernel (M <= 64, the block step): a workgroup of NW waves owns
//    NT 16-column n-tiles and every row; its waves split K, stream their
//    weight fragments straight from HBM once, reuse the activation fragments
//    across the NT tiles, and add their partial accumulators through LDS in
//    wave order.  16-wide tiles give N/16 workgroups (256 for N = 4096).
//  * gemm_big_kernel (large M: cache passes, big batches): a workgroup owns a
//    tile of up to 192x192 outputs; fragments of both operands are copied
//    into a multi-stage LDS ring by the DMA path and shared by the waves.
#pragma once
#include <type_traits>

#include "mfma.h"

namespace dllm {

struct RowGeom {
  int M;          // rows of this forward = batch * nr
  int nr;         // rows per sequence
  int row_start;  // canvas position of each sequence's first row
};

// N consecutive 16-bit elements (N = 2 or 4, p aligned to 2N bytes) as one
// store; fp32 elements one by one.  Rounding as Elem<T>::cvt.
template <typename T, int N>
__device__ __forceinline__ void store_run(T* p, const float (&v)[N]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) w[i] = Elem<T>::bits(v[2 * i]) | (Elem<T>::bits(v[2 * i + 1]) << 16);
    if constexpr (N == 4) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    else *reinterpret_cast<uint32_t*>(p) = w[0];
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) p[i] = Elem<T>::cvt(v[i]);
  }
}

// ---------------------------------------------------------------------------
// epilogues: called once per (16-col n-tile, 16-row m-tile); lane l holds
// rows n = 16*nt + 4*(l/16) + r (r = 0..3) of token m = 16*mt + l%16.
// ---------------------------------------------------------------------------

// Column of canvas position pos in a V^T cache row.  16-bit caches store the
// keys of each 32-key tile in the order the attention P V product consumes
// them: slot 8 g + e (g = 2 c + h) holds key 16 c + 4 h + e for e < 4 and
// key 16 c + 4 h + e + 4 for e >= 4, so each (key half c, lane half h)
// fragment is 16 contiguous bytes.  fp32 caches keep natural order.
template <typename T>
__host__ __device__ __forceinline__ int vt_col(int pos) {
  if constexpr (sizeof(T) == 2) {
    const int k = pos & 31, c = k >> 4, rem = k & 15;
    const int h = (rem >> 2) & 1, e = (rem & 3) + ((rem >> 3) << 2);
    return (pos & ~31) + ((2 * c + h) << 3) + e;
  } else {
    return pos;
  }
}

// Q/K/V projection: rotary embedding on q and k (the packed weight rows of
// each head are ordered so that dims (j, j + dh/2) are adjacent output
// columns 2j, 2j+1), q to a row buffer, k and v into the layer's cache rows.
template <typename T>
struct EpiQKV {
  RowGeom g;
  int d, dh, H, seq_pad;
  T* q;             // [rows][d], per-head rotary pair order
  T* kc;            // [batch][H][seq_pad][dh], rotary pair order
  T* vt;            // [batch][H][dh][seq_pad], key order vt_col
  // [seq][dh/4][4]: cos, sin of rotary pair 2g, then of pair 2g+1, so a
  // lane's two pairs (columns 4g .. 4g+3) take one 16-byte load and the 16
  // rows of a tile two cache lines per position run (measured on MI355X at
  // 512 rows against separate [seq][dh/2] cos and sin tables, four loads:
  // 62.7 -> 58 us with 192x128 tiles, 90-91 -> 79-81 us with 192x256)
  const float* rot;
  __device__ void operator()(int nt, int mt, const f32x4& acc, int lane) const {
    const int m = mt * 16 + (lane & 15);
    if (m >= g.M) return;
    const int b = m / g.nr;
    const int pos = g.row_start + m % g.nr;
    const int n0 = nt * 16 + 4 * (lane >> 4);
    float v[4] = {acc[0], acc[1], acc[2], acc[3]};
    const int region = n0 / d, nn = n0 % d, h = nn / dh, p = nn % dh;
    if (region < 2) {
      // p % 4 == 0: pairs p/2 and p/2 + 1 are group p/4
      const f32x4 r = *reinterpret_cast<const f32x4*>(rot + ((size_t)pos * (dh / 4) + (p >> 2)) * 4);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float c = r[2 * t], s = r[2 * t + 1];
        const float e = v[2 * t], o = v[2 * t + 1];
        v[2 * t] = e * c - o * s;
        v[2 * t + 1] = o * c + e * s;
      }
      T* dst = region == 0 ? q + (size_t)m * d + nn : kc + (((size_t)b * H + h) * seq_pad + pos) * dh + p;
      store_run<T, 4>(dst, v);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) vt[(((size_t)b * H + h) * dh + p + t) * seq_pad + vt_col<T>(pos)] = Elem<T>::cvt(v[t]);
    }
  }
};

// Output of a residual update that feeds an RMSNorm: the next projection's
// packed input xg = x * gain (the per-row 1/rms factor is applied by the
// consumer after its matmul, see GemmArgs::ssq), plus per (16-column tile,
// row) partial sums of x^2 in a fixed order.  rows map the producer's rows to
// the consumer's: row m -> (m / nr) * blk + (m % nr - off) when that lies in
// [0, blk), else skipped.
template <typename T>
struct NormOut {
  T* xg;             // packed [rows][d], or null (disabled)
  float* ssq;        // [d/16][rows_out]
  const float* gain;
  int rows_out;      // leading dimension of ssq
  int nr, off, blk;  // row map
  __device__ void put(int nt, int m, const float v[4], int lane, int d) const {
    const int i = m % nr - off;
    const bool keep = xg != nullptr && i >= 0 && i < blk;
    const int mo = (m / nr) * blk + i;
    const int n0 = nt * 16 + 4 * (lane >> 4);
    float s = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (!keep) return;
    if constexpr (sizeof(T) == 2) {
      // 16-bit packing keeps k = n0..n0+3 (n0 % 4 == 0) in adjacent slots
      const float w[4] = {v[0] * gain[n0], v[1] * gain[n0 + 1], v[2] * gain[n0 + 2], v[3] * gain[n0 + 3]};
      store_run<T, 4>(xg + packed_off<T>(mo, n0, d), w);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) xg[packed_off<T>(mo, n0 + t, d)] = Elem<T>::cvt(v[t] * gain[n0 + t]);
    }
    if (lane < 16) ssq[(size_t)nt * rows_out + mo] = s;
  }
};

// Residual update x[m][n] += y (fp32 residual stream), optionally emitting the
// normalised input of the next projection (nxt) and of the LM head (head).
template <typename T>
struct EpiResidual {
  int M, ld;
  float* x;
  NormOut<T> nxt, head;
  __device__ void operator()(int nt, int mt, const f32x4& acc, int lane) const {
    const int m = mt * 16 + (lane & 15);
    const bool valid = m < M;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
      float4* p = reinterpret_cast<float4*>(x + (size_t)m * ld + nt * 16 + 4 * (lane >> 4));
      float4 r = *p;
      r.x += acc[0];
      r.y += acc[1];
      r.z += acc[2];
      r.w += acc[3];
      *p = r;
      v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    }
    // the partial-sum shuffles involve every lane; invalid rows store nothing
    const int mm = valid ? m : 0;
    if (nxt.xg) {
      NormOut<T> o = nxt;
      if (!valid) o.xg = nullptr;
      o.put(nt, mm, v, lane, ld);
    }
    if (head.xg) {
      NormOut<T> o = head;
      if (!valid) o.xg = nullptr;
      o.put(nt, mm, v, lane, ld);
    }
  }
};

// SiLU g / (1 + e^-g) from the hardware's 2^x and reciprocal (each within a
// few ulp of fp32; the product is rounded to 16 bits after): about 2 us less
// per large-M gate/up launch on MI355X than an IEEE division of expf.  Very
// negative g: 2^x overflows to inf, its reciprocal is 0, silu -> -0.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}

// SwiGLU: packed rows 2i / 2i+1 are gate row i / up row i, so each lane holds
// (g_i, u_i, g_{i+1}, u_{i+1}); a_i = silu(g_i) * u_i goes to the packed input
// of the down projection.
template <typename T>
struct EpiSwiGLU {
  int M, F;
  T* a;  // packed [rows][F]
  __device__ void operator()(int nt, int mt, const f32x4& acc, int lane) const {
    const int m = mt * 16 + (lane & 15);
    if (m >= M) return;
    const int i0 = (nt * 16 + 4 * (lane >> 4)) >> 1;
    float h[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float gt = acc[2 * t], up = acc[2 * t + 1];
      h[t] = silu(gt) * up;
    }
    if constexpr (sizeof(T) == 2) {
      store_run<T, 2>(a + packed_off<T>(m, i0, F), h);  // i0 even: adjacent slots
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) a[packed_off<T>(m, i0 + t, F)] = h[t];
    }
  }
};

// LM head: planted bias, mask_id excluded, then per (16-entry vocab tile,
// row) the (max, argmax, sum exp(l - max)) that the merge kernel combines.
// Ties keep the lowest vocabulary index.  Logits never leave registers unless
// a debug buffer is given.  With group > 1 (the skinny kernel, group = its
// n-tiles per workgroup) a workgroup first combines its group consecutive
// tiles in LDS, in tile order, and stores one partial per (row, group): the
// partial arrays are [M][n_tiles / group].
struct EpiLMHead {
  static constexpr bool kGroupMerge = true;
  int M;                  // head rows = batch * block_len
  int blk;                // block_len
  int gen_len, gen_off;   // row m -> bias index (m/blk)*gen_len + gen_off + m%blk
  const int* target;      // may be null
  const float* alpha;
  int mask_id, vocab;
  int n_tiles;            // vocab / 16
  float* pmax;            // [M][n_tiles / group]: each row's partials contiguous for the merge
  float* psum;
  int* parg;
  float* dbg;             // [M][vocab] (block rows) or null
  // optional compaction: partial row m is block row rowmap[m], rows >= *count
  // are not written
  const int* rowmap;
  const int* count;
  int group = 1;
  __device__ bool row_valid(int m) const { return m < (count ? *count : M); }
  // (max, sum exp(l - max), argmax) of tile nt for row mt * 16 + lane % 16,
  // complete in lanes 0..15
  __device__ void reduce(int nt, int mt, const f32x4& acc, int lane, float& mx, float& s, int& am) const {
    const int m = mt * 16 + (lane & 15);
    const bool valid = row_valid(m);
    const int br = rowmap ? rowmap[valid ? m : 0] : m;   // block row
    int tgt = -1;
    float al = 0.f;
    if (valid && target) {
      const int bi = (br / blk) * gen_len + gen_off + br % blk;
      tgt = target[bi];
      al = alpha[bi];
    }
    float v[4];
    mx = -INFINITY;
    am = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int voc = nt * 16 + acc16_row(r, lane);
      float x = acc[r];
      if (voc == tgt) x += al;
      if (voc == mask_id) x = -INFINITY;
      v[r] = x;
      if (x > mx) { mx = x; am = voc; }
      if (valid && dbg) dbg[(size_t)br * vocab + voc] = x;
    }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float omx = __shfl_xor(mx, o);
      const int oam = __shfl_xor(am, o);
      if (omx > mx || (omx == mx && oam < am)) { mx = omx; am = oam; }
    }
    s = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) s += expf(v[r] - mx);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
  }
  __device__ void store(int part, int m, float mx, float s, int am) const {
    const size_t n_parts = n_tiles / group;
    pmax[(size_t)m * n_parts + part] = mx;
    psum[(size_t)m * n_parts + part] = s;
    parg[(size_t)m * n_parts + part] = am;
  }
  __device__ void operator()(int nt, int mt, const f32x4& acc, int lane) const {
    float mx, s;
    int am;
    reduce(nt, mt, acc, lane, mx, s, am);
    const int m = mt * 16 + (lane & 15);
    if (row_valid(m) && lane < 16) store(nt, m, mx, s, am);
  }
};

template <class E, class = void> struct GroupMerge : std::false_type {};
template <class E> struct GroupMerge<E, std::void_t<decltype(E::kGroupMerge)>> : std::true_type {};

// ---------------------------------------------------------------------------
struct GemmArgs {
  const Frag16* X;      // packed [m_tiles*16][K]
  const Frag16* W;      // packed [n_tiles*16][K]
  int KT;               // K / KF
  int n_tiles, m_tiles; // 16-row tiles
  int m_groups;
  // RMSNorm of the input applied after the matmul: when ssq is set, X holds
  // x * gain and row m of the result is scaled by
  // 1 / sqrt(sum_t ssq[t][m] / K + eps), t over ssq_tiles partial sums.
  const float* ssq;
  int ssq_tiles, ssq_ld;
  float inv_k, eps;
  // gemm_big_kernel: per-row 1/rms computed beforehand by rstd_kernel
  // (required there when ssq is set)
  const float* rstd;
  // gemm_big_kernel split over K: with k_splits > 1, workgroup group s of
  // the grid (s slowest) sums k-stages [nst*s/k_splits, nst*(s+1)/k_splits)
  // and stores its raw 16x16 tiles to part[s][m_tile][n_tile][lane][4]
  // (fp32); gemm_split_reduce_kernel adds them in split order and runs the
  // epilogue.
  int k_splits;
  float* part;
  // gemm_big_kernel: when set, only rows < *m_count are needed; workgroups
  // whose rows all lie beyond it return at once
  const int* m_count;
};

// Pipelined skinny loop over a rotated K order (see gemm_skinny_kernel): on
// for the Q/K/V projection, whose 32-row LLaDA-8B launch measured 20.5 ->
// 19.7 us with it on MI355X (the same as with its activation loads removed);
// O and down measured no gain.  Rotation changes the order in which each
// wave accumulates its K range, not the result's reproducibility.
template <class Epi> constexpr bool kRotateK = false;
template <typename T> constexpr bool kRotateK<EpiQKV<T>> = true;

// Workgroup i runs on XCD i % 8; map consecutive logical ids to one XCD so the
// workgroups that share weight tiles share an L2.
__device__ __forceinline__ int xcd_remap(int hw, int total) {
  const int per = total / 8;
  if (hw >= per * 8) return hw;
  return (hw % 8) * per + hw / 8;
}

// PIPE: two register sets, the next batch in flight during the current MFMAs
// (for grids of at most one workgroup per CU); otherwise one set.
template <typename T, int MT, int NT, int NW, class Epi, int U = 4, bool PIPE = true>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_kernel(GemmArgs a, Epi epi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int mg = lin % a.m_groups, ng = lin / a.m_groups;
  const int nt0 = ng * NT, mt0 = mg * MT;
  const int nmt = min(MT, a.m_tiles - mt0);
  const int k0 = a.KT * wave / NW, k1 = a.KT * (wave + 1) / NW;

  f32x4 acc[NT][MT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's share of the input rows' sums of squares: tiles t with
  // t % (4 NW) == 4 wave + lane/16, loaded now so the latency hides behind
  // the weight stream, combined after the main loop
  // Loads are unconditional (indices clamped into range, out-of-range values
  // masked at use) so the loop bodies stay branch-free and the compiler can
  // wait on individual loads instead of draining all of them before each MFMA.
  constexpr int QS = 8;  // covers 32*NW tiles (K <= 4096 at NW = 8) without a second pass
  float ssv[MT][QS];
  const int t_first = 4 * wave + (lane >> 4);
  if (a.ssq) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = min((mt0 + i) * 16 + (lane & 15), a.ssq_ld - 1);
#pragma unroll
      for (int q = 0; q < QS; ++q)
        ssv[i][q] = a.ssq[(size_t)min(t_first + q * 4 * NW, a.ssq_tiles - 1) * a.ssq_ld + m];
    }
  }

  const Frag16* wp = a.W + (size_t)nt0 * a.KT * 64 + lane;
  const Frag16* xq[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) xq[i] = a.X + (size_t)min(mt0 + i, a.m_tiles - 1) * a.KT * 64 + lane;

  // batches of U fragments in two register sets: batch b+1 is requested
  // before batch b feeds the MFMAs
  Frag16 wa[U][NT], xa[U][MT], wb[U][NT], xb[U][MT];
  auto load = [&](Frag16 (&wf)[U][NT], Frag16 (&xf)[U][MT], int k) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j) wf[u][j] = __builtin_nontemporal_load(&wp[((size_t)j * a.KT + k + u) * 64]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MT; ++i) xf[u][i] = xq[i][(size_t)(k + u) * 64];
  };
  auto compute = [&](const Frag16 (&wf)[U][NT], const Frag16 (&xf)[U][MT]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[j][i] = Mfma16<T>::mma(wf[u][j], xf[u][i], acc[j][i]);
  };
  const int nbat = (k1 - k0) / U;
  int kt = k0;
  if constexpr (PIPE) {
    // batch b of the wave's K range is batch (b + rot) % nbat: with kRotateK
    // every workgroup starts at a different point of the range
    const int rot = kRotateK<Epi> && nbat > 1 ? lin % nbat : 0;
    auto kb = [&](int b) {
      const int bb = b + rot;
      return k0 + (bb >= nbat ? bb - nbat : bb) * U;
    };
    if (nbat > 0) load(wa, xa, kb(0));
    for (int b = 0; b < nbat; b += 2) {
      if (b + 1 < nbat) load(wb, xb, kb(b + 1));
      compute(wa, xa);
      if (b + 1 < nbat) {
        if (b + 2 < nbat) load(wa, xa, kb(b + 2));
        compute(wb, xb);
      }
    }
  } else {
    // one register set (fewer VGPRs, several workgroups resident per CU); the
    // activation loads are skipped for m-tiles past the last one (measured
    // faster here than the clamped form)
    const Frag16* xp = a.X + (size_t)mt0 * a.KT * 64 + lane;
    for (int b = 0; b < nbat; ++b, kt += U) {
      Frag16 wf[U][NT], xf[U][MT];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NT; ++j) wf[u][j] = __builtin_nontemporal_load(&wp[((size_t)j * a.KT + kt + u) * 64]);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < MT; ++i)
          if (i < nmt) xf[u][i] = xp[((size_t)i * a.KT + kt + u) * 64];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int i = 0; i < MT; ++i)
            if (i < nmt) acc[j][i] = Mfma16<T>::mma(wf[u][j], xf[u][i], acc[j][i]);
    }
  }
  for (kt = k0 + nbat * U; kt < k1; ++kt) {
    Frag16 wf[NT], xf[MT];
#pragma unroll
    for (int j = 0; j < NT; ++j) wf[j] = __builtin_nontemporal_load(&wp[((size_t)j * a.KT + kt) * 64]);
#pragma unroll
    for (int i = 0; i < MT; ++i) xf[i] = xq[i][(size_t)kt * 64];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[j][i] = Mfma16<T>::mma(wf[j], xf[i], acc[j][i]);
  }

  // per-wave sums of squares (tiles past the prefetched ones, for K > 4096,
  // are read here), then the four lane groups of each row
  float ssq_part[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    float s = 0.f;
    const int m = (mt0 + i) * 16 + (lane & 15);
    const bool row_ok = a.ssq && i < nmt && m < a.ssq_ld;
#pragma unroll
    for (int q = 0; q < QS; ++q) s += (row_ok && t_first + q * 4 * NW < a.ssq_tiles) ? ssv[i][q] : 0.f;
    if (row_ok)
      for (int t = t_first + QS * 4 * NW; t < a.ssq_tiles; t += 4 * NW) s += a.ssq[(size_t)t * a.ssq_ld + m];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    ssq_part[i] = s;
  }
  __shared__ float ssq_red[NW][MT][16];
  if (a.ssq && lane < 16) {
#pragma unroll
    for (int i = 0; i < MT; ++i) ssq_red[wave][i][lane] = ssq_part[i];
  }
  // every wave's partial accumulators to LDS; output tile t = j*MT + i is then
  // summed in wave order and finished by wave t % NW, so the epilogues of the
  // tiles run in parallel
  constexpr int TILES = NT * MT;
  __shared__ float red[NW][TILES * 4][64];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][(j * MT + i) * 4 + r][lane] = acc[j][i][r];
  __syncthreads();
  // LM head with group = NT: the tile reductions meet in LDS and one wave per
  // m-tile combines the workgroup's NT tiles in tile order
  constexpr bool kGroup = GroupMerge<Epi>::value;
  __shared__ float g_mx[kGroup ? MT : 1][kGroup ? NT : 1][16], g_s[kGroup ? MT : 1][kGroup ? NT : 1][16];
  __shared__ int g_am[kGroup ? MT : 1][kGroup ? NT : 1][16];
  bool grouped = false;
  if constexpr (kGroup) grouped = epi.group == NT && NT > 1;
  for (int t = wave; t < TILES; t += NW) {
    const int j = t / MT, i = t % MT;
    if (i >= nmt) continue;
    f32x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = red[0][t * 4 + r][lane];
    for (int w = 1; w < NW; ++w)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] += red[w][t * 4 + r][lane];
    if (a.ssq) {
      float s2 = 0.f;
      for (int w = 0; w < NW; ++w) s2 += ssq_red[w][i][lane & 15];
      v *= 1.0f / sqrtf(s2 * a.inv_k + a.eps);
    }
    if constexpr (kGroup) {
      if (grouped) {
        float mx, s;
        int am;
        epi.reduce(nt0 + j, mt0 + i, v, lane, mx, s, am);
        if (lane < 16) {
          g_mx[i][j][lane] = mx;
          g_s[i][j][lane] = s;
          g_am[i][j][lane] = am;
        }
        continue;
      }
    }
    epi(nt0 + j, mt0 + i, v, lane);
  }
  if constexpr (kGroup) {
    if (grouped) {
      __syncthreads();
      const int m = (mt0 + wave) * 16 + lane;
      if (wave < nmt && lane < 16 && epi.row_valid(m)) {
        float mx = -INFINITY;
        int am = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const float x = g_mx[wave][j][lane];
          const int ax = g_am[wave][j][lane];
          if (x > mx || (x == mx && ax < am)) { mx = x; am = ax; }
        }
        float s = 0.f;
        if (mx != -INFINITY) {
#pragma unroll
          for (int j = 0; j < NT; ++j) s += g_s[wave][j][lane] * expf(g_mx[wave][j][lane] - mx);
        }
        epi.store(nt0 / NT, m, mx, s, am);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large-M projection (cache passes, big batches).  A workgroup of WN x WM waves
// owns NTW x MTW 16x16 output tiles.  Operand fragments are copied straight
// from HBM/L2 into LDS by the DMA path (global_load_lds_dwordx4: 64 lanes x
// 16 B = one packed fragment per wave instruction, no VGPR staging) through a
// ring of S stages of KS k-fragments each; S-1 stages are in flight while the
// MFMAs consume the oldest.  Waits are explicit: vmcnt for this wave's own
// copies, then s_barrier so every wave's copies of the stage have landed;
// lgkmcnt(0) before the barrier that hands a stage back to the copier.
// Out-of-range tiles are clamped to the last valid one (valid memory; their
// results are discarded by the epilogue guards).
// ---------------------------------------------------------------------------
// rstd[m] = 1 / sqrt(sum_t ssq[t][m] / K + eps), one wave per row; the 64
// lanes take tiles t = lane, lane + 64, ... and add in a fixed tree.
__global__ __launch_bounds__(256) void rstd_kernel(const float* ssq, int tiles, int ld, float inv_k, float eps,
                                                   float* rstd) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= ld) return;
  float s = 0.f;
  for (int t = lane; t < tiles; t += 64) s += ssq[(size_t)t * ld + m];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) rstd[m] = 1.0f / sqrtf(s * inv_k + eps);
}

// f(integral_constant<int, i>) for i = B .. E-1, unrolled
template <int B, int E, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int V>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(V >= 0 && V < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | (15 << 8) | ((V >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

template <typename T, class Epi, int NTW, int MTW, int WN, int WM, int KS, int S>
__global__ __launch_bounds__(64 * WN * WM) void gemm_big_kernel(GemmArgs a, Epi epi) {
  constexpr int NWAVE = WN * WM;
  constexpr int F = KS * (NTW + MTW);     // fragments per stage
  // copies per wave per stage; when F is not a multiple of the waves, the
  // spare copy slots repeat the stage's last fragment (the same bytes into
  // the same LDS block), so every wave issues LW copies and waits alike
  constexpr int LW = (F + NWAVE - 1) / NWAVE;
  constexpr int TN = NTW / WN, TM = MTW / WM;  // wave tile in 16x16 tiles
  static_assert(NTW % WN == 0 && MTW % WM == 0, "wave grid must divide the tile");
  __shared__ Frag16 lds[S][F][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m_wg = (a.m_tiles + MTW - 1) / MTW;
  const int lin_all = xcd_remap(blockIdx.x, gridDim.x);
  const int k_splits = a.k_splits > 1 ? a.k_splits : 1;
  const int per_split = gridDim.x / k_splits;
  const int split = lin_all / per_split, lin = lin_all % per_split;
  const int wg_m = lin % m_wg, wg_n = lin / m_wg;   // m fastest: neighbours share the weight tile
  const int nt0 = wg_n * NTW, mt0 = wg_m * MTW;
  if (a.m_count && mt0 * 16 >= *a.m_count) return;
  const int wn = wave % WN, wm = wave / WN;
  const int nst_all = a.KT / KS;
  const int st_first = (int)((long)nst_all * split / k_splits);
  const int nst = (int)((long)nst_all * (split + 1) / k_splits) - st_first;

  // this wave's copies: fragment f = wave + q * NWAVE of each stage
  const Frag16* src[LW];
  int soff[LW];
#pragma unroll
  for (int q = 0; q < LW; ++q) {
    const int f = min(wave + q * NWAVE, F - 1);
    const bool isw = f < KS * NTW;
    const int ff = isw ? f : f - KS * NTW;
    const int tile = ff / KS, kk = ff % KS;
    const int t = isw ? min(nt0 + tile, a.n_tiles - 1) : min(mt0 + tile, a.m_tiles - 1);
    src[q] = (isw ? a.W : a.X) + ((size_t)t * a.KT + (size_t)st_first * KS + kk) * 64 + lane;
    soff[q] = f;
  }
  // stage st's copies; stages past the end copy the last stage again (valid
  // memory whose data is never used), so every iteration issues the same
  // number of copies and every wait count below is a constant
  auto issue = [&](int st, int buf) {
    const size_t s = (size_t)min(st, nst - 1) * KS * 64;
#pragma unroll
    for (int q = 0; q < LW; ++q)
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(src[q] + s),
                                       (__attribute__((address_space(3))) void*)&lds[buf][soff[q]][0], 16, 0, 0);
  };

  f32x4 acc[TN][TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one (stage, k-fragment) step computes from one register set while the
  // next step's fragments are read from LDS into the other
  auto read = [&](int buf, int kk, Frag16 (&wf)[TN], Frag16 (&xf)[TM]) {
#pragma unroll
    for (int j = 0; j < TN; ++j) wf[j] = lds[buf][(wn * TN + j) * KS + kk][lane];
#pragma unroll
    for (int i = 0; i < TM; ++i) xf[i] = lds[buf][KS * NTW + (wm * TM + i) * KS + kk][lane];
  };
  auto mma = [&](const Frag16 (&wf)[TN], const Frag16 (&xf)[TM]) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[j][i] = Mfma16<T>::mma(wf[j], xf[i], acc[j][i]);
  };
  // all S buffers in flight; stage st + S is copied into buffer st % S once
  // every wave has finished reading stage st.  The loop body covers S stages
  // so that every buffer index is a compile-time constant: with a run-time
  // index the compiler cannot tell the LDS reads from the copies in flight
  // and waits for all of them (vmcnt(0)) before each stage's first read.
  // With 3 or more stages in the ring each stage's copies are spread over the
  // MFMAs of its last k-fragment (measured on MI355X: 4.5-6% faster for the
  // 192x192, 192x128 and 256x128 tiles; with 2 stages the burst after the
  // barrier measured as fast or 2.5% faster)
  constexpr bool kSpreadCopies = S >= 3;
  static_for<0, S>([&](auto s_c) { issue(decltype(s_c)::value, decltype(s_c)::value); });
  wait_vmcnt<(S - 1) * LW>();
  __builtin_amdgcn_s_barrier();
  // two register sets; step t = st*KS + kk computes from set t%2 (S*KS is
  // even for every configuration, so a loop body starts on set 0)
  static_assert(KS == 1 || KS == 2, "k-fragments per stage");
  static_assert((S * KS) % 2 == 0, "register sets alternate across the loop body");
  Frag16 fw[2][TN], fx[2][TM];
  read(0, 0, fw[0], fx[0]);
  auto stage = [&](int st, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    static_for<0, KS>([&](auto kk_c) {
      constexpr int kk = decltype(kk_c)::value;
      constexpr int cur = (buf * KS + kk) % 2, nxt = 1 - cur;
      if constexpr (kk + 1 < KS) {
        read(buf, kk + 1, fw[nxt], fx[nxt]);
      } else {
        // stage st + 1 landed (S - 2 later stages in flight) and every wave
        // has read stage st: its buffer takes stage st + S
        wait_vmcnt<(S - 2) * LW>();
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
        if constexpr (!kSpreadCopies) issue(st + S, buf);
        read((buf + 1) % S, 0, fw[nxt], fx[nxt]);
        if constexpr (kSpreadCopies) {
          // the stage's copies spread over this k-fragment's MFMAs, one
          // before each group of G, so the two waves of a SIMD do not both
          // stop issuing MFMAs for the whole burst after the barrier (same
          // copies, same order, same wait counts)
          constexpr int NM = TN * TM, G = (NM + LW - 1) / LW;
          const size_t so = (size_t)min(st + S, nst - 1) * KS * 64;
          static_for<0, LW>([&](auto q_c) {
            constexpr int q = decltype(q_c)::value;
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(src[q] + so),
                                             (__attribute__((address_space(3))) void*)&lds[buf][soff[q]][0], 16, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            static_for<q * G, ((q + 1) * G < NM ? (q + 1) * G : NM)>([&](auto t_c) {
              constexpr int t = decltype(t_c)::value;
              acc[t / TM][t % TM] = Mfma16<T>::mma(fw[cur][t / TM], fx[cur][t % TM], acc[t / TM][t % TM]);
            });
          });
          static_for<(LW * G < NM ? LW * G : NM), NM>([&](auto t_c) {
            constexpr int t = decltype(t_c)::value;
            acc[t / TM][t % TM] = Mfma16<T>::mma(fw[cur][t / TM], fx[cur][t % TM], acc[t / TM][t % TM]);
          });
          __builtin_amdgcn_sched_barrier(0);
          return;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      mma(fw[cur], fx[cur]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  int st = 0;
  for (; st + S <= nst; st += S)
    static_for<0, S>([&](auto i_c) { stage(st + decltype(i_c)::value, i_c); });
  static_for<0, S>([&](auto i_c) {
    if (st + decltype(i_c)::value < nst) stage(st + decltype(i_c)::value, i_c);
  });
  wait_vmcnt<0>();   // the copies past the end
  if (k_splits > 1) {
    // raw partial tiles; the reduce kernel scales by 1/rms and runs the epilogue
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int nt = nt0 + wn * TN + j;
      if (nt >= a.n_tiles) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int mt = mt0 + wm * TM + i;
        if (mt < a.m_tiles)
          *reinterpret_cast<f32x4*>(a.part + ((((size_t)split * a.m_tiles + mt) * a.n_tiles + nt) * 64 + lane) * 4) =
              acc[j][i];
      }
    }
    return;
  }
  if (a.ssq) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const float rs = a.rstd[min((mt0 + wm * TM + i) * 16 + (lane & 15), a.ssq_ld - 1)];
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[j][i] *= rs;
    }
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int nt = nt0 + wn * TN + j;
    if (nt >= a.n_tiles) continue;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int mt = mt0 + wm * TM + i;
      if (mt < a.m_tiles) epi(nt, mt, acc[j][i], lane);
    }
  }
}

// Second half of a K-split gemm_big_kernel launch: one wave per 16x16 output
// tile adds the KS partial tiles in split order (so results are run-to-run
// identical), applies the row's 1/rms and runs the epilogue exactly once.
// KS is a compile-time constant, so all KS partial loads are issued before the
// first is used (with a run-time count the reduce took 1.5-1.6x as long on
// MI355X: 9.3 -> 6.0 us for two splits of 2M outputs, 15.7 -> 9.7 us for
// four).  Grid: ceil(m_tiles * n_tiles / 4) workgroups of 4 waves.
template <int KS, class Epi>
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(GemmArgs a, Epi epi) {
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= a.m_tiles * a.n_tiles) return;
  const int mt = tile / a.n_tiles, nt = tile % a.n_tiles;
  const size_t stride = (size_t)a.m_tiles * a.n_tiles * 256;
  const float* p = a.part + ((size_t)tile * 64 + lane) * 4;
  f32x4 parts[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) parts[s] = *reinterpret_cast<const f32x4*>(p + s * stride);
  f32x4 v = parts[0];
#pragma unroll
  for (int s = 1; s < KS; ++s) v += parts[s];
  if (a.ssq) v *= a.rstd[min(mt * 16 + (lane & 15), a.ssq_ld - 1)];
  epi(nt, mt, v, lane);
}

}  // namespace dllm
