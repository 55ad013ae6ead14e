// Row-wise and per-sequence kernels around the projections: token embedding,
// RMSNorm into the packed MFMA layout, the LM-head (max, sum, argmax) merge,
// the select/commit step, and weight packing.
#pragma once
#include "gemm.h"

namespace dllm {

// ---- block reductions in a fixed order ------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += sh[i];
  __syncthreads();
  return t;
}

// ---- embedding: x[m] = E[token at (sequence, position) of row m] ----------
// x[m] = E[token of row m] (fp32 residual stream), plus the first layer's
// normalised-input pieces: packed x * gain and per-16-column sums of x^2
// (ssq [d/16][M]).  Token ids outside [0, vocab) are clamped (the table is
// never over-read).
template <typename Tin, typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int* tokens, int seq_len, RowGeom g,
                                                    const Tin* emb, int d, int vocab, float* x,
                                                    const float* gain, T* xg, float* ssq, int* err_reset) {
  const int m = blockIdx.x;
  // a forward that ends in the LM head starts the step's error flags at zero
  if (err_reset && m == 0 && threadIdx.x < 2) err_reset[threadIdx.x] = 0;
  const int b = m / g.nr, pos = g.row_start + m % g.nr;
  const int tok = min(max(tokens[(size_t)b * seq_len + pos], 0), vocab - 1);
  const Tin* e = emb + (size_t)tok * d;
  if constexpr (sizeof(Tin) == 2 && sizeof(T) == 2) {
    // 16 consecutive columns per thread with 16-byte accesses: the packed
    // input holds columns 8j .. 8j+7 of a row in one 16-byte slot group
    for (int t = threadIdx.x; t < d / 16; t += 256) {
      Tin ev[16];
      *reinterpret_cast<uint4*>(ev) = reinterpret_cast<const uint4*>(e + t * 16)[0];
      *reinterpret_cast<uint4*>(ev + 8) = reinterpret_cast<const uint4*>(e + t * 16)[1];
      float v[16], gv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<float4*>(gv + 4 * q) = reinterpret_cast<const float4*>(gain + t * 16)[q];
      float s = 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        v[u] = Elem<Tin>::load(ev + u);
        s += v[u] * v[u];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        reinterpret_cast<float4*>(x + (size_t)m * d + t * 16)[q] = float4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        T o[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) o[u] = Elem<T>::cvt(v[8 * h + u] * gv[8 * h + u]);
        *reinterpret_cast<uint4*>(xg + packed_off<T>(m, t * 16 + 8 * h, d)) = *reinterpret_cast<const uint4*>(o);
      }
      ssq[(size_t)t * g.M + m] = s;
    }
  } else {
    for (int t = threadIdx.x; t < d / 16; t += 256) {
      float s = 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int k = t * 16 + u;
        const float v = Elem<Tin>::load(e + k);
        x[(size_t)m * d + k] = v;
        xg[packed_off<T>(m, k, d)] = Elem<T>::cvt(v * gain[k]);
        s += v * v;
      }
      ssq[(size_t)t * g.M + m] = s;
    }
  }
}

// ---- LM-head merge: per row, combine the vocabulary partials --------------
// max and argmax (lowest index among equal maxima), then
// S = sum_t s_t exp(m_t - max); confidence = 1 / S.  Partials are [M][n_tiles]
// (n_tiles: partials per row, each covering consecutive vocabulary tiles);
// one workgroup of kMergeThreads per row.  Each thread keeps its first
// kMergePer tiles in registers (every load issued before the first use), so
// the second pass re-reads memory only for vocabularies beyond
// kMergeThreads * kMergePer tiles.  Reduction orders are fixed.
constexpr int kMergeThreads = 1024, kMergePer = 8;

__device__ __forceinline__ void argmax_take(float& mx, int& am, float v, int a) {
  if (v > mx || (v == mx && a < am)) { mx = v; am = a; }
}

// rowmap/count (optional, see head_rows_kernel): partial row m belongs to block
// row rowmap[m]; rows m >= count are skipped.
__global__ __launch_bounds__(kMergeThreads) void lm_merge_kernel(const float* pmax, const float* psum,
                                                                 const int* parg, int n_tiles, int M,
                                                                 float* conf, int* tok, int* err,
                                                                 const int* rowmap, const int* count) {
  (void)M;
  constexpr int NWV = kMergeThreads / 64;
  __shared__ float shm[NWV];
  __shared__ int sha[NWV];
  __shared__ float shs[NWV];
  const int m = blockIdx.x, t0 = threadIdx.x, lane = t0 & 63, wv = t0 >> 6;
  if (count && m >= *count) return;
  const int out_row = rowmap ? rowmap[m] : m;
  const float* rmax = pmax + (size_t)m * n_tiles;
  const float* rsum = psum + (size_t)m * n_tiles;
  const int* rarg = parg + (size_t)m * n_tiles;
  float vm[kMergePer], vs[kMergePer];
  int va[kMergePer];
#pragma unroll
  for (int j = 0; j < kMergePer; ++j) {
    const int t = min(t0 + j * kMergeThreads, n_tiles - 1);
    vm[j] = rmax[t];
    va[j] = rarg[t];
    vs[j] = rsum[t];
  }
  float mx = -INFINITY;
  int am = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < kMergePer; ++j)
    if (t0 + j * kMergeThreads < n_tiles) argmax_take(mx, am, vm[j], va[j]);
  for (int t = t0 + kMergePer * kMergeThreads; t < n_tiles; t += kMergeThreads) argmax_take(mx, am, rmax[t], rarg[t]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) argmax_take(mx, am, __shfl_xor(mx, o), __shfl_xor(am, o));
  if (lane == 0) { shm[wv] = mx; sha[wv] = am; }
  __syncthreads();
  float gm = shm[0];
  int ga = sha[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) argmax_take(gm, ga, shm[w], sha[w]);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kMergePer; ++j)
    if (t0 + j * kMergeThreads < n_tiles) s += vs[j] * expf(vm[j] - gm);
  for (int t = t0 + kMergePer * kMergeThreads; t < n_tiles; t += kMergeThreads) s += rsum[t] * expf(rmax[t] - gm);
  s = block_sum<kMergeThreads>(s, shs);
  if (t0 == 0) {
    conf[out_row] = 1.0f / s;
    tok[out_row] = ga;
    if (!(fabsf(gm) <= 3.0e38f) || !(s >= 1.0f && s <= 3.0e38f)) atomicOr(err, 1);
  }
}

// ---- LM head over the still-masked rows ------------------------------------
// With more block rows than one skinny launch covers, the LM head runs only on
// the rows whose canvas position still holds MASK (committed rows take no part
// in the selection).  rowmap[k] = the k-th such block row b * blk + i, in row
// order; count[0] = their number.  One workgroup of 1024 threads, each owning
// `per` consecutive rows (rows <= 32 * 1024).
__global__ __launch_bounds__(1024) void head_rows_kernel(const int* tokens, int seq_len, int start, int blk,
                                                         int rows, int mask_id, int* rowmap, int* count) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (rows + 1023) / 1024;
  unsigned flags = 0;
  int n = 0;
  for (int u = 0; u < per; ++u) {
    const int r = t * per + u;
    const bool msk = r < rows && tokens[(size_t)(r / blk) * seq_len + start + r % blk] == mask_id;
    flags |= (msk ? 1u : 0u) << u;
    n += msk ? 1 : 0;
  }
  part[t] = n;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {   // inclusive scan of the per-thread counts
    const int v = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int k = part[t] - n;
  for (int u = 0; u < per; ++u)
    if ((flags >> u) & 1u) rowmap[k++] = t * per + u;
  if (t == 1023) count[0] = part[1023];
}

// Packed row k of xc = packed row rowmap[k] of xh (in every k-fragment, row i
// of a 16-row tile is lanes i + 16 g, g < 4), and the row's sum-of-squares
// partials: ssq_c[t][k] = ssq[t][rowmap[k]] (both [tiles][ld]).
__global__ __launch_bounds__(256) void head_gather_kernel(const Frag16* xh, const float* ssq, int ld, int KT,
                                                          int ssq_tiles, const int* rowmap, const int* count,
                                                          Frag16* xc, float* ssq_c) {
  const int k = blockIdx.x;
  if (k >= *count) return;
  const int r = rowmap[k];
  const Frag16* src = xh + (size_t)(r >> 4) * KT * 64 + (r & 15);
  Frag16* dst = xc + (size_t)(k >> 4) * KT * 64 + (k & 15);
  for (int c = threadIdx.x; c < KT * 4; c += 256) {
    const size_t o = (size_t)(c >> 2) * 64 + 16 * (c & 3);
    dst[o] = src[o];
  }
  for (int t = threadIdx.x; t < ssq_tiles; t += 256) ssq_c[(size_t)t * ld + k] = ssq[(size_t)t * ld + r];
}

// ---- select / commit: one workgroup per sequence ---------------------------
struct SelectArgs {
  int* tokens;          // canvas [batch][seq_len]
  int seq_len, prompt_len, gen_len, blk, start;  // start = canvas position of the block
  int mask_id;
  const float* conf;    // [batch*blk]
  const int* tok;
  int rule;             // 0 threshold, 1 factor, 2 top-k
  float tau, factor;
  int k;
  int* step_ctr;        // [batch] steps taken by each sequence
  int block_idx;        // block of this step
  int* blk_id;          // [batch] block of each sequence's last step (-1: none)
  int* blk_steps;       // [batch] steps taken on that block
  int* commit_step;     // [batch][gen_len] or null
  int* ncommit;         // [batch]
  int* done;            // [batch]
  const int* err;       // nonzero: commit nothing
  // pinned host status block [ncommit[max_batch], done[max_batch], err]:
  // written with system-scope stores, read by the host after the stream
  // synchronises (no copy back)
  int* host_stat;
  int max_batch;
  float* dbg_conf;      // [batch*blk] or null
  int* dbg_tok;
};

__global__ __launch_bounds__(256) void select_commit_kernel(SelectArgs a) {
  __shared__ float sc[256];
  __shared__ int sm[256];
  __shared__ float eps_by_rank[256];
  __shared__ float red[4];
  __shared__ int nbudget;
  const int b = blockIdx.x, i = threadIdx.x;
  const bool in = i < a.blk;
  int* row = a.tokens + (size_t)b * a.seq_len + a.start;
  const bool masked = in && row[i] == a.mask_id;
  const float c = masked ? a.conf[b * a.blk + i] : -1.0f;
  const int y = masked ? a.tok[b * a.blk + i] : -1;
  sc[i] = c;
  sm[i] = masked ? 1 : 0;
  if (in && a.dbg_conf) { a.dbg_conf[b * a.blk + i] = c; a.dbg_tok[b * a.blk + i] = y; }
  __syncthreads();
  int rank = 0;
  for (int j = 0; j < a.blk; ++j)
    rank += (sm[j] && (sc[j] > c || (sc[j] == c && j < i))) ? 1 : 0;
  const int n_masked = (int)block_sum<256>(masked ? 1.f : 0.f, red);
  const int s_blk = a.blk_id[b] == a.block_idx ? a.blk_steps[b] : 0;  // steps already taken on this block
  bool sel = false;
  if (a.rule == 0) {
    sel = masked && c >= a.tau;
    const int any = (int)block_sum<256>(sel ? 1.f : 0.f, red);
    if (any == 0) sel = masked && rank == 0;
  } else if (a.rule == 1) {
    // largest n with (n+1)(1 - c_(n)) < f, c_(n) the n-th largest: the
    // candidate of rank n-1 tests n = rank+1
    const float lhs = __fmul_rn((float)(rank + 2), __fsub_rn(1.0f, c));
    const float cand = (masked && lhs < a.factor) ? (float)(rank + 1) : 0.f;
    // block max of cand (exact small integers)
    float v = cand;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if ((i & 63) == 0) red[i >> 6] = v;
    __syncthreads();
    int nstar = (int)fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    if (nstar == 0) nstar = 1;
    sel = masked && rank < nstar;
  } else if (a.rule == 3) {
    // eq. 9 in confidence order: the float32 running sum of eps_j in that
    // order, plus eps_n, must stay below 1; one thread walks the ranks
    if (masked) eps_by_rank[rank] = __fsub_rn(1.0f, c);
    __syncthreads();
    if (i == 0) {
      float sum = 0.f;
      int best = 0;
      for (int n = 1; n <= n_masked; ++n) {
        const float e = eps_by_rank[n - 1];
        sum = __fadd_rn(sum, e);
        if (__fadd_rn(sum, e) < 1.0f) best = n;
      }
      nbudget = best > 0 ? best : 1;
    }
    __syncthreads();
    sel = masked && rank < nbudget;
  } else if (a.rule == 4) {
    const int left = a.k - s_blk;
    const int n_keep = left > 0 ? n_masked / left : n_masked;
    sel = masked && rank < n_keep;
  } else {
    sel = masked && rank < a.k;
  }
  if (*a.err) sel = false;
  const int step = a.step_ctr[b];
  if (sel) {
    row[i] = y;
    if (a.commit_step) a.commit_step[(size_t)b * a.gen_len + (a.start - a.prompt_len) + i] = step;
  }
  const int cnt = (int)block_sum<256>(sel ? 1.f : 0.f, red);
  if (i == 0) {
    const int dn = (n_masked - cnt == 0) ? 1 : 0;
    a.ncommit[b] = cnt;
    a.done[b] = dn;
    __hip_atomic_store(a.host_stat + b, cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(a.host_stat + a.max_batch + b, dn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (b == 0) __hip_atomic_store(a.host_stat + 2 * a.max_batch, *a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (n_masked > 0 && !*a.err) {
      a.step_ctr[b] = step + 1;
      a.blk_id[b] = a.block_idx;
      a.blk_steps[b] = s_blk + 1;
    }
  }
}

// ---- staleness diagnostics ---------------------------------------------------
// out[b][i] = (conf, tok) of block row i of sequence b if that row is still
// MASK, else (-1, -1).
__global__ __launch_bounds__(256) void masked_copy_kernel(const int* tokens, int seq_len, int start, int blk,
                                                          int mask_id, const float* conf, const int* tok,
                                                          float* out_conf, int* out_tok) {
  const int b = blockIdx.x, i = threadIdx.x;
  if (i >= blk) return;
  const bool masked = tokens[(size_t)b * seq_len + start + i] == mask_id;
  if (out_conf) out_conf[b * blk + i] = masked ? conf[b * blk + i] : -1.0f;
  if (out_tok) out_tok[b * blk + i] = masked ? tok[b * blk + i] : -1;
}

// Cosine similarity, per (sequence, canvas position), between two copies of
// one layer's K (and V) over all heads: <a, b> / (|a| |b|), 1 when both are
// zero, 0 when one is.  One wave per position; K [batch][H][seq_pad][dh], V^T
// [batch][H][dh][seq_pad] in vt_col order.
template <typename T>
__global__ __launch_bounds__(256) void kv_cosine_kernel(const T* k_a, const T* v_a, const T* k_b, const T* v_b,
                                                        int H, int dh, int seq_pad, int N, int batch,
                                                        float* k_cos, float* v_cos) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= batch * N) return;
  const int b = item / N, pos = item % N;
  float kd = 0.f, ka = 0.f, kb = 0.f, vd = 0.f, va = 0.f, vb = 0.f;
  for (int e = lane; e < H * dh; e += 64) {
    const int h = e / dh, d = e % dh;
    const size_t ko = (((size_t)b * H + h) * seq_pad + pos) * dh + d;
    const size_t vo = (((size_t)b * H + h) * dh + d) * seq_pad + vt_col<T>(pos);
    const float x = Elem<T>::load(k_a + ko), y = Elem<T>::load(k_b + ko);
    const float u = Elem<T>::load(v_a + vo), w = Elem<T>::load(v_b + vo);
    kd += x * y; ka += x * x; kb += y * y;
    vd += u * w; va += u * u; vb += w * w;
  }
  kd = wave_sum(kd); ka = wave_sum(ka); kb = wave_sum(kb);
  vd = wave_sum(vd); va = wave_sum(va); vb = wave_sum(vb);
  if (lane != 0) return;
  auto cosv = [](float d, float a, float bb) {
    if (a == 0.f || bb == 0.f) return (a == 0.f && bb == 0.f) ? 1.f : 0.f;
    return d / sqrtf(a * bb);
  };
  if (k_cos) k_cos[item] = cosv(kd, ka, kb);
  if (v_cos) v_cos[item] = cosv(vd, va, vb);
}

// ---- canvas check: prompt holds no mask, answer region is all mask ---------
__global__ __launch_bounds__(256) void canvas_check_kernel(const int* tokens, int n, int seq_len,
                                                           int prompt_len, int mask_id, int vocab,
                                                           int* bad) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const int pos = t % seq_len, v = tokens[t];
  const bool ok = pos < prompt_len ? (v >= 0 && v < vocab && v != mask_id) : (v == mask_id);
  if (!ok) atomicOr(bad, 1);
}

// ---- weight packing -----------------------------------------------------------
// dst rows [row0, row0 + rows) of a packed [*, K] matrix from row-major sources.
//   mode 0: dst row r <- src row r
//   mode 1: rotary pair order inside heads of size dh:
//           dst row h*dh + p <- src row h*dh + p/2 + (p%2)*(dh/2)
//   mode 2: interleave: dst row 2i <- src row i, dst row 2i+1 <- src2 row i
// Elements are converted from the input type Tin to the compute type T
// (bf16 -> fp16 is exact except for |w| < 2^-17, which rounds to 2^-24 steps);
// a value that is not finite after the conversion (|w| > 65504 in fp16, or a
// non-finite input) sets *range_err.
template <typename Tin, typename T>
__global__ __launch_bounds__(256) void pack_kernel(const Tin* src, const Tin* src2, int rows, int K,
                                                   int mode, int dh, T* dst, int row0, int* range_err) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (size_t)rows * K) return;
  const int r = (int)(t / K), k = (int)(t % K);
  const Tin* s = src;
  int sr = r;
  if (mode == 1) {
    const int h = r / dh, p = r % dh;
    sr = h * dh + p / 2 + (p % 2) * (dh / 2);
  } else if (mode == 2) {
    s = (r & 1) ? src2 : src;
    sr = r >> 1;
  }
  const T v = Elem<T>::cvt(Elem<Tin>::load(s + (size_t)sr * K + k));
  if (!(fabsf(Elem<T>::load(&v)) <= 3.0e38f)) atomicOr(range_err, 1);
  dst[packed_off<T>(row0 + r, k, K)] = v;
}

__global__ __launch_bounds__(64) void fill_i32_kernel(int* p, int n, int v) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = v;
}

template <typename T>
__global__ __launch_bounds__(256) void to_f32_kernel(const T* src, float* dst, int n) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < n) dst[t] = Elem<T>::load(src + t);
}

}  // namespace dllm
