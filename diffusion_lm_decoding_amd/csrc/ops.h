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
                                                    const float* gain, T* xg, float* ssq) {
  const int m = blockIdx.x;
  const int b = m / g.nr, pos = g.row_start + m % g.nr;
  const int tok = min(max(tokens[(size_t)b * seq_len + pos], 0), vocab - 1);
  const Tin* e = emb + (size_t)tok * d;
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

// ---- LM-head merge: per row, combine the vocab-tile partials ---------------
// max and argmax (lowest index among equal maxima), then
// S = sum_t s_t exp(m_t - max); confidence = 1 / S.
__global__ __launch_bounds__(256) void lm_merge_kernel(const float* pmax, const float* psum,
                                                       const int* parg, int n_tiles, int M,
                                                       float* conf, int* tok, int* err) {
  __shared__ float shm[256];
  __shared__ int sha[256];
  __shared__ float shs[4];
  const int m = blockIdx.x, t0 = threadIdx.x;
  float mx = -INFINITY;
  int am = 0x7fffffff;
  for (int t = t0; t < n_tiles; t += 256) {
    const float v = pmax[(size_t)t * M + m];
    const int a = parg[(size_t)t * M + m];
    if (v > mx || (v == mx && a < am)) { mx = v; am = a; }
  }
  shm[t0] = mx;
  sha[t0] = am;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t0 < s) {
      const float v = shm[t0 + s];
      const int a = sha[t0 + s];
      if (v > shm[t0] || (v == shm[t0] && a < sha[t0])) { shm[t0] = v; sha[t0] = a; }
    }
    __syncthreads();
  }
  const float gm = shm[0];
  const int ga = sha[0];
  float s = 0.f;
  for (int t = t0; t < n_tiles; t += 256) s += psum[(size_t)t * M + m] * expf(pmax[(size_t)t * M + m] - gm);
  s = block_sum<256>(s, shs);
  if (t0 == 0) {
    conf[m] = 1.0f / s;
    tok[m] = ga;
    if (!(fabsf(gm) <= 3.0e38f) || !(s >= 1.0f && s <= 3.0e38f)) atomicOr(err, 1);
  }
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
  int* commit_step;     // [batch][gen_len] or null
  int* ncommit;         // [batch]
  int* done;            // [batch]
  const int* err;       // nonzero: commit nothing
  float* dbg_conf;      // [batch*blk] or null
  int* dbg_tok;
};

__global__ __launch_bounds__(256) void select_commit_kernel(SelectArgs a) {
  __shared__ float sc[256];
  __shared__ int sm[256];
  __shared__ float red[4];
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
    a.ncommit[b] = cnt;
    a.done[b] = (n_masked - cnt == 0) ? 1 : 0;
    if (n_masked > 0 && !*a.err) a.step_ctr[b] = step + 1;
  }
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
// (bf16 -> fp16 is exact except for |w| < 2^-17, which rounds to 2^-24 steps).
template <typename Tin, typename T>
__global__ __launch_bounds__(256) void pack_kernel(const Tin* src, const Tin* src2, int rows, int K,
                                                   int mode, int dh, T* dst, int row0) {
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
  dst[packed_off<T>(row0 + r, k, K)] = Elem<T>::cvt(Elem<Tin>::load(s + (size_t)sr * K + k));
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
