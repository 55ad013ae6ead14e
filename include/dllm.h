/*
 * dllm.h - C ABI of the MI355X block-wise masked-diffusion decoding library.
 *
 * The library runs the denoising step of Fast-dLLM-style decoding for a
 * LLaDA-like non-causal transformer on one AMD Instinct MI355X (gfx950):
 * recompute the current block (or block + suffix, or everything), attend to
 * cached and fresh K/V, reduce the LM head of the still-masked positions to
 * (argmax token, max-softmax confidence), and commit positions under the
 * threshold, factor or fixed-count rule.
 *
 * Sources (web pages on diffusion-LM decoding):
 *   [RN]  "Fast-dLLM reading notes" (zhongzhuzhou.org): eq. (3) attention;
 *         sec. 3 PrefixCache / DualCache and Algorithm 1; Algorithm 2
 *         (threshold + top-1 fallback); sec. 6, eq. (13), Algorithm 3 (factor).
 *   [DS]  "Diffusion LMs: decoding steps, caches and real speed"
 *         (tianyi-zhang-02.github.io): "what one step does" (fixed count per
 *         step, low-confidence remasking); "KV cache" section (block diffusion
 *         with an exact cache written after each block).
 *   [FD]  dian8dian.com article on Fast-dLLM: cache reuse inside a block with a
 *         global refresh after the block; threshold with top-1 fallback.
 *
 * Conventions for every call:
 *   - Every call returns dllm_status; DLLM_OK is 0.  On any other status
 *     dllm_last_error() returns a message (thread-local, valid until the next
 *     call on that thread).  No C++ exception crosses this boundary.
 *   - Arguments are validated before any GPU work is enqueued.  A call that
 *     fails validation changes nothing.
 *   - "device" pointers are HIP device allocations on the context's GPU;
 *     "host" pointers are ordinary CPU memory.  The caller owns every pointer
 *     it passes; the context owns its packed weights, KV cache and workspaces
 *     (sized at dllm_init_weights from max_batch / max_seq) and frees them in
 *     dllm_destroy.
 *   - All GPU work is enqueued on the HIP stream given to dllm_init_weights.
 *     A context is not thread-safe: use one context per stream.
 *   - Token ids are int32.  The canvas of a sequence is prompt_len prompt
 *     tokens followed by gen_len answer positions, row-major [batch, seq].
 */
#ifndef DLLM_H
#define DLLM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DLLM_OK = 0,
  DLLM_ERR_ARG = 1,      /* invalid argument or configuration                 */
  DLLM_ERR_OOM = 2,      /* device allocation failed, or it would exceed the
                            limit set by dllm_set_device_limit                */
  DLLM_ERR_DEVICE = 3,   /* a HIP call failed                                 */
  DLLM_ERR_STATE = 4,    /* call out of order (a step or commit pass with no
                            cache pass over the canvas since
                            dllm_begin_decode), or a step committed nothing   */
  DLLM_ERR_NUMERIC = 5   /* non-finite logits / confidences were produced     */
} dllm_status;

typedef enum { DLLM_F32 = 0, DLLM_BF16 = 1 } dllm_dtype;

/* Which positions a denoising step recomputes ([RN] sec. 3, Algorithm 1):
 *   NONE   every position, every step (no cache; [DS] KV-cache section);
 *   PREFIX current block and the masked suffix; prompt and finished blocks
 *          come from the cache (PrefixCache);
 *   DUAL   only the current block; prefix and suffix K/V are reused
 *          (DualCache);
 *   BLOCK_CAUSAL  block diffusion ([DS] KV-cache section): attention is
 *          bidirectional inside a block and to everything before it, never to
 *          later blocks; the prompt is one bidirectional segment; finished
 *          blocks hold exact K/V written by one pass after the block. */
typedef enum {
  DLLM_CACHE_NONE = 0,
  DLLM_CACHE_PREFIX = 1,
  DLLM_CACHE_DUAL = 2,
  DLLM_CACHE_BLOCK_CAUSAL = 3
} dllm_cache_mode;

/* Selection rule applied to the block's still-masked positions, ordered by
 * confidence descending then position ascending:
 *   THRESHOLD  commit every c_i >= tau; if none, the top one ([RN] Alg. 2);
 *   FACTOR     commit the top n for the largest n with
 *              (n+1)(1 - c_(n)) < factor; if none, the top one ([RN] eq. 13,
 *              Alg. 3);
 *   TOPK       commit the top min(k, #masked) ([DS] "what one step does");
 *   BUDGET     with eps_j = 1 - c_(j), commit the top n for the largest n with
 *              eps_1 + ... + eps_n + eps_n < 1 (the sum accumulated in that
 *              order); if none, the top one ([RN] sec. 5.1, eq. 9: in
 *              confidence order eps_n is the largest of the n);
 *   STEPS      LLaDA's fixed-steps schedule with k steps per block: the
 *              block's s-th step (s = 0 .. k-1, counted since
 *              dllm_begin_decode or the last step on another block) commits
 *              the top floor(#masked / (k - s)), possibly none; the k-th
 *              commits the rest ([DS] the sample() listing).  With
 *              block_len = gen_len and CACHE_NONE this is LLaDA's unblocked
 *              sampler.
 * Comparisons are evaluated in float32. */
typedef enum {
  DLLM_RULE_THRESHOLD = 0,
  DLLM_RULE_FACTOR = 1,
  DLLM_RULE_TOPK = 2,
  DLLM_RULE_BUDGET = 3,
  DLLM_RULE_STEPS = 4
} dllm_rule;

/* Model shape.  The architecture is pre-norm RMSNorm, rotary position
 * embedding (rotate-half pairing, absolute canvas positions), multi-head
 * attention softmax(QK^T / sqrt(head_dim)) V ([RN] eq. 3) without masking
 * inside the attended range, SwiGLU feed-forward, final RMSNorm, untied LM
 * head.  Supported: dtype DLLM_BF16 or DLLM_F32; d_model = n_heads*head_dim;
 * head_dim in {32, 64, 128}; d_model, d_ffn, vocab multiples of 32;
 * 0 <= mask_id < vocab. */
typedef struct {
  int32_t n_layers, d_model, n_heads, head_dim, d_ffn, vocab, mask_id;
  float rms_eps, rope_theta;
  int32_t dtype;       /* dllm_dtype of the weights.  DLLM_F32 computes in
                          fp32 (fp32 MFMA).  DLLM_BF16 holds the weights as
                          fp16 copies (exact for |w| >= 2^-17) and runs fp16
                          activations, KV cache and MFMA inputs with fp32
                          accumulation and softmax: with bf16's 8-bit
                          significand the rounding at each projection input
                          compounds over deep models into logit errors of
                          order 0.1, fp16's 11 bits keep them ~8x smaller.
                          fp16 range: residual-stream values must stay below
                          65504 in magnitude, else DLLM_ERR_NUMERIC.          */
  int32_t max_batch;   /* largest batch any later call may use               */
  int32_t max_seq;     /* largest prompt_len + gen_len any later call may use */
} dllm_model_cfg;

/* One decode problem ([RN] Algorithm 1 inputs: prompt, answer length L,
 * block size B, selection rule).  gen_len must be a multiple of block_len;
 * tau in (0, 1]; factor > 0; k >= 1 (TOPK: tokens per step; STEPS: steps
 * per block).  refresh_every > 0 additionally
 * refreshes the cache every refresh_every steps inside a block (PREFIX/DUAL
 * only; [RN] sec. 11 decouples the refresh interval from the block size);
 * 0 refreshes only at block boundaries. */
typedef struct {
  int32_t batch, prompt_len, gen_len, block_len;
  int32_t cache;          /* dllm_cache_mode */
  int32_t rule;           /* dllm_rule       */
  float tau, factor;
  int32_t k;
  int32_t refresh_every;
} dllm_decode_cfg;

/* Caller-owned decode state (all device memory).
 *   tokens       int32 [batch, prompt_len + gen_len]; prompt then mask_id;
 *                committed answer tokens are written in place.
 *   bias_target  int32 [batch, gen_len] or NULL; bias_alpha float [batch,
 *                gen_len] or NULL: a planted logit bias alpha_i added to token
 *                target_i of answer position i before the softmax (used to make
 *                the confidence of random-weight models controllable).
 *   commit_step  int32 [batch, gen_len] or NULL: receives, for each answer
 *                position, the 0-based index of the step (counted per sequence
 *                over the whole decode) that committed it. */
typedef struct {
  int32_t* tokens;
  const int32_t* bias_target;
  const float* bias_alpha;
  int32_t* commit_step;
} dllm_canvas;

/* Decode statistics.  The three device-time fields follow the cost split of
 * [RN] sec. 7, eq. (15): T = S C_active + R + T_selection.
 *   ms_step    S C_active: the denoising steps' forward passes, from the
 *              embedding through the LM-head projection of the masked rows;
 *   ms_refresh R: refresh, prompt and commit passes;
 *   ms_select  T_selection: turning the LM-head partials into (argmax,
 *              confidence) and applying the rule (merge + select/commit);
 * each the device time between HIP events on the context's stream: every
 * cache pass is timed; the step split is timed on every 8th denoising step
 * that is not a cache pass (the 1st, 9th, ...) and scaled to all of them,
 * since each event lengthens the launch gaps around it by microseconds.
 * Under PREFIX and DUAL, dllm_decode makes each refresh the forward of the
 * step that follows it (see dllm_decode): such a step counts in steps and in
 * refreshes, and all of its device time (forward, LM head, selection) in
 * ms_refresh.  ms_total - (ms_step + ms_refresh + ms_select) is host time:
 * launches and the per-step status readback. */
typedef struct {
  int64_t steps;          /* denoising steps (forward passes with a commit)   */
  int64_t refreshes;      /* full-canvas K/V refresh passes                   */
  int64_t committed;      /* tokens committed over all sequences              */
  int64_t max_seq_steps;  /* largest per-sequence step count                  */
  double ms_total;        /* wall time of the call                            */
  double ms_refresh;      /* device time in refresh / prefill / commit passes */
  double ms_step;         /* device time in the other steps' forward passes   */
  double ms_select;       /* device time in their LM-head merge + selection   */
} dllm_stats;

typedef struct dllm_ctx dllm_ctx;

/* Create a context and load the weights.
 *   tensors: host array of 2 + 9*n_layers DEVICE pointers, in this order:
 *     emb [vocab, d_model];
 *     per layer l: attn_norm [d_model], wq, wk, wv, wo [d_model, d_model],
 *                  ffn_norm [d_model], wg, wu [d_ffn, d_model],
 *                  wd [d_model, d_ffn];
 *     final_norm [d_model]; lm_head [vocab, d_model].
 *   Linear maps are row-major [out, in] (y = x W^T).  Element type is float
 *   for DLLM_F32 and bfloat16 (uint16 bit patterns) for DLLM_BF16, norm
 *   gains included.  The weights are copied into the context's packed layout;
 *   the caller may free its tensors when the call returns.
 *   hip_stream: hipStream_t on which all later work runs (NULL = default).
 * Errors: DLLM_ERR_ARG (unsupported shape, NULL pointer, a weight that is not
 *   finite or - for DLLM_BF16, computed in fp16 - has |w| > 65504),
 *   DLLM_ERR_OOM (also when the context would exceed dllm_set_device_limit),
 *   DLLM_ERR_DEVICE.  *out is NULL on failure. */
dllm_status dllm_init_weights(dllm_ctx** out, const dllm_model_cfg* cfg,
                              const void* const* tensors, void* hip_stream);

/* Cache pass over the canvas (writes K and V of every layer in place).
 *   cache PREFIX / DUAL / NONE: a full bidirectional pass over all
 *     prompt_len + gen_len positions ([RN] Algorithm 1: initialise before
 *     the first block, refresh before each next block).  Commits nothing.
 *     block_idx is ignored.
 *   cache BLOCK_CAUSAL: block_idx < 0 runs the prompt pass (prompt positions
 *     only, bidirectional among themselves); block_idx = j >= 0 runs the
 *     commit pass of answer block j: its final tokens attend to [0, end of
 *     block j) and their exact K/V are stored ([DS] KV-cache section).
 * A pass over the whole canvas, or the prompt pass, marks the cache as holding
 * K/V of a canvas of this batch / prompt_len / gen_len (what dllm_block_step
 * and the commit pass require).
 * Errors: DLLM_ERR_ARG (bad cfg, batch > max_batch, seq > max_seq),
 *   DLLM_ERR_STATE (a commit pass with no prompt pass since
 *   dllm_begin_decode), DLLM_ERR_DEVICE. */
dllm_status dllm_refresh_cache(dllm_ctx* ctx, const dllm_canvas* canvas,
                               const dllm_decode_cfg* cfg, int32_t block_idx);

/* One denoising step on answer block block_idx (0-based) of every sequence.
 * The positions given by the cache mode are recomputed; their fresh K/V
 * overwrite the cached rows they replace; the block's still-masked positions
 * get y_i = argmax (lowest id on ties; mask_id excluded) and
 * c_i = max softmax probability; the rule selects positions; selected
 * positions receive y_i simultaneously ([RN] Algorithm 2 step 5).  A sequence
 * whose block holds no mask commits nothing.  Every rule but STEPS commits at
 * least one token of a block that holds a mask.
 *   n_committed, block_done: host int32 [batch] outputs (tokens committed by
 *     this step; 1 if the block holds no mask afterwards), or NULL.
 *   dbg_logits: device float [batch * block_len, vocab] or NULL: biased
 *     logits of every block row (mask_id column = -inf) - a slow debug path.
 *   dbg_conf, dbg_tok: device float / int32 [batch * block_len] or NULL:
 *     c_i and y_i of the block's masked rows (-1 for rows already committed).
 * Blocks the host until the 8-byte-per-sequence result is read back.
 * Errors: DLLM_ERR_ARG, DLLM_ERR_STATE (cache modes other than NONE: no
 *   dllm_refresh_cache over a canvas of this batch / prompt_len / gen_len
 *   since dllm_begin_decode - block diffusion: no prompt pass), DLLM_ERR_NUMERIC
 *   (non-finite confidence; the canvas is left unchanged), DLLM_ERR_DEVICE. */
dllm_status dllm_block_step(dllm_ctx* ctx, dllm_canvas* canvas, const dllm_decode_cfg* cfg,
                            int32_t block_idx, int32_t* n_committed, int32_t* block_done,
                            float* dbg_logits, float* dbg_conf, int32_t* dbg_tok);

/* dllm_block_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, arguments, outputs and errors, with its per-step
 * workspaces (LM-head partial (max, sum, argmax) per 16-entry vocabulary
 * tile, confidences, tokens, attention key-share partials) in the library's
 * static device scratch instead of the context's.  The scratch is one
 * 16 MiB array per GPU, held until the process ends; every call on a GPU
 * shares it and leaves its contents behind (each call writes every entry it
 * reads before reading it, so nothing needs clearing), so calls that overlap
 * on one GPU - from two streams, threads or contexts - race.  Serves steps
 * whose forward and LM head cover at most 64 rows (batch x rows recomputed
 * by the cache mode) and whose LM-head partials fit the scratch (vocab up to
 * about 200k at 64 rows); any other step fails with DLLM_ERR_ARG before device
 * work.  Allocates nothing (no hipMalloc, hipFree or allocating library call). */
dllm_status dllm_block_step_noalloc(dllm_ctx* ctx, dllm_canvas* canvas, const dllm_decode_cfg* cfg,
                                    int32_t block_idx, int32_t* n_committed, int32_t* block_done,
                                    float* dbg_logits, float* dbg_conf, int32_t* dbg_tok);

/* Cached-vs-fresh diagnostics at the current canvas ([RN] sec. 14 and
 * Algorithm 4 steps 4-5: compare fresh and cached predictions at the commit
 * positions, and how far the cached K/V have drifted).  For block block_idx
 * of every sequence it evaluates the block's rows twice without committing:
 * as a block step of cfg->cache would, from the current (possibly stale)
 * cache, and from a full fresh forward over the canvas (the no-cache step).
 * It also compares, per layer and canvas position, the cached K and V (as
 * they were on entry) with the fresh ones.  The cache is restored before the
 * call returns, so a decode continues exactly as without it.  cfg->cache must
 * be NONE, PREFIX or DUAL.  Allocates a temporary device snapshot of the K/V
 * of cfg->batch sequences (2 x n_layers x batch x n_heads x max_seq x head_dim
 * elements).
 *   conf_cached, tok_cached, conf_fresh, tok_fresh: device float / int32
 *     [batch * block_len] or NULL: c_i and y_i of the block's masked rows
 *     (-1 for rows already committed).
 *   k_cos, v_cos: device float [n_layers, batch, prompt_len + gen_len] or NULL:
 *     <cached, fresh> / (|cached| |fresh|) over all heads of the position
 *     (1 if both are zero, 0 if one is).
 * Blocks until done.  Errors: DLLM_ERR_ARG, DLLM_ERR_STATE (as
 *   dllm_block_step), DLLM_ERR_OOM, DLLM_ERR_NUMERIC, DLLM_ERR_DEVICE. */
dllm_status dllm_staleness(dllm_ctx* ctx, const dllm_canvas* canvas, const dllm_decode_cfg* cfg, int32_t block_idx,
                           float* conf_cached, int32_t* tok_cached, float* conf_fresh, int32_t* tok_fresh,
                           float* k_cos, float* v_cos);

/* Start of a decode driven by the caller with dllm_refresh_cache /
 * dllm_block_step: checks that the prompt holds no mask_id (and lies in
 * [0, vocab)) and the answer region is all mask_id, and resets the
 * per-sequence step counters (commit_step numbering, the STEPS schedule).
 * The cache counts as empty afterwards (the next step needs a cache pass).
 * dllm_decode does this itself.  Errors: DLLM_ERR_ARG, DLLM_ERR_DEVICE. */
dllm_status dllm_begin_decode(dllm_ctx* ctx, const dllm_canvas* canvas, const dllm_decode_cfg* cfg);

/* Whole decode ([RN] Algorithm 1, or block diffusion for BLOCK_CAUSAL):
 * dllm_begin_decode, then for each block: refresh (PREFIX / DUAL) and steps until the
 * block holds no mask in any sequence (lock-step over the batch; finished
 * sequences commit nothing).  No refresh follows the last block.
 * A refresh and the step after it share one forward: the step evaluates the
 * block from a forward over the whole canvas, which rewrites every cached K/V
 * exactly as dllm_refresh_cache does, and right after a refresh the cached
 * step is exact ([RN] sec. 3), so its logits are the ones the refresh +
 * dllm_block_step sequence computes, without the second forward over the
 * block.  The same holds for the refreshes that refresh_every inserts.
 *   stats: host output or NULL.
 * Tracing: with the environment variable DLLM_TRACE set to a path, one JSON
 *   line is appended there per cache pass ({"event":"refresh", block,
 *   in_block, pass = block_idx given to dllm_refresh_cache (0 for the
 *   PREFIX / DUAL refreshes), ms}), per step ({"event":"step", block,
 *   in_block, step, committed[batch], done[batch], cache_pass = 1 on a step
 *   that refreshed the cache (its refresh line comes first), and on every
 *   8th other step ms_forward / ms_select}) and per decode
 *   ({"event":"decode", steps, refreshes, committed}).  dllm_decode, each
 *   block, dllm_refresh_cache and dllm_block_step push roctx ranges
 *   (rocprofv3 --marker-trace).
 * Errors: DLLM_ERR_ARG (also: DLLM_TRACE names a file that cannot be opened
 *   for appending), DLLM_ERR_STATE (a step of a rule other than STEPS
 *   committed nothing while masks remained, or a block outlived its step
 *   bound), DLLM_ERR_NUMERIC, DLLM_ERR_DEVICE. */
dllm_status dllm_decode(dllm_ctx* ctx, dllm_canvas* canvas, const dllm_decode_cfg* cfg,
                        dllm_stats* stats);

/* Kernel timing for measurement.  Kernel classes of one forward/step: */
typedef enum {
  DLLM_K_EMBED = 0,   /* token embedding gather                          */
  DLLM_K_RMSNORM,     /* RMSNorm into the packed projection input        */
  DLLM_K_QKV,         /* Q/K/V projection + rotary + K/V cache write     */
  DLLM_K_ATTN,        /* attention over the cache                        */
  DLLM_K_OPROJ,       /* output projection + residual                    */
  DLLM_K_GATEUP,      /* gate/up projection + SwiGLU                     */
  DLLM_K_DOWN,        /* down projection + residual                      */
  DLLM_K_LMHEAD,      /* LM head + planted bias + (max, sum, argmax)     */
  DLLM_K_MERGE,       /* per-row merge of the LM-head partials           */
  DLLM_K_SELECT,      /* select / commit                                 */
  DLLM_K_COUNT
} dllm_kernel_class;

typedef struct {
  int64_t launches;   /* timed launches                                           */
  double ms;          /* summed device time between HIP events around each launch */
  double bytes;       /* summed algorithmic HBM bytes: every operand read once and
                         every output written once (weights, activations, K/V)     */
  double flops;       /* summed algorithmic floating-point operations              */
} dllm_kernel_time;

/* Bracket later launches of the kernel classes in class_mask (bit i =
 * class i) with HIP events on the context's stream; 0 turns timing off.
 * Of each class's launches (counted separately for denoising steps and cache
 * passes, from this call on) the 1st, (1+sample_every)th, ... are timed:
 * sample_every = 1 times them all.  The events themselves lengthen the gaps
 * around a timed launch by a few microseconds, so a throughput measurement
 * samples (e.g. 31, coprime to the layer count, so the sample rotates over
 * the layers).  Counters accumulate until read with reset = 1.
 * Errors: DLLM_ERR_ARG (ctx NULL, sample_every 0). */
dllm_status dllm_set_timing(dllm_ctx* ctx, uint32_t class_mask, uint32_t sample_every);

/* Wait for the stream, then copy the counters to out, a host array of
 * 2 * DLLM_K_COUNT entries: [0, DLLM_K_COUNT) for launches made by
 * dllm_block_step (denoising steps), [DLLM_K_COUNT, 2 * DLLM_K_COUNT) for
 * launches made by dllm_refresh_cache (cache passes); reset != 0 zeroes them.
 * Errors: DLLM_ERR_ARG, DLLM_ERR_DEVICE. */
dllm_status dllm_get_timing(dllm_ctx* ctx, dllm_kernel_time* out, int32_t reset);

/* Achievable peaks on the current device, measured with the library's own
 * microkernels (no context needed): hbm_gbs = GB/s of a streaming read of
 * `bytes` bytes (a temporary device buffer; pass >= 4 GiB so the memory-side
 * cache does not hold it; best of three grid sizes), mfma_f16_tflops = TFLOP/s
 * of register-resident 32x32x16 fp16 MFMA chains on every CU.  Either output may be NULL.
 * Errors: DLLM_ERR_ARG (bytes < 1 MiB), DLLM_ERR_OOM, DLLM_ERR_DEVICE. */
dllm_status dllm_probe_peaks(uint64_t bytes, double* hbm_gbs, double* mfma_f16_tflops);

/* Streaming-read rate at a given size: the best GB/s of hbm_read_kernel
 * reading one `bytes`-byte buffer (one launch, kernel duration from its
 * dispatch packet; 256, 512 and 1024 workgroups tried), the buffer rotating
 * over copies that together exceed the memory-side cache, so every read comes
 * from HBM.  At the size of one projection's weights this is the ceiling of
 * a kernel that streams them once, ramp-up and drain included, which a read
 * of gigabytes (dllm_probe_peaks) hides.  Allocates its buffers (up to 32 x
 * bytes, at least 1 GiB) for the duration of the call.
 * Errors: DLLM_ERR_ARG (bytes < 1 MiB or gbs NULL), DLLM_ERR_OOM, DLLM_ERR_DEVICE. */
dllm_status dllm_probe_read(uint64_t bytes, double* gbs);

/* Matrix-pipe throughput of an MFMA stream that shares the CU with LDS
 * traffic: one workgroup of 4 * waves_per_simd waves per CU, each wave issuing
 * per 16 fp16 32x32x16 MFMAs (4 accumulators, operands in registers and
 * independent of the loads) `lds_reads` 1 KiB ds_read_b128 reads and
 * `dma_kib` 1 KiB global_load_lds copies (from a buffer that stays in L2,
 * into LDS).  These are the proportions of a large-M projection's main loop
 * (a 128x128 wave tile reads 8 KiB of operands per 16 MFMAs; a 256x256
 * workgroup tile copies 4 KiB per wave per 16 MFMAs).  *tflops = MFMA
 * TFLOP/s of the whole device, best of 3 launches.  Allocates 260 KiB for the
 * duration of the call.
 * Errors: DLLM_ERR_ARG (waves_per_simd not 1 or 2, lds_reads not 0 or 8,
 *   dma_kib not 0, 2 or 4, tflops NULL), DLLM_ERR_OOM, DLLM_ERR_DEVICE. */
dllm_status dllm_probe_mfma_mix(int32_t waves_per_simd, int32_t lds_reads, int32_t dma_kib, double* tflops);

/* Process-wide cap on the device memory a context may hold: dllm_init_weights
 * fails with DLLM_ERR_OOM, before allocating past it, when the packed weights,
 * KV cache and workspaces of the requested shape exceed `bytes`, and
 * dllm_staleness does the same for its snapshot; contexts created earlier are
 * not affected.  0 (the default) removes the cap.  For callers that budget
 * device memory, and to exercise the out-of-memory path. */
void dllm_set_device_limit(uint64_t bytes);

/* Release every device allocation of the context.  NULL is ignored. */
void dllm_destroy(dllm_ctx* ctx);

/* Message of the last non-OK status on the calling thread ("" if none). */
const char* dllm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DLLM_H */
