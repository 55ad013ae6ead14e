"""Plain CPU oracle for Fast-dLLM-style block-wise masked-diffusion decoding.

TEST INFRASTRUCTURE ONLY.  Nothing in the product library imports this
package; only the tests, the smoke check and the benchmark's CPU-baseline leg
may import or run it.  It shares no code with the HIP path: the only thing both
sides consume is the seeded input generator in ``workloads``.

Arithmetic is float64 NumPy (the pages fix no precision).  Decisions that
turn a float into an integer (argmax over the vocabulary, threshold / factor
comparisons) are taken in float32, the GPU kernels' precision.

Sources (web pages on diffusion-LM decoding):
  * "Fast-dLLM reading notes" (zhongzhuzhou.org): eq. (3) attention; sec. 3
    PrefixCache / DualCache and Algorithm 1 (block-wise cached decoding);
    Algorithm 2 (threshold with top-1 fallback); sec. 6, eq. (13) and
    Algorithm 3 (factor rule); sec. 5, eqs. (4)-(12) (Theorem 1 and bounds).
  * "Diffusion LMs: decoding steps, caches and real speed"
    (tianyi-zhang-02.github.io): "what one step does" (fixed-count
    low-confidence remasking), "KV cache" section (block diffusion with an
    exact cache written by one pass after each block).
  * dian8dian.com article on Fast-dLLM: block-level cache reuse and global
    refresh after each block; threshold with top-1 fallback.

Parity status per function is listed in the module headers; the model
forward at random initialisation has no printed values on the pages and is
pinned by library reductions (transformers' LLaMA with a bidirectional mask,
torch SDPA / rms_norm / silu), closed forms and exact invariants.
"""
from .model import OracleModel, KVCache
from .sampler import (select_threshold, select_factor, select_topk, select_nkeep, select_budget,
                      order_by_confidence)
from .decode import OracleDecoder, StepRecord, lm_head_reduce
from .diagnostics import cosine_rows, staleness

__all__ = [
    "OracleModel", "KVCache", "select_threshold", "select_factor", "select_topk",
    "select_nkeep", "select_budget", "order_by_confidence", "OracleDecoder", "StepRecord", "lm_head_reduce",
    "cosine_rows", "staleness",
]
