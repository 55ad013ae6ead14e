"""Model shapes and the five synthetic decode workloads.

The shapes are those of a LLaDA-8B-like non-causal transformer (pre-norm
RMSNorm, RoPE, SwiGLU, untied LM head, multi-head attention without GQA) and a
two-layer toy model of the same family.  The web pages name LLaDA 8B and a
"decoder-only, non-causal" architecture; the exact sizes are fixed here.

Workload shapes follow the pages' experiments: block size 32 (Fast-dLLM
reading notes, sec. 3 and sec. 8 "default block 32, threshold 0.9"), generation
lengths 256 / 1024 (Table 5), prompt 128 / generation 128 / block 32 for the
batch study (decoding-and-speed page, "hand-computed cost" section), and
blocks of 256 for block diffusion (same page, KV-cache section).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    mask_id: int
    dtype: str            # "f32" or "bf16": storage/compute type of the GPU path
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def n_params(self) -> int:
        d, f, v = self.d_model, self.d_ffn, self.vocab
        per_layer = 4 * d * d + 3 * d * f + 2 * d
        return self.n_layers * per_layer + 2 * v * d + d


TINY = ModelShape("tiny", n_layers=2, d_model=128, n_heads=4, head_dim=32, d_ffn=384,
                  vocab=512, mask_id=511, dtype="f32")
LLADA_8B = ModelShape("llada8b", n_layers=32, d_model=4096, n_heads=32, head_dim=128,
                      d_ffn=12288, vocab=126464, mask_id=126463, dtype="bf16")

CACHE_MODES = ("none", "prefix", "dual", "block_causal")
RULES = ("threshold", "factor", "topk")


@dataclass(frozen=True)
class Workload:
    """One synthetic decode problem: prompt + gen_len MASKs, block size, rule."""
    name: str
    model: ModelShape
    batch: int
    prompt_len: int
    gen_len: int
    block_len: int
    cache: str = "dual"
    rule: str = "threshold"
    tau: float = 0.9
    factor: float = 1.0
    k: int = 1
    alpha_max: float = 8.0
    weight_seed: int = 0
    prompt_seed: int = 1
    bias_seed: int = 2

    @property
    def seq_len(self) -> int:
        return self.prompt_len + self.gen_len

    @property
    def n_blocks(self) -> int:
        return self.gen_len // self.block_len

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _w(j: int, **kw) -> Workload:
    # seeds: weights 0; workload j's prompts 1000*j+1, bias 1000*j+2
    return Workload(prompt_seed=1000 * j + 1, bias_seed=1000 * j + 2, **kw)


WORKLOADS = {
    # 1: tiny fp32 model, DualCache, tau 0.9, alpha ~ U(0, 8)
    "tiny": _w(1, name="tiny", model=TINY, batch=1, prompt_len=32, gen_len=64, block_len=16,
               cache="dual", rule="threshold", tau=0.9, alpha_max=8.0),
    # 2: 8B shape, batch 1, P 512 + L 256, block 32; alpha ~ U(0, 12)
    "llada8b_p512_g256": _w(2, name="llada8b_p512_g256", model=LLADA_8B, batch=1, prompt_len=512,
                            gen_len=256, block_len=32, cache="dual", rule="threshold", tau=0.9,
                            alpha_max=12.0),
    # 3: 8B shape, batch 1/4/8/16, P 128 + L 128, block 32
    "llada8b_p128_g128": _w(3, name="llada8b_p128_g128", model=LLADA_8B, batch=16, prompt_len=128,
                            gen_len=128, block_len=32, cache="dual", rule="threshold", tau=0.9,
                            alpha_max=12.0),
    # 4: 8B shape, long canvas P 1024 + L 1024, block 32
    "llada8b_p1024_g1024": _w(4, name="llada8b_p1024_g1024", model=LLADA_8B, batch=1,
                              prompt_len=1024, gen_len=1024, block_len=32, cache="dual",
                              rule="threshold", tau=0.9, alpha_max=12.0),
    # 5: block diffusion, batch 8, P 2048 + L 1024 in blocks of 256
    "llada8b_blockdiff": _w(5, name="llada8b_blockdiff", model=LLADA_8B, batch=8, prompt_len=2048,
                            gen_len=1024, block_len=256, cache="block_causal", rule="threshold",
                            tau=0.9, alpha_max=12.0),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w
