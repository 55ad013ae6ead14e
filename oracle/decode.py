"""Oracle block-wise decoding loop (float64).  TEST INFRASTRUCTURE ONLY.

Follows Algorithm 1 of the Fast-dLLM reading notes (sec. 3): append L MASKs to
the prompt, initialise K/V over the full context, then for each block of B
answer positions, left to right, repeat denoising steps while the block still
holds a MASK, and refresh the cached representations before moving to the next
block (no refresh follows the last block).  Cache modes:

  * "none"   - every step recomputes all positions (LLaDA's plain sampler is
               incompatible with a KV cache: decoding-and-speed page, KV-cache
               section); same block schedule.
  * "prefix" - PrefixCache: each step recomputes the current block and the
               masked suffix; prompt and finished blocks come from the cache.
  * "dual"   - DualCache: each step recomputes only the current block; the
               suffix K/V are reused too.
  * "block_causal" - block diffusion (decoding-and-speed page, KV-cache
               section): blocks left to right, attention bidirectional inside
               a block and to all earlier blocks, never to later ones; the
               prompt is one bidirectional segment; after a block completes
               one pass over its final tokens writes its exact K/V.

A step computes logits only for the block's still-masked positions, adds the
planted bias alpha_i at target token t_i, excludes the MASK id (a committed
position must stop being MASK), takes y_i = argmax and c_i = max softmax
probability (Algorithm 2 steps 1-2), selects positions with a rule from
`sampler`, and writes y_i into all selected positions at once.

Readings where the pages are silent: the refresh pass commits nothing; the
candidate set is the current block's MASK positions; argmax ties go to the
lowest token id; in a batch every sequence decodes independently (the GPU
runs blocks in lock-step and skips finished sequences, which changes no
output).

Parity: pinned by exact invariants (DualCache/PrefixCache with a refresh
before every step equal uncached decoding; the first step after a refresh is
exact), schedule closed forms (fixed-1 and tau=1 take L steps, fixed-k takes
L/k, a dominant planted bias finishes each block in one step, LLaDA's
fixed-steps schedule commits floor(masked / (steps - k)) at step k) and the
LM-head closed form with a zero head.

Rules: "threshold", "factor", "topk" (k per step), "budget" (eq. (9)) and
"steps" (LLaDA's fixed-steps schedule with k = steps per block; with
block_len = gen_len and cache "none" it is the unblocked sampler of the
decoding-and-speed page).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from .model import KVCache, OracleModel
from .sampler import select_budget, select_factor, select_nkeep, select_threshold, select_topk


def lm_head_reduce(logits: np.ndarray, mask_id: int, target: Optional[np.ndarray] = None,
                   alpha: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Planted bias, MASK exclusion, argmax and max-softmax confidence.

    logits: [R, V] float64.  Returns (y int32 [R], c float64 [R], biased
    logits [R, V]).  y is the lowest index of the float32 maximum;
    c = 1 / sum_v exp(l_v - l_max)."""
    l = np.array(logits, dtype=np.float64, copy=True)
    if target is not None:
        r = np.arange(l.shape[0])
        l[r, target] += np.asarray(alpha, dtype=np.float32).astype(np.float64)
    l[:, mask_id] = -np.inf
    y = np.argmax(l.astype(np.float32), axis=1).astype(np.int32)
    mx = l.max(axis=1, keepdims=True)
    c = 1.0 / np.exp(l - mx).sum(axis=1)
    return y, c, l


@dataclass
class StepRecord:
    block: int
    step: int                 # index of the step inside its block
    cand: np.ndarray          # candidate positions (MASK in the block), ascending
    conf: np.ndarray          # float64 confidence per candidate
    tok: np.ndarray           # argmax token per candidate
    selected: np.ndarray      # committed positions, ascending
    logits: Optional[np.ndarray] = None   # biased logits of the candidates


@dataclass
class SeqState:
    canvas: np.ndarray
    kv: KVCache
    target: np.ndarray
    alpha: np.ndarray
    steps: int = 0
    refreshes: int = 0
    records: List[StepRecord] = field(default_factory=list)


class OracleDecoder:
    def __init__(self, model: OracleModel, prompt_len: int, gen_len: int, block_len: int,
                 cache: str = "dual", rule: str = "threshold", tau: float = 0.9,
                 factor: float = 1.0, k: int = 1, keep_logits: bool = False,
                 refresh_every: Optional[int] = None):
        if gen_len % block_len:
            raise ValueError("gen_len must be a multiple of block_len")
        if cache not in ("none", "prefix", "dual", "block_causal"):
            raise ValueError(cache)
        if rule not in ("threshold", "factor", "topk", "budget", "steps"):
            raise ValueError(rule)
        if rule in ("topk", "steps") and k < 1:
            raise ValueError("k must be >= 1")
        self.m = model
        self.P, self.L, self.B = prompt_len, gen_len, block_len
        self.N = prompt_len + gen_len
        self.cache, self.rule = cache, rule
        self.tau, self.factor, self.k = tau, factor, k
        self.keep_logits = keep_logits
        # Refresh interval inside a block (LLaDA-V experiment, reading notes
        # sec. 11): None = only at block boundaries.
        self.refresh_every = refresh_every

    # ---- geometry -------------------------------------------------------
    def block_range(self, j: int) -> Tuple[int, int]:
        s = self.P + j * self.B
        return s, s + self.B

    def key_limit(self, rows: np.ndarray) -> np.ndarray:
        rows = np.asarray(rows)
        if self.cache != "block_causal":
            return np.full(rows.shape, self.N)
        blk = np.maximum(rows - self.P, -1) // self.B           # -1 for prompt rows
        return np.where(rows < self.P, self.P, self.P + (blk + 1) * self.B)

    def step_rows(self, j: int) -> np.ndarray:
        s, e = self.block_range(j)
        if self.cache == "none":
            return np.arange(0, self.N)
        if self.cache == "prefix":
            return np.arange(s, self.N)
        return np.arange(s, e)            # dual and block_causal

    # ---- state ------------------------------------------------------------
    def new_state(self, prompt: np.ndarray, target: np.ndarray, alpha: np.ndarray) -> SeqState:
        m = self.m.shape
        canvas = np.concatenate([np.asarray(prompt, dtype=np.int32),
                                 np.full(self.L, m.mask_id, dtype=np.int32)])
        kv = KVCache(m.n_layers, self.N, m.n_heads, m.head_dim)
        return SeqState(canvas, kv, np.asarray(target), np.asarray(alpha, dtype=np.float32))

    # ---- passes -----------------------------------------------------------
    def refresh(self, st: SeqState) -> None:
        """Full-sequence pass that rewrites every cached K/V (commits nothing)."""
        rows = np.arange(self.N)
        self.m.forward_rows(st.canvas, rows, st.kv, self.key_limit(rows))
        st.refreshes += 1

    def prefill(self, st: SeqState) -> None:
        """Block diffusion: exact K/V of the prompt segment."""
        rows = np.arange(self.P)
        self.m.forward_rows(st.canvas, rows, st.kv, self.key_limit(rows))

    def commit_pass(self, st: SeqState, j: int) -> None:
        """Block diffusion: exact K/V of a finished block from its final tokens."""
        s, e = self.block_range(j)
        rows = np.arange(s, e)
        self.m.forward_rows(st.canvas, rows, st.kv, self.key_limit(rows))

    def evaluate(self, st: SeqState, j: int):
        """Forward of one step: returns (candidate positions, y, c, biased
        logits) without committing.  Updates the cache rows it recomputes."""
        m = self.m.shape
        s, e = self.block_range(j)
        rows = self.step_rows(j)
        hidden = self.m.forward_rows(st.canvas, rows, st.kv, self.key_limit(rows))
        blk = np.arange(s, e)
        cand = blk[st.canvas[blk] == m.mask_id]
        h = hidden[np.searchsorted(rows, cand)]
        gi = cand - self.P
        y, c, l = lm_head_reduce(self.m.logits(h), m.mask_id, st.target[gi], st.alpha[gi])
        return cand, y, c, l

    def choose(self, cand: np.ndarray, c: np.ndarray, k_in_block: int = 0) -> np.ndarray:
        """k_in_block: steps already taken in this block (the "steps" rule's k)."""
        if self.rule == "threshold":
            return select_threshold(c, cand, self.tau)
        if self.rule == "factor":
            return select_factor(c, cand, self.factor)
        if self.rule == "budget":
            return select_budget(c, cand)
        if self.rule == "steps":
            return select_nkeep(c, cand, self.k, k_in_block)
        return select_topk(c, cand, self.k)

    def step(self, st: SeqState, j: int) -> StepRecord:
        k_in_block = sum(1 for r in st.records if r.block == j)
        cand, y, c, l = self.evaluate(st, j)
        sel = self.choose(cand, c, k_in_block)
        idx = np.searchsorted(cand, sel)
        st.canvas[sel] = y[idx]                       # simultaneous commit
        rec = StepRecord(j, k_in_block, cand, c, y, sel, l if self.keep_logits else None)
        st.records.append(rec)
        st.steps += 1
        return rec

    def block_has_mask(self, st: SeqState, j: int) -> bool:
        s, e = self.block_range(j)
        return bool((st.canvas[s:e] == self.m.shape.mask_id).any())

    def decode(self, prompt: np.ndarray, target: np.ndarray, alpha: np.ndarray) -> SeqState:
        st = self.new_state(prompt, target, alpha)
        nb = self.L // self.B
        if self.cache == "block_causal":
            self.prefill(st)
        for j in range(nb):
            if self.cache in ("prefix", "dual"):
                self.refresh(st)
            n_in_block = 0
            while self.block_has_mask(st, j):
                if (self.refresh_every and n_in_block > 0 and self.cache in ("prefix", "dual")
                        and n_in_block % self.refresh_every == 0):
                    self.refresh(st)
                self.step(st, j)
                n_in_block += 1
                # every rule but "steps" commits >= 1 per step; "steps" ends a block in k
                if n_in_block > (self.k if self.rule == "steps" else self.B):
                    raise RuntimeError("a block outlived its step bound")
            if self.cache == "block_causal":
                self.commit_pass(st, j)
        return st

    def decode_batch(self, prompts: np.ndarray, targets: np.ndarray, alphas: np.ndarray) -> List[SeqState]:
        return [self.decode(prompts[b], targets[b], alphas[b]) for b in range(prompts.shape[0])]
