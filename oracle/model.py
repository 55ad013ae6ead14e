"""Oracle transformer forward (float64), TEST INFRASTRUCTURE ONLY.

A LLaDA-like non-causal transformer: decoder-only with non-causal attention
(dian8dian article, "dLLM mechanism" section).  Attention follows eq. (3) of
the Fast-dLLM reading notes, softmax(Q K^T / sqrt(d)) V, per head.  The other
components are not described on the pages; the readings taken are: pre-norm
residual blocks, RMSNorm (eps 1e-5, learned gain), rotary position embedding
with theta 10000 and half-split (rotate-half) pairing at absolute canvas
positions, multi-head attention with no bias, SwiGLU feed-forward
W_d (silu(W_g h) * W_u h), final RMSNorm and an untied LM head.

Pins: the whole forward against transformers' LLaMA implementation driven
with an all-visible (bidirectional) or block-causal 4-D mask; RMSNorm against
torch.nn.functional.rms_norm; attention against torch's
scaled_dot_product_attention; RoPE against a complex-multiplication
formulation and the relative-position property.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np


def _as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:  # bfloat16 bit patterns: widen exactly
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * gain


def rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate pairs (x[j], x[j + dh/2]) by angle pos * theta^(-2j/dh).
    x: [T, H, dh]; positions: [T] absolute canvas indices."""
    dh = x.shape[-1]
    half = dh // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / dh)
    ang = positions.astype(np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, key_limit: np.ndarray) -> np.ndarray:
    """Eq. (3) per head.  q: [Tq, H, dh]; k, v: [Tk, H, dh]; query t sees keys
    [0, key_limit[t]).  Returns [Tq, H, dh]."""
    dh = q.shape[-1]
    s = (q.transpose(1, 0, 2) @ k.transpose(1, 2, 0)) / np.sqrt(dh)      # [H, Tq, Tk]
    keys = np.arange(k.shape[0])
    visible = keys[None, :] < key_limit[:, None]            # [Tq, Tk]
    s = np.where(visible[None, :, :], s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return (p @ v.transpose(1, 0, 2)).transpose(1, 0, 2)                   # [Tq, H, dh]


class KVCache:
    """Per-layer K and V for every canvas position of one sequence: [N, H, dh]
    (K after RoPE).  The fresh K/V of a forward over some rows overwrite the
    cached rows they replace."""

    def __init__(self, n_layers: int, n_pos: int, n_heads: int, head_dim: int):
        self.k = np.zeros((n_layers, n_pos, n_heads, head_dim))
        self.v = np.zeros((n_layers, n_pos, n_heads, head_dim))

    def copy(self) -> "KVCache":
        c = KVCache.__new__(KVCache)
        c.k = self.k.copy()
        c.v = self.v.copy()
        return c


class OracleModel:
    """Weights are given as float32 arrays or uint16 bf16 bit patterns
    ([out, in] for linear maps) and widened to float64 on use."""

    def __init__(self, shape, tensors: Dict[str, np.ndarray], keep_f64: Optional[bool] = None):
        self.shape = shape
        self.tensors = tensors
        if keep_f64 is None:
            keep_f64 = shape.n_params < 50_000_000
        self._cache: Dict[str, np.ndarray] = {}
        self._keep = keep_f64

    def materialize(self, threads: int = 16) -> None:
        """Widen every tensor to float64 once, in parallel (large models)."""
        from concurrent.futures import ThreadPoolExecutor
        self._keep = True
        names = [n for n in self.tensors if n not in self._cache]
        with ThreadPoolExecutor(threads) as ex:
            for n, a in zip(names, ex.map(lambda n: _as_f64(self.tensors[n]), names)):
                self._cache[n] = a

    def w(self, name: str) -> np.ndarray:
        if name in self._cache:
            return self._cache[name]
        a = _as_f64(self.tensors[name])
        if self._keep:
            self._cache[name] = a
        return a

    def forward_rows(self, tokens: np.ndarray, rows: np.ndarray, kv: KVCache,
                     key_limit: np.ndarray) -> np.ndarray:
        """Run the model over canvas positions `rows` of one sequence.

        Each layer computes q, k, v for the rows, writes k, v into `kv` at those
        rows, then lets row t attend to keys [0, key_limit[t]) of the cache
        (cached rows plus the fresh ones just written).  Returns the final
        RMS-normed hidden states [len(rows), d_model]."""
        m = self.shape
        H, dh = m.n_heads, m.head_dim
        rows = np.asarray(rows, dtype=np.int64)
        x = self.w("emb")[tokens[rows]]
        for l in range(m.n_layers):
            p = f"l{l}."
            h = rms_norm(x, self.w(p + "attn_norm"), m.rms_eps)
            q = (h @ self.w(p + "wq").T).reshape(-1, H, dh)
            k = (h @ self.w(p + "wk").T).reshape(-1, H, dh)
            v = (h @ self.w(p + "wv").T).reshape(-1, H, dh)
            q = rope(q, rows, m.rope_theta)
            k = rope(k, rows, m.rope_theta)
            kv.k[l, rows] = k
            kv.v[l, rows] = v
            o = attention(q, kv.k[l], kv.v[l], key_limit)
            x = x + o.reshape(-1, H * dh) @ self.w(p + "wo").T
            h2 = rms_norm(x, self.w(p + "ffn_norm"), m.rms_eps)
            a = silu(h2 @ self.w(p + "wg").T) * (h2 @ self.w(p + "wu").T)
            x = x + a @ self.w(p + "wd").T
        return rms_norm(x, self.w("final_norm"), m.rms_eps)

    def logits(self, hidden: np.ndarray) -> np.ndarray:
        return hidden @ self.w("lm_head").T
