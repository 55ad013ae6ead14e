"""Roofline arithmetic for the decode step.

`teaching_*` reproduce the teaching model of the decoding-and-speed page
("hand-computed cost" section): a 7B bf16 model of 1.4e10 weight bytes on a
3.352 TB/s, 989.4 TFLOP/s part; one forward over n positions costs at least
max(W, n C) with W the weight-read time and C = 2 * params / peak per
position.  The MI355X functions give the algorithmic bytes and flops of this
library's kernels for the LLaDA-8B shape.
"""
from __future__ import annotations

from dataclasses import dataclass

MI355X_HBM_BYTES_PER_S = 8.0e12
MI355X_BF16_DENSE_FLOPS = 2.5e15
MI355X_FP32_VECTOR_FLOPS = 157.3e12


@dataclass(frozen=True)
class Teaching:
    weight_bytes: float = 1.4e10
    bw: float = 3.352e12
    peak: float = 989.4e12

    @property
    def W_ms(self) -> float:            # one read of the weights
        return self.weight_bytes / self.bw * 1e3

    @property
    def C_ms(self) -> float:            # compute per position: 2N flops, N = bytes/2 params
        return self.weight_bytes / self.peak * 1e3

    def step_ms(self, n: int) -> float:
        return max(self.W_ms, n * self.C_ms)

    @property
    def crossover(self) -> float:
        return self.W_ms / self.C_ms


def step_bytes_8b(shape, n_keys: int, rows: int, lm_rows: int = 1) -> dict:
    """Algorithmic HBM bytes of one cached block step (bf16): every projection
    weight once, the LM head once, K/V of all n_keys positions read and the
    fresh rows' K/V written, for every layer."""
    d, f, v, L = shape.d_model, shape.d_ffn, shape.vocab, shape.n_layers
    layer_w = (4 * d * d + 3 * d * f) * 2
    head_w = v * d * 2
    kv_per_pos = L * 2 * d * 2            # K and V, all layers, bf16
    return {
        "weights": L * layer_w + head_w,
        "kv_read": kv_per_pos * n_keys,
        "kv_write": kv_per_pos * rows,
        "total": L * layer_w + head_w + kv_per_pos * (n_keys + rows),
    }


def step_flops_8b(shape, rows: int, n_keys: int, lm_rows: int) -> float:
    d, f, v, L = shape.d_model, shape.d_ffn, shape.vocab, shape.n_layers
    proj = 2.0 * rows * L * (4 * d * d + 3 * d * f)
    attn = 4.0 * rows * n_keys * d * L
    head = 2.0 * lm_rows * v * d
    return proj + attn + head
