"""Counter-based synthetic inputs (weights, prompts, planted bias).

Every value is a pure function of (seed, stream id, element index), so any
slice of any tensor can be regenerated on its own, in any order, by any
consumer.  The mixing function is Chris Wellons' "lowbias32" 32-bit integer
hash (hash-prospector, 2018); all arithmetic is on numpy uint32 arrays, whose
multiply and shifts are exact modulo 2**32.

Weights are "normal, std 0.02" in the sense of an Irwin-Hall(4) variate: the
sum of four independent 16-bit uniforms, centred and scaled to the requested
standard deviation (bounded tails at +-3.46 sigma, 262141 levels).  It is
computed in float32 with a single rounding, so it is bit-reproducible.
bf16 copies are round-to-nearest-even truncations of those float32 values,
carried as uint16 bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np

from .configs import ModelShape

_U32 = np.uint32
_CHUNK = 1 << 20


def _lowbias32(x: np.ndarray) -> np.ndarray:
    x = x ^ (x >> _U32(16))
    x = x * _U32(0x7FEB352D)
    x = x ^ (x >> _U32(15))
    x = x * _U32(0x846CA68B)
    x = x ^ (x >> _U32(16))
    return x


def _key(seed: int, stream: int) -> np.uint32:
    a = _lowbias32(np.array([(stream * 0x9E3779B1 + 0x632BE5AB) & 0xFFFFFFFF], dtype=_U32))
    b = _lowbias32(np.array([seed & 0xFFFFFFFF], dtype=_U32) ^ a)
    return _U32(int(b[0]))


def _bits(key: np.uint32, start: int, count: int) -> np.ndarray:
    """Hash words for counters start..start+count-1 (counter < 2**32)."""
    if start + count > (1 << 32):
        raise ValueError("counter range exceeds 2**32")
    ctr = np.arange(start, start + count, dtype=np.uint64).astype(_U32)
    return _lowbias32(ctr ^ key)


# Irwin-Hall(4) of U{0..65535}: mean 131070, variance 4*(65536**2-1)/12
_IH_MEAN = 131070
_IH_SIGMA = float(np.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0))


def _gaussianish(key: np.uint32, start: int, count: int, std: float) -> np.ndarray:
    ha = _bits(key, 2 * start, 2 * count)          # two words per element
    w0 = ha[0::2]
    w1 = ha[1::2]
    s = ((w0 & _U32(0xFFFF)).astype(np.int32) + (w0 >> _U32(16)).astype(np.int32)
         + (w1 & _U32(0xFFFF)).astype(np.int32) + (w1 >> _U32(16)).astype(np.int32))
    centred = (s - _IH_MEAN).astype(np.float32)     # exact: |s - mean| < 2**18
    return centred * np.float32(std / _IH_SIGMA)    # one float32 rounding


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.
    Inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(_U32)
    lsb = (u >> _U32(16)) & _U32(1)
    r = (u + _U32(0x7FFF) + lsb) >> _U32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(_U32) << _U32(16)).view(np.float32)


def tensor_names(m: ModelShape) -> List[Tuple[str, Tuple[int, ...]]]:
    """Canonical tensor order and shapes.  Linear weights are [out, in] (y = x W^T)."""
    d, f, v = m.d_model, m.d_ffn, m.vocab
    out = [("emb", (v, d))]
    for l in range(m.n_layers):
        out += [
            (f"l{l}.attn_norm", (d,)),
            (f"l{l}.wq", (d, d)), (f"l{l}.wk", (d, d)), (f"l{l}.wv", (d, d)), (f"l{l}.wo", (d, d)),
            (f"l{l}.ffn_norm", (d,)),
            (f"l{l}.wg", (f, d)), (f"l{l}.wu", (f, d)), (f"l{l}.wd", (d, f)),
        ]
    out += [("final_norm", (d,)), ("lm_head", (v, d))]
    return out


def _stream_id(m: ModelShape, name: str) -> int:
    for i, (n, _) in enumerate(tensor_names(m)):
        if n == name:
            return i + 1
    raise KeyError(name)


def _shape(m: ModelShape, name: str) -> Tuple[int, ...]:
    for n, s in tensor_names(m):
        if n == name:
            return s
    raise KeyError(name)


def _threads() -> int:
    n = os.environ.get("OMP_NUM_THREADS")
    try:
        return max(1, min(16, int(n) if n else (os.cpu_count() or 1)))
    except ValueError:
        return 1


def gen_tensor(m: ModelShape, name: str, seed: int = 0, as_bf16: Optional[bool] = None,
               std: float = 0.02, gain_jitter: float = 0.0) -> np.ndarray:
    """One named tensor.  Norm gains are 1 (plus gain_jitter * N~(0,1) when
    nonzero, used by tests to exercise the gain path).  Returns float32, or
    uint16 bf16 bits when as_bf16 (default: the model's dtype)."""
    if as_bf16 is None:
        as_bf16 = m.dtype == "bf16"
    shape = _shape(m, name)
    count = int(np.prod(shape))
    key = _key(seed, _stream_id(m, name))
    is_gain = name.endswith("norm")
    out = np.empty(count, dtype=np.uint16 if as_bf16 else np.float32)

    def work(start: int) -> None:
        n = min(_CHUNK, count - start)
        if is_gain:
            if gain_jitter:
                vals = np.float32(1.0) + _gaussianish(key, start, n, gain_jitter)
            else:
                vals = np.ones(n, dtype=np.float32)
        else:
            vals = _gaussianish(key, start, n, std)
        out[start:start + n] = f32_to_bf16_bits(vals) if as_bf16 else vals

    starts = range(0, count, _CHUNK)
    if count > 4 * _CHUNK:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, starts))
    else:
        for s in starts:
            work(s)
    return out.reshape(shape)


def gen_weights(m: ModelShape, seed: int = 0, as_bf16: Optional[bool] = None,
                gain_jitter: float = 0.0) -> Dict[str, np.ndarray]:
    return {n: gen_tensor(m, n, seed, as_bf16, gain_jitter=gain_jitter)
            for n, _ in tensor_names(m)}


def _uniform_int(key: np.uint32, count: int, hi_exclusive: int) -> np.ndarray:
    h = _bits(key, 0, count).astype(np.uint64)
    return ((h * np.uint64(hi_exclusive)) >> np.uint64(32)).astype(np.int32)


def gen_prompt(m: ModelShape, batch: int, prompt_len: int, seed: int) -> np.ndarray:
    """Uniform random prompt tokens in [0, vocab-2] (never the MASK id)."""
    v = _uniform_int(_key(seed, 0xA11CE), batch * prompt_len, m.vocab - 1)
    return v.reshape(batch, prompt_len)


def gen_bias(m: ModelShape, batch: int, gen_len: int, seed: int,
             alpha_max: float) -> Tuple[np.ndarray, np.ndarray]:
    """Planted logit bias for generated position i: target t_i uniform in
    [0, vocab-2] and strength alpha_i uniform in [0, alpha_max) (float32)."""
    n = batch * gen_len
    t = _uniform_int(_key(seed, 0xB1A5), n, m.vocab - 1).reshape(batch, gen_len)
    u = (_bits(_key(seed, 0xA1FA), 0, n) >> _U32(8)).astype(np.float32) * np.float32(2.0 ** -24)
    a = (u * np.float32(alpha_max)).astype(np.float32).reshape(batch, gen_len)
    return t, a
