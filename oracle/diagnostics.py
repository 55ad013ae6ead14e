"""Oracle cached-vs-fresh diagnostics.  TEST INFRASTRUCTURE ONLY.

Fast-dLLM reading notes, sec. 14 and Algorithm 4 (steps 4-5): at the moment
of a commit, compare the prediction made from the (stale) cache with the one
a fresh computation makes, and relate the gap to how far the cached K/V have
drifted.  For block j of one sequence, at its current canvas and cache:

  * the cached evaluation is the step of the decoder's cache mode, without
    committing (`OracleDecoder.evaluate`);
  * the fresh evaluation is a forward over every canvas row with every key
    (the no-cache step), into a separate cache;
  * per layer and canvas position, the cosine similarity between the cached
    K (and V) as they were on entry and the fresh ones, over all heads:
    <a, b> / (|a| |b|), 1 when both are zero, 0 when one is.

The sequence's cache is left as it was on entry.  Parity pins:
tests/test_oracle_diagnostics.py.
"""
from __future__ import annotations

import numpy as np

from .decode import OracleDecoder, SeqState, lm_head_reduce
from .model import KVCache


def cosine_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Cosine similarity of a[..., p, :, :] and b[..., p, :, :] flattened over
    the last two axes."""
    a = a.reshape(*a.shape[:-2], -1)
    b = b.reshape(*b.shape[:-2], -1)
    dot = (a * b).sum(-1)
    na = (a * a).sum(-1)
    nb = (b * b).sum(-1)
    out = np.where((na > 0) & (nb > 0), dot / np.sqrt(np.maximum(na * nb, 1e-300)), 0.0)
    return np.where((na == 0) & (nb == 0), 1.0, out)


def staleness(dec: OracleDecoder, st: SeqState, j: int) -> dict:
    if dec.cache == "block_causal":
        raise ValueError("the block-causal cache is exact")
    m = dec.m.shape
    entry = st.kv.copy()
    cand, y_c, c_c, l_c = dec.evaluate(st, j)
    fresh = KVCache(m.n_layers, dec.N, m.n_heads, m.head_dim)
    rows = np.arange(dec.N)
    hidden = dec.m.forward_rows(st.canvas, rows, fresh, np.full(dec.N, dec.N))
    gi = cand - dec.P
    y_f, c_f, l_f = lm_head_reduce(dec.m.logits(hidden[cand]), m.mask_id, st.target[gi], st.alpha[gi])
    st.kv = entry
    return {"cand": cand, "tok_cached": y_c, "conf_cached": c_c, "tok_fresh": y_f, "conf_fresh": c_f,
            "logits_cached": l_c, "logits_fresh": l_f,
            "k_cos": cosine_rows(entry.k, fresh.k), "v_cos": cosine_rows(entry.v, fresh.v)}
