"""Oracle selection rules (which masked positions a step commits).
TEST INFRASTRUCTURE ONLY.

Inputs are the block's candidate positions (still MASK) and their
confidences c_i = max_v p_i(v).  Comparisons are evaluated in float32.

  * threshold rule with top-1 fallback: Fast-dLLM reading notes,
    Algorithm 2 (keep every c_i >= tau; if none, keep the single most
    confident position).  ">=" is the listing's comparison.
  * factor rule: reading notes sec. 6, eq. (13) and Algorithm 3: sort by
    confidence descending, keep the largest n with (n+1)(1 - c_(n)) < f,
    where c_(n) is the n-th largest; if no n qualifies keep the top one.
  * fixed count per step (top-k): decoding-and-speed page, "what one step
    does": low-confidence remasking keeps the most confident predictions
    (Kim et al.'s fixed 4 tokens per step).
  * n_keep schedule of LLaDA's sampler (same section): with `steps` total
    steps, step k keeps len(masked) // (steps - k) positions (possibly
    none; the last step keeps every remaining one).
  * non-uniform error budget: reading notes sec. 5.1, eq. (9): with
    eps_j = 1 - c_(j) over the candidates in confidence order, keep the
    largest n with sum_{j<=n} eps_j + max_{j<=n} eps_j < 1.  In that order
    max_{j<=n} eps_j = eps_n.  Evaluated in float32 (eps_j = 1 - c_(j)
    rounded, the sum accumulated in order); if no n qualifies keep the top
    one, as the factor rule does.

Ties in confidence are broken by lower position (the pages are silent).
Pins: brute-force enumeration over small inputs (tests/test_oracle_sampler.py).
"""
from __future__ import annotations

import numpy as np


def order_by_confidence(conf: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Indices of candidates sorted by (confidence desc, position asc)."""
    c = np.asarray(conf, dtype=np.float32)
    return np.lexsort((np.asarray(pos), -c.astype(np.float64)))


def select_threshold(conf: np.ndarray, pos: np.ndarray, tau: float) -> np.ndarray:
    c = np.asarray(conf, dtype=np.float32)
    pos = np.asarray(pos)
    if c.size == 0:
        return pos[:0]
    keep = c >= np.float32(tau)
    if keep.any():
        return np.sort(pos[keep])
    return pos[order_by_confidence(c, pos)[:1]]


def select_factor(conf: np.ndarray, pos: np.ndarray, f: float) -> np.ndarray:
    c = np.asarray(conf, dtype=np.float32)
    pos = np.asarray(pos)
    if c.size == 0:
        return pos[:0]
    order = order_by_confidence(c, pos)
    best = 0
    for n in range(1, c.size + 1):
        c_n = c[order[n - 1]]
        lhs = np.float32(n + 1) * (np.float32(1.0) - c_n)
        if lhs < np.float32(f):
            best = n
    if best == 0:
        best = 1
    return np.sort(pos[order[:best]])


def select_topk(conf: np.ndarray, pos: np.ndarray, k: int) -> np.ndarray:
    c = np.asarray(conf, dtype=np.float32)
    pos = np.asarray(pos)
    order = order_by_confidence(c, pos)
    return np.sort(pos[order[:min(k, c.size)]])


def select_budget(conf: np.ndarray, pos: np.ndarray) -> np.ndarray:
    c = np.asarray(conf, dtype=np.float32)
    pos = np.asarray(pos)
    if c.size == 0:
        return pos[:0]
    order = order_by_confidence(c, pos)
    best = 0
    total = np.float32(0.0)
    for n in range(1, c.size + 1):
        eps_n = np.float32(np.float32(1.0) - c[order[n - 1]])
        total = np.float32(total + eps_n)
        if np.float32(total + eps_n) < np.float32(1.0):
            best = n
    if best == 0:
        best = 1
    return np.sort(pos[order[:best]])


def select_nkeep(conf: np.ndarray, pos: np.ndarray, steps: int, k: int) -> np.ndarray:
    """LLaDA's fixed-steps schedule: remaining masks spread over remaining steps."""
    n_keep = len(pos) // (steps - k)
    return select_topk(conf, pos, n_keep)
