"""Joint-versus-product-of-marginals facts behind parallel decoding.
TEST INFRASTRUCTURE ONLY.

Fast-dLLM reading notes, sec. 4 (two-position example, eq. 4), sec. 5
(Theorem 1, eqs. 5-8, and its tightness construction), sec. 5.1 (eq. 9,
non-uniform error budget), sec. 5.2 (eqs. 10-12: L_r / total-variation and
forward-KL bounds; KL(p||q) equals the total correlation).  A joint
distribution over n positions with vocabulary V is an array of shape (V,)*n.
"""
from __future__ import annotations

import itertools
from typing import List

import numpy as np


def marginals(p: np.ndarray) -> List[np.ndarray]:
    n = p.ndim
    return [p.sum(axis=tuple(a for a in range(n) if a != j)) for j in range(n)]


def product_of_marginals(p: np.ndarray) -> np.ndarray:
    q = np.ones(())
    for mj in marginals(p):
        q = np.multiply.outer(q, mj)
    return q


def tv(p: np.ndarray, q: np.ndarray) -> float:
    return 0.5 * float(np.abs(p - q).sum())


def lr_norm(p: np.ndarray, q: np.ndarray, r: float) -> float:
    return float((np.abs(p - q) ** r).sum() ** (1.0 / r))


def kl(p: np.ndarray, q: np.ndarray) -> float:
    """sum p log(p/q) in nats; infinite when q = 0 where p > 0."""
    p = p.ravel()
    q = q.ravel()
    s = 0.0
    for a, b in zip(p, q):
        if a > 0:
            if b <= 0:
                return float("inf")
            s += a * np.log(a / b)
    return float(s)


def entropy(p: np.ndarray) -> float:
    p = p.ravel()
    p = p[p > 0]
    return float(-(p * np.log(p)).sum())


def total_correlation(p: np.ndarray) -> float:
    """sum_j H(X_j) - H(X_1..X_n)  (eq. 11, first line)."""
    return sum(entropy(m) for m in marginals(p)) - entropy(p)


def argmax_set(p: np.ndarray) -> List[tuple]:
    mx = p.max()
    return [tuple(int(i) for i in ix) for ix in zip(*np.nonzero(p == mx))]


def greedy_marginal_choice(p: np.ndarray) -> tuple:
    return tuple(int(np.argmax(m)) for m in marginals(p))


def theorem1_premise(p: np.ndarray, eps: float) -> bool:
    """Every position's top marginal exceeds 1 - eps and (n+1) eps <= 1."""
    n = p.ndim
    return all(m.max() > 1.0 - eps for m in marginals(p)) and (n + 1) * eps <= 1.0


def tightness_joint(n: int, eta: float) -> np.ndarray:
    """Mass 1/(n+1) - eta on the all-zero string and 1/(n+1) + eta/n on each
    string with exactly one 1 (sec. 5, closing paragraph)."""
    p = np.zeros((2,) * n)
    p[(0,) * n] = 1.0 / (n + 1) - eta
    for j in range(n):
        ix = [0] * n
        ix[j] = 1
        p[tuple(ix)] = 1.0 / (n + 1) + eta / n
    return p


def tv_bound(n: int, eps: float) -> float:
    """eq. 10, last line: TV(p, q) < (3n - 1)/2 * eps."""
    return (3 * n - 1) / 2.0 * eps


def lr_bound(n: int, eps: float, r: float) -> float:
    """eq. 10, second line: ||p - q||_r < ((n-1)^r + 2n)^(1/r) eps."""
    return ((n - 1) ** r + 2 * n) ** (1.0 / r) * eps


def binary_entropy(e: float) -> float:
    if e <= 0 or e >= 1:
        return 0.0
    return float(-e * np.log(e) - (1 - e) * np.log(1 - e))


def kl_bound(n: int, eps: float, vocab: int) -> float:
    """eq. 12: KL(p||q) < (n-1) [h_b(eps) + eps log(V-1)]."""
    return (n - 1) * (binary_entropy(eps) + eps * np.log(vocab - 1))


def nonuniform_budget_ok(eps_j: np.ndarray) -> bool:
    """eq. 9: sum_j eps_j + max_j eps_j < 1 is sufficient for the top choices
    to form the joint argmax."""
    eps_j = np.asarray(eps_j, dtype=np.float64)
    return float(eps_j.sum() + eps_j.max()) < 1.0


def all_strings(vocab: int, n: int):
    return itertools.product(range(vocab), repeat=n)
