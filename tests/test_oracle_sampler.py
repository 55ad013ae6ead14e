"""Pins of the oracle's selection rules (Algorithm 2, Algorithm 3 / eq. 13,
fixed count per step, eq. 9 error budget, LLaDA's fixed-steps schedule)
against brute-force enumeration over subsets, exact rational arithmetic and
the pages' worked examples."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle.sampler import (order_by_confidence, select_budget, select_factor, select_nkeep,
                            select_threshold, select_topk)


def _beats(a, b):
    """candidate a=(c, pos) ranks before b: higher confidence, then lower position."""
    return a[0] > b[0] or (a[0] == b[0] and a[1] < b[1])


def _is_top_set(S, cands):
    return all(_beats(s, o) for s in S for o in cands if o not in S)


def _brute_threshold(cands, tau):
    above = [p for c, p in cands if c >= np.float32(tau)]
    if above:
        return sorted(above)
    best = [s for s in cands if all(s == o or _beats(s, o) for o in cands)]
    return [best[0][1]]


def _brute_factor(cands, f):
    best = None
    for r in range(1, len(cands) + 1):
        for S in itertools.combinations(cands, r):
            if not _is_top_set(S, cands):
                continue
            cmin = min(c for c, _ in S)
            if np.float32(r + 1) * (np.float32(1) - cmin) < np.float32(f):
                if best is None or len(S) > len(best):
                    best = S
    if best is None:
        best = [s for s in cands if all(s == o or _beats(s, o) for o in cands)][:1]
    return sorted(p for _, p in best)


def _brute_topk(cands, k):
    for S in itertools.combinations(cands, min(k, len(cands))):
        if _is_top_set(S, cands):
            return sorted(p for _, p in S)


def _cases(seed, n_cases=400):
    rng = np.random.default_rng(seed)
    levels = np.array([0.05, 0.3, 0.5, 0.6, 0.7, 0.8, 0.85, 0.9, 0.95, 0.99, 1.0], np.float32)
    for _ in range(n_cases):
        m = int(rng.integers(1, 8))
        pos = np.sort(rng.choice(32, m, replace=False))
        if rng.random() < 0.5:
            conf = levels[rng.integers(0, len(levels), m)]        # many ties
        else:
            conf = rng.random(m).astype(np.float32)
        yield conf, pos


def test_threshold_matches_brute_force():
    for conf, pos in _cases(1):
        for tau in (0.5, 0.9, 1.0):
            cands = list(zip(conf.tolist(), pos.tolist()))
            assert select_threshold(conf, pos, tau).tolist() == _brute_threshold(cands, tau)


def test_factor_matches_brute_force():
    for conf, pos in _cases(2):
        for f in (0.5, 1.0, 2.0):
            cands = [(np.float32(c), p) for c, p in zip(conf.tolist(), pos.tolist())]
            assert select_factor(conf, pos, f).tolist() == _brute_factor(cands, f)


def test_topk_matches_brute_force():
    for conf, pos in _cases(3):
        for k in (1, 2, 4, 9):
            cands = list(zip(conf.tolist(), pos.tolist()))
            assert select_topk(conf, pos, k).tolist() == _brute_topk(cands, k)


def test_fallback_always_commits_one():
    for conf, pos in _cases(4):
        assert len(select_threshold(conf, pos, 1.0 + 1e-3)) == 1
        assert len(select_factor(conf, pos, 0.0)) == 1        # (n+1)(1-c) < 0 never holds
        for tau in (0.1, 0.9):
            assert len(select_threshold(conf, pos, tau)) >= 1
        assert len(select_factor(conf, pos, 1e-9)) >= 1


def test_factor_one_matches_theorem_boundary():
    # f = 1: (n+1)(1 - c_(n)) < 1  <=>  c_(n) > n/(n+1)   (Theorem 1 boundary)
    conf = np.array([0.8, 0.7, 0.6, 0.99], np.float32)
    pos = np.array([3, 5, 7, 9])
    # sorted: .99 (n=1: 2*.01), .8 (n=2: 3*.2=.6), .7 (n=3: 4*.3=1.2) -> n*=2
    assert select_factor(conf, pos, 1.0).tolist() == [3, 9]
    # f = 2 always admits n = 1 for c > 0
    assert len(select_factor(np.array([0.01], np.float32), np.array([0]), 2.0)) == 1


def test_order_and_ties():
    conf = np.array([0.5, 0.9, 0.9, 0.1], np.float32)
    pos = np.array([10, 4, 2, 1])
    assert pos[order_by_confidence(conf, pos)].tolist() == [2, 4, 10, 1]
    assert select_threshold(np.array([0.3, 0.3], np.float32), np.array([6, 5]), 0.9).tolist() == [5]


def test_llada_nkeep_schedule_spreads_masks():
    # 'what one step does': remaining masks spread over remaining steps
    rng = np.random.default_rng(5)
    L, steps = 12, 4
    masked = np.arange(L)
    total = 0
    for k in range(steps):
        sel = select_nkeep(rng.random(len(masked)).astype(np.float32), masked, steps, k)
        total += len(sel)
        masked = np.setdiff1d(masked, sel)
    assert total == L and len(masked) == 0


# ---- eq. (9): non-uniform error budget --------------------------------------
def _brute_budget(cands):
    """Largest top-set S with sum_{j in S} eps_j + max_{j in S} eps_j < 1 in exact
    rational arithmetic (eps_j = 1 - c_j); else the single top candidate."""
    best = None
    for r in range(1, len(cands) + 1):
        for S in itertools.combinations(cands, r):
            if not _is_top_set(S, cands):
                continue
            eps = [1 - Fraction(c) for c, _ in S]
            if sum(eps) + max(eps) < 1 and (best is None or len(S) > len(best)):
                best = S
    if best is None:
        best = [s for s in cands if all(s == o or _beats(s, o) for o in cands)][:1]
    return sorted(p for _, p in best)


def _grid_cases(seed, n_cases=400):
    """Confidences on a 1/64 grid: 1 - c and every partial sum of <= 8 such
    terms are exact in float32, so the float32 rule must equal the exact one."""
    rng = np.random.default_rng(seed)
    for _ in range(n_cases):
        m = int(rng.integers(1, 8))
        pos = np.sort(rng.choice(32, m, replace=False))
        conf = (rng.integers(40, 65, m) / 64.0).astype(np.float32)
        yield conf, pos


def test_budget_matches_exact_brute_force():
    for conf, pos in _grid_cases(6):
        cands = list(zip(conf.tolist(), pos.tolist()))
        assert select_budget(conf, pos).tolist() == _brute_budget(cands)


def test_budget_uniform_confidence_is_theorem_one():
    # equal eps: sum + max = (n+1) eps < 1, the strict form of eq. (8)
    for eps64 in range(1, 24):
        c = np.float32(1 - eps64 / 64.0)
        for m in range(1, 9):
            conf = np.full(m, c, np.float32)
            pos = np.arange(m)
            n = len(select_budget(conf, pos))
            expect = max(1, min(m, max(k for k in range(0, m + 1) if (k + 1) * eps64 < 64)))
            assert n == expect


def test_budget_contains_factor_one_selection():
    # sum_{j<=n} eps_j <= n eps_n, so (n+1) eps_n < 1 implies eq. (9)
    for conf, pos in _grid_cases(7):
        assert set(select_factor(conf, pos, 1.0).tolist()) <= set(select_budget(conf, pos).tolist())


def test_budget_worked_examples():
    # reading notes sec. 1: three positions above 0.95 -> (3+1) x 0.05 = 0.2 <= 1, all commit;
    # poker: eps = 0.5 each, n = 2 gives 0.5 + 0.5 + 0.5 = 1.5 -> only the top one
    assert select_budget(np.array([0.96, 0.97, 0.98], np.float32), np.array([1, 2, 3])).tolist() == [1, 2, 3]
    assert select_budget(np.array([0.5, 0.5], np.float32), np.array([4, 9])).tolist() == [4]
    # non-uniform: eps = (0.01, 0.02, 0.3): 0.01+0.02+0.3+0.3 = 0.63 < 1 -> 3; the factor
    # rule at f = 1 stops at n = 2 (4 x 0.3 = 1.2)
    conf = np.array([0.99, 0.98, 0.7], np.float32)
    pos = np.array([0, 1, 2])
    assert select_budget(conf, pos).tolist() == [0, 1, 2]
    assert select_factor(conf, pos, 1.0).tolist() == [0, 1]


# ---- LLaDA's fixed-steps schedule --------------------------------------------
def test_nkeep_worked_example():
    # decoding page: "the tea is cold", generation length 4 in 2 steps, 2 kept per step
    conf = np.array([0.9, 0.3, 0.8, 0.6], np.float32)
    pos = np.arange(4)
    first = select_nkeep(conf, pos, 2, 0)
    assert len(first) == 2 and first.tolist() == [0, 2]
    rest = np.setdiff1d(pos, first)
    assert select_nkeep(conf[rest], rest, 2, 1).tolist() == [1, 3]


def test_nkeep_counts_closed_form():
    # step k keeps floor(masked_k / (steps - k)); the last step keeps the rest
    for L, steps in ((64, 10), (7, 3), (5, 8), (32, 32)):
        masked = L
        for k in range(steps):
            n = len(select_nkeep(np.linspace(0, 1, masked, dtype=np.float32), np.arange(masked), steps, k))
            assert n == masked // (steps - k)
            masked -= n
        assert masked == 0
