"""The GPU-vs-oracle step comparison itself (tests/parity.py), on synthetic
step data: planted GPU mistakes must be reported, and only differences at a
rule's cut may be exempt.  Runs on the CPU."""
import numpy as np
import pytest

from oracle import OracleDecoder, OracleModel
from workloads import TINY, gen_weights

from .parity import Report, Tol, compare_step


@pytest.fixture(scope="module")
def model():
    return OracleModel(TINY, gen_weights(TINY, seed=0))


def _step(dec, c, gc, gpu_sel=None, gpu_tok=None, k_in_block=0):
    """Candidates 40..40+n-1; oracle tokens 100+i; the GPU reports gc and
    commits gpu_sel (default: the rule on gc) with tokens gpu_tok."""
    n = len(c)
    cand = np.arange(40, 40 + n)
    y = 100 + np.arange(n)
    gt = y.copy() if gpu_tok is None else np.asarray(gpu_tok)
    before = np.full(40 + n, TINY.mask_id)
    before[:40] = 3
    after = before.copy()
    sel = dec.choose(cand, np.asarray(gc), k_in_block) if gpu_sel is None else np.asarray(gpu_sel)
    after[sel] = gt[np.searchsorted(cand, sel)]
    return cand, y, np.asarray(c, float), np.asarray(gc, float), gt, before, after


def _run(dec, tol, *args, **kw):
    rep = Report()
    cand, y, c, gc, gt, before, after = _step(dec, *args, **kw)
    compare_step(rep, tol, dec, cand, y, c, None, gc, gt, None, before, after, kw.get("k_in_block", 0))
    return rep


def test_identical_step_passes(model):
    dec = OracleDecoder(model, 40, 16, 16, rule="threshold", tau=0.9)
    c = [0.95, 0.3, 0.91, 0.1]
    rep = _run(dec, Tol(fp32=False), c, c)
    assert not rep.bad and rep.exempt == 0 and rep.decisions == 4


def test_extra_commit_is_reported_even_at_low_confidence(model):
    dec = OracleDecoder(model, 40, 16, 16, rule="threshold", tau=0.9)
    c = [0.95, 0.001, 0.002, 0.001]
    rep = _run(dec, Tol(fp32=False), c, c, gpu_sel=[40, 41])
    assert any("its own confidences select" in b for b in rep.bad)
    assert any("selection differs at 41" in b for b in rep.bad)


def test_committed_token_must_be_gpu_argmax(model):
    dec = OracleDecoder(model, 40, 16, 16, rule="topk", k=2)
    c = [0.5, 0.4, 0.3, 0.2]
    rep = Report()
    cand, y, c_, gc, gt, before, after = _step(dec, c, c)
    after[40] = 999                              # committed something else than the reported argmax
    compare_step(rep, Tol(fp32=False), dec, cand, y, c_, None, gc, gt, None, before, after)
    assert any("own argmax" in b for b in rep.bad)


def test_near_tau_difference_is_exempt_in_bf16_only(model):
    dec = OracleDecoder(model, 40, 16, 16, rule="threshold", tau=0.9)
    c = [0.95, 0.895, 0.3, 0.1]
    gc = [0.95, 0.903, 0.3, 0.1]                 # the GPU's rounding lifts position 41 over tau
    rep = _run(dec, Tol(fp32=False), c, gc)
    assert not rep.bad and rep.exempt_sel == 1
    rep = _run(dec, Tol(fp32=True), c, gc)
    assert any("selection differs at 41" in b for b in rep.bad)


def test_difference_away_from_the_cut_is_reported(model):
    # top-2: the cut lies between 0.5 and 0.2, so a GPU that reports the
    # 0.5 position low and commits the 0.2 one (by its own numbers) is a
    # real difference, not a near-tie at the cut
    dec = OracleDecoder(model, 40, 16, 16, rule="topk", k=2)
    c = [0.6, 0.5, 0.2, 0.19, 0.01]
    gc = [0.6, 0.15, 0.2, 0.19, 0.01]            # (conf error 0.35: also reported)
    rep = _run(dec, Tol(fp32=False), c, gc)
    assert any("selection differs at 41" in b for b in rep.bad)
    assert any("selection differs at 42" in b for b in rep.bad)
    assert any("conf err" in b for b in rep.bad)
    # a swap across the cut of two confidences within 0.02 is exempt
    c = [0.6, 0.5, 0.49, 0.19, 0.01]
    gc = [0.6, 0.494, 0.496, 0.19, 0.01]
    rep = _run(dec, Tol(fp32=False), c, gc)
    assert not rep.bad and rep.exempt_sel == 2


def test_fallback_near_tie_is_exempt(model):
    dec = OracleDecoder(model, 40, 16, 16, rule="threshold", tau=0.9)
    c = [0.301, 0.30, 0.1]
    gc = [0.300, 0.302, 0.1]
    rep = _run(dec, Tol(fp32=False), c, gc)
    assert not rep.bad and rep.exempt_sel == 2


def test_factor_count_change_exempt_only_when_near_critical(model):
    dec = OracleDecoder(model, 40, 16, 16, rule="factor", factor=1.0)
    # n = 2 needs 3 (1 - c_2) < 1, i.e. c_2 > 2/3: oracle just below, GPU just above
    c = [0.9, 0.665, 0.1]
    gc = [0.9, 0.668, 0.1]
    rep = _run(dec, Tol(fp32=False), c, gc)
    assert not rep.bad and rep.exempt_sel == 1
    # a count change with c_2 far from 2/3 is a real difference
    rep = _run(dec, Tol(fp32=False), [0.9, 0.5, 0.1], [0.9, 0.5, 0.1], gpu_sel=[40, 41])
    assert rep.bad


def test_exemption_cap(model):
    rep = Report(decisions=150, exempt_sel=2)
    rep.check_exemptions(0.01)
    assert rep.bad
    rep = Report(decisions=250, exempt_sel=2, exempt_tok=2)
    rep.check_exemptions(0.01)
    assert not rep.bad
