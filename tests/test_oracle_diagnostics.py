"""Pins of the oracle's cached-vs-fresh diagnostics (reading notes sec. 14,
Algorithm 4): the cosine against scipy, exactness right after a refresh and
in the uncached mode, and that the diagnostic leaves the decode state alone."""
import numpy as np
import pytest
from scipy.spatial.distance import cosine as scipy_cosine

from oracle import OracleDecoder, OracleModel, cosine_rows, staleness
from workloads import TINY, gen_bias, gen_prompt, gen_weights


@pytest.fixture(scope="module")
def tiny_model():
    return OracleModel(TINY, gen_weights(TINY, seed=0, gain_jitter=0.1))


def test_cosine_matches_scipy_and_zero_conventions():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((2, 5, 4, 8))
    b = a + 0.3 * rng.standard_normal(a.shape)
    got = cosine_rows(a, b)
    for l in range(2):
        for p in range(5):
            assert abs(got[l, p] - (1 - scipy_cosine(a[l, p].ravel(), b[l, p].ravel()))) < 1e-12
    z = np.zeros((1, 2, 4, 8))
    one = z.copy()
    one[0, 1] = 1.0
    assert cosine_rows(z, z).tolist() == [[1.0, 1.0]]
    assert cosine_rows(z, one).tolist() == [[1.0, 0.0]]


def _state(model, cache, steps, alpha_max=16.0):
    pr = gen_prompt(TINY, 1, 32, 11)
    t, a = gen_bias(TINY, 1, 64, 12, alpha_max)
    dec = OracleDecoder(model, 32, 64, 16, cache=cache, rule="threshold", tau=0.9)
    st = dec.new_state(pr[0], t[0], a[0])
    if cache in ("prefix", "dual"):
        dec.refresh(st)
    for _ in range(steps):
        dec.step(st, 0)
    return dec, st


@pytest.mark.parametrize("cache", ["dual", "prefix"])
def test_exact_right_after_refresh(tiny_model, cache):
    dec, st = _state(tiny_model, cache, 0)
    r = staleness(dec, st, 0)
    assert np.array_equal(r["tok_cached"], r["tok_fresh"])
    assert np.abs(r["conf_cached"] - r["conf_fresh"]).max() < 1e-12
    assert np.abs(r["k_cos"] - 1).max() < 1e-12 and np.abs(r["v_cos"] - 1).max() < 1e-12


def test_uncached_evaluations_agree(tiny_model):
    dec, st = _state(tiny_model, "none", 2)
    r = staleness(dec, st, 0)
    assert np.array_equal(r["tok_cached"], r["tok_fresh"])
    assert np.abs(r["conf_cached"] - r["conf_fresh"]).max() < 1e-12


def test_dual_cache_drifts_and_state_is_untouched(tiny_model):
    dec, st = _state(tiny_model, "dual", 3)
    k0, v0, canvas0 = st.kv.k.copy(), st.kv.v.copy(), st.canvas.copy()
    r = staleness(dec, st, 0)
    assert np.array_equal(st.kv.k, k0) and np.array_equal(st.kv.v, v0) and np.array_equal(st.canvas, canvas0)
    # committed tokens changed the context: some cached K/V are stale
    assert r["k_cos"].min() < 1 - 1e-6 and r["v_cos"].min() < 1 - 1e-6
    assert (r["k_cos"] <= 1 + 1e-12).all()
    # the cached evaluation is the step's own evaluation
    cand, y, c, _ = dec.evaluate(st, 0)
    st.kv.k[:], st.kv.v[:] = k0, v0
    assert np.array_equal(cand, r["cand"]) and np.array_equal(y, r["tok_cached"])
    assert np.abs(c - r["conf_cached"]).max() == 0.0
