"""Pins of the oracle's decode loop and LM-head reduction: closed forms,
schedule step counts and exact cache invariants (tiny model, float64)."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import OracleDecoder, OracleModel, lm_head_reduce
from workloads import TINY, gen_bias, gen_prompt, gen_weights, workload


@pytest.fixture(scope="module")
def tiny_model():
    return OracleModel(TINY, gen_weights(TINY, seed=0, gain_jitter=0.1))


def _inputs(P=32, L=64, seed=1, alpha_max=8.0, batch=1):
    pr = gen_prompt(TINY, batch, P, seed)
    t, a = gen_bias(TINY, batch, L, seed + 1, alpha_max)
    return pr, t, a


def test_lm_head_closed_form_zero_head():
    V, mask = TINY.vocab, TINY.mask_id
    alpha = np.array([0.0, 1.5, 7.25, 30.0], np.float32)
    tgt = np.array([17, 3, 400, 0], np.int32)
    y, c, _ = lm_head_reduce(np.zeros((4, V)), mask, tgt, alpha)
    a = alpha.astype(np.float64)
    expect_c = np.exp(a) / (np.exp(a) + V - 2)
    assert np.allclose(c, expect_c, rtol=1e-14)
    assert y[0] == 0 and (y[1:] == tgt[1:]).all()
    assert abs(c[0] - 1.0 / (V - 1)) < 1e-15


def test_lm_head_matches_scipy_softmax():
    rng = np.random.default_rng(0)
    l = rng.normal(size=(6, 512)) * 3
    tgt = rng.integers(0, 511, 6)
    alpha = rng.random(6).astype(np.float32) * 5
    y, c, lb = lm_head_reduce(l, 511, tgt, alpha)
    ref = l.copy()
    ref[np.arange(6), tgt] += alpha.astype(np.float64)
    p = softmax(np.delete(ref, 511, axis=1), axis=1)
    assert np.allclose(c, p.max(axis=1), rtol=1e-13)
    assert (y == p.argmax(axis=1)).all()
    assert np.isneginf(lb[:, 511]).all()


def test_mask_token_never_chosen():
    l = np.zeros((2, 512))
    l[:, 511] = 100.0
    y, c, _ = lm_head_reduce(l, 511)
    assert (y != 511).all() and np.allclose(c, 1 / 511)


@pytest.mark.parametrize("k,expect", [(1, 64), (4, 16), (16, 4)])
def test_fixed_k_step_counts(tiny_model, k, expect):
    pr, t, a = _inputs()
    dec = OracleDecoder(tiny_model, 32, 64, 16, cache="dual", rule="topk", k=k)
    st = dec.decode(pr[0], t[0], a[0])
    assert st.steps == expect and st.refreshes == 4
    assert (st.canvas != TINY.mask_id).all()


def test_unblocked_fixed_steps_sampler(tiny_model):
    # LLaDA's sampler (decoding page): one block over the whole answer, every
    # step a full forward, step k commits floor(masked / (steps - k))
    pr, t, a = _inputs()
    steps = 10
    dec = OracleDecoder(tiny_model, 32, 64, 64, cache="none", rule="steps", k=steps)
    st = dec.decode(pr[0], t[0], a[0])
    assert st.steps == steps and st.refreshes == 0
    masked = 64
    for k, r in enumerate(st.records):
        assert r.step == k and len(r.selected) == masked // (steps - k)
        masked -= len(r.selected)
    assert masked == 0 and (st.canvas != TINY.mask_id).all()


def test_fixed_steps_per_block(tiny_model):
    # semi-autoregressive use: the schedule restarts in every block
    pr, t, a = _inputs()
    dec = OracleDecoder(tiny_model, 32, 64, 16, cache="dual", rule="steps", k=5)
    st = dec.decode(pr[0], t[0], a[0])
    assert st.steps == 4 * 5
    assert [len(r.selected) for r in st.records[:5]] == [3, 3, 3, 3, 4]


def test_budget_rule_decodes(tiny_model):
    pr, t, a = _inputs(alpha_max=16.0)
    dec = OracleDecoder(tiny_model, 32, 64, 16, cache="dual", rule="budget")
    st = dec.decode(pr[0], t[0], a[0])
    assert (st.canvas != TINY.mask_id).all()
    for r in st.records:
        c = np.sort(r.conf[np.isin(r.cand, r.selected)].astype(np.float32))[::-1]
        eps = 1.0 - c.astype(np.float64)
        assert len(r.selected) == 1 or eps.sum() + eps.max() < 1.0 + 1e-6


def test_tau_one_takes_L_steps(tiny_model):
    pr, t, a = _inputs(alpha_max=8.0)
    dec = OracleDecoder(tiny_model, 32, 64, 16, cache="dual", rule="threshold", tau=1.0)
    st = dec.decode(pr[0], t[0], a[0])
    assert st.steps == 64
    assert all(len(r.selected) == 1 for r in st.records)


def test_dominant_bias_finishes_each_block_in_one_step(tiny_model):
    pr, t, _ = _inputs()
    a = np.full((1, 64), 30.0, np.float32)
    for cache in ("none", "prefix", "dual", "block_causal"):
        dec = OracleDecoder(tiny_model, 32, 64, 16, cache=cache, rule="threshold", tau=0.9)
        st = dec.decode(pr[0], t[0], a[0])
        assert st.steps == 4, cache
        assert (st.canvas[32:] == t[0]).all()


def test_each_block_finishes_within_B_steps(tiny_model):
    pr, t, a = _inputs(alpha_max=16.0)
    for rule, kw in (("threshold", dict(tau=0.9)), ("factor", dict(factor=1.0)),
                     ("factor", dict(factor=2.0))):
        dec = OracleDecoder(tiny_model, 32, 64, 16, cache="dual", rule=rule, **kw)
        st = dec.decode(pr[0], t[0], a[0])
        assert st.steps <= 64
        for j in range(4):
            assert sum(1 for r in st.records if r.block == j) <= 16
        assert all(len(r.selected) >= 1 for r in st.records)


@pytest.mark.parametrize("cache", ["dual", "prefix"])
def test_refresh_every_step_equals_uncached(tiny_model, cache):
    pr, t, a = _inputs(alpha_max=16.0)
    ref = OracleDecoder(tiny_model, 32, 64, 16, cache="none", rule="threshold", tau=0.9,
                        keep_logits=True).decode(pr[0], t[0], a[0])
    got = OracleDecoder(tiny_model, 32, 64, 16, cache=cache, rule="threshold", tau=0.9,
                        keep_logits=True, refresh_every=1).decode(pr[0], t[0], a[0])
    assert np.array_equal(ref.canvas, got.canvas) and ref.steps == got.steps
    for r1, r2 in zip(ref.records, got.records):
        assert np.array_equal(r1.selected, r2.selected)
        assert np.allclose(r1.logits[np.isfinite(r1.logits)], r2.logits[np.isfinite(r2.logits)],
                           rtol=0, atol=1e-10)


def test_first_step_after_refresh_is_exact(tiny_model):
    pr, t, a = _inputs(alpha_max=16.0)
    dec = OracleDecoder(tiny_model, 32, 64, 16, cache="dual", rule="threshold", tau=0.9)
    nc = OracleDecoder(tiny_model, 32, 64, 16, cache="none", rule="threshold", tau=0.9)
    st = dec.decode(pr[0], t[0], a[0])
    # replay: at each block start the canvas equals the decode's canvas then
    canvas = np.concatenate([pr[0], np.full(64, TINY.mask_id, np.int32)])
    for j in range(4):
        s0 = dec.new_state(pr[0], t[0], a[0])
        s0.canvas[:] = canvas
        dec.refresh(s0)
        c1, y1, cf1, _ = dec.evaluate(s0, j)
        s1 = nc.new_state(pr[0], t[0], a[0])
        s1.canvas[:] = canvas
        c2, y2, cf2, _ = nc.evaluate(s1, j)
        assert np.array_equal(c1, c2) and np.array_equal(y1, y2)
        assert np.allclose(cf1, cf2, rtol=1e-12)
        s, e = dec.block_range(j)
        canvas[s:e] = st.canvas[s:e]


def test_block_causal_commit_pass_is_exact_cache(tiny_model):
    pr, t, a = _inputs(alpha_max=16.0)
    dec = OracleDecoder(tiny_model, 32, 64, 16, cache="block_causal")
    st = dec.decode(pr[0], t[0], a[0])
    # one block-causal pass over the final sequence gives the same K/V
    ref = dec.new_state(pr[0], t[0], a[0])
    ref.canvas[:] = st.canvas
    rows = np.arange(dec.N)
    tiny_model.forward_rows(ref.canvas, rows, ref.kv, dec.key_limit(rows))
    assert np.allclose(st.kv.k, ref.kv.k, atol=1e-12) and np.allclose(st.kv.v, ref.kv.v, atol=1e-12)


def test_block_causal_never_sees_later_blocks(tiny_model):
    pr, t, a = _inputs(alpha_max=16.0)
    dec = OracleDecoder(tiny_model, 32, 64, 16, cache="block_causal")
    st1 = dec.decode(pr[0], t[0], a[0])
    # change the planted bias of the last block only: earlier blocks unchanged
    a2 = a.copy()
    a2[0, 48:] = 0
    st2 = dec.decode(pr[0], t[0], a2[0])
    assert np.array_equal(st1.canvas[:80], st2.canvas[:80])


def test_tiny_workload_decodes_with_fallback(tiny_model):
    w = workload("tiny")
    m = OracleModel(TINY, gen_weights(TINY, w.weight_seed))
    pr = gen_prompt(TINY, 1, w.prompt_len, w.prompt_seed)
    t, a = gen_bias(TINY, 1, w.gen_len, w.bias_seed, w.alpha_max)
    st = OracleDecoder(m, w.prompt_len, w.gen_len, w.block_len, w.cache, w.rule, w.tau).decode(pr[0], t[0], a[0])
    assert (st.canvas[:32] == pr[0]).all() and (st.canvas != TINY.mask_id).all()
    assert 4 <= st.steps <= 64 and st.refreshes == 4
