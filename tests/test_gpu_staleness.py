"""GPU parity of the cached-vs-fresh diagnostics (dllm_staleness, reading
notes sec. 14 / Algorithm 4) against the float64 oracle, through the C ABI:
the GPU decodes a few DualCache / PrefixCache steps, the oracle follows in
lock-step with its own cache, then both run the diagnostic on the same state.
Also: the diagnostic leaves the decode unchanged."""
import numpy as np
import pytest
import torch

from oracle import OracleDecoder, OracleModel, staleness
from workloads import LLADA_8B, TINY, gen_bias, gen_prompt, gen_tensor, gen_weights, tensor_names

from .parity import Tol, top2_gap

pytestmark = pytest.mark.gpu


def _lockstep(eng, om, shape, cache, P, L, B, steps, seed, alpha_max):
    """GPU decode of `steps` steps of block 0 with the oracle following;
    returns (engine canvas, cfg, oracle decoder, oracle state)."""
    from diffusion_lm_decoding_amd.engine import Engine
    pr = gen_prompt(shape, 1, P, seed)
    t, a = gen_bias(shape, 1, L, seed + 1, alpha_max)
    cfg = Engine.decode_cfg(1, P, L, B, cache=cache, rule="threshold", tau=0.9)
    cv = eng.canvas(pr, t, a, L)
    dec = OracleDecoder(om, P, L, B, cache=cache, rule="threshold", tau=0.9)
    st = dec.new_state(pr[0], t[0], a[0])
    eng.begin(cv, cfg)
    eng.refresh(cv, cfg, 0)
    dec.refresh(st)
    for _ in range(steps):
        st.canvas[:] = cv.tokens.cpu().numpy()[0]
        dec.evaluate(st, 0)          # the oracle's cache follows the step's recomputed rows
        eng.step(cv, cfg, 0)
    st.canvas[:] = cv.tokens.cpu().numpy()[0]
    return cv, cfg, dec, st


def _compare(g, o, P, B, conf_tol, cos_tol, gap_ok):
    cand = o["cand"]
    rows = cand - P
    for kind in ("cached", "fresh"):
        gc = g[f"conf_{kind}"].cpu().numpy()[rows].astype(np.float64)
        gt = g[f"tok_{kind}"].cpu().numpy()[rows]
        assert np.abs(gc - o[f"conf_{kind}"]).max() <= conf_tol, kind
        bad = np.nonzero(gt != o[f"tok_{kind}"])[0]
        assert all(gap_ok(kind, i) for i in bad), (kind, bad)
    # committed rows report -1
    done = np.setdiff1d(np.arange(B), rows)
    assert (g["conf_cached"].cpu().numpy()[done] == -1).all() and (g["tok_fresh"].cpu().numpy()[done] == -1).all()
    for kind in ("k_cos", "v_cos"):
        gk = g[kind].cpu().numpy()[:, 0, :].astype(np.float64)
        assert np.abs(gk - o[kind]).max() <= cos_tol, (kind, np.abs(gk - o[kind]).max())


@pytest.fixture(scope="module")
def tiny_engines():
    from diffusion_lm_decoding_amd.engine import Engine
    w32 = gen_weights(TINY, seed=0, gain_jitter=0.1)
    bshape = TINY.__class__(**{**TINY.__dict__, "dtype": "bf16", "name": "tiny_bf16"})
    wbf = gen_weights(bshape, seed=0, gain_jitter=0.1)
    e32 = Engine(TINY, w32, max_batch=2, max_seq=128)
    ebf = Engine(bshape, wbf, max_batch=2, max_seq=128)
    yield {"f32": (e32, OracleModel(TINY, w32)), "bf16": (ebf, OracleModel(bshape, wbf))}
    e32.close()
    ebf.close()


@pytest.mark.parametrize("cache", ["dual", "prefix"])
@pytest.mark.parametrize("steps", [0, 3])
def test_tiny_f32_staleness_matches_oracle(tiny_engines, cache, steps):
    eng, om = tiny_engines["f32"]
    cv, cfg, dec, st = _lockstep(eng, om, TINY, cache, 32, 64, 16, steps, seed=91, alpha_max=16.0)
    g = eng.staleness(cv, cfg, 0)
    o = staleness(dec, st, 0)
    _compare(g, o, 32, 16, conf_tol=1e-5, cos_tol=1e-5, gap_ok=lambda kind, i: False)
    if steps == 0:
        assert np.abs(g["k_cos"].cpu().numpy() - 1).max() < 1e-5


def test_tiny_bf16_staleness_matches_oracle(tiny_engines):
    eng, om = tiny_engines["bf16"]
    cv, cfg, dec, st = _lockstep(eng, om, TINY, "dual", 40, 48, 16, 3, seed=93, alpha_max=16.0)
    g = eng.staleness(cv, cfg, 0)
    o = staleness(dec, st, 0)
    gaps = {k: top2_gap(o[f"logits_{k}"]) for k in ("cached", "fresh")}
    _compare(g, o, 40, 16, conf_tol=1e-2, cos_tol=2e-3,
             gap_ok=lambda kind, i: gaps[kind][i] <= Tol(fp32=False).top2_gap)


def test_staleness_leaves_the_decode_unchanged(tiny_engines):
    """Decode with a diagnostic call after every step equals the plain decode."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, _ = tiny_engines["f32"]
    pr = gen_prompt(TINY, 2, 32, 95)
    t, a = gen_bias(TINY, 2, 64, 96, 16.0)
    cfg = Engine.decode_cfg(2, 32, 64, 16, cache="dual")
    ref = eng.canvas(pr, t, a, 64)
    eng.decode(ref, cfg)
    cv = eng.canvas(pr, t, a, 64)
    eng.begin(cv, cfg)
    for j in range(4):
        eng.refresh(cv, cfg, 0)
        while (cv.tokens[:, 32 + 16 * j:48 + 16 * j] == TINY.mask_id).any().item():
            eng.staleness(cv, cfg, j)
            eng.step(cv, cfg, j)
    assert np.array_equal(cv.tokens.cpu().numpy(), ref.tokens.cpu().numpy())
    assert np.array_equal(cv.commit_step.cpu().numpy(), ref.commit_step.cpu().numpy())


@pytest.mark.timeout(900)
def test_8b_staleness_matches_oracle():
    """LLaDA-8B shape, P 128 / L 128 / B 32, DualCache after 2 steps."""
    from diffusion_lm_decoding_amd.engine import Engine
    host = {n: gen_tensor(LLADA_8B, n, 0) for n, _ in tensor_names(LLADA_8B)}
    eng = Engine(LLADA_8B, host, max_batch=1, max_seq=256)
    om = OracleModel(LLADA_8B, host)
    om.materialize()
    try:
        cv, cfg, dec, st = _lockstep(eng, om, LLADA_8B, "dual", 128, 128, 32, 2, seed=3001, alpha_max=24.0)
        g = eng.staleness(cv, cfg, 0)
        o = staleness(dec, st, 0)
        # token disagreements only where the oracle's top-2 probability gap is small
        gaps = {k: top2_gap(o[f"logits_{k}"]) for k in ("cached", "fresh")}

        def gap_ok(kind, i):
            return gaps[kind][i] <= Tol(fp32=False).top2_gap
        _compare(g, o, 128, 32, conf_tol=1e-2, cos_tol=2e-3, gap_ok=gap_ok)
        kc = g["k_cos"].cpu().numpy()
        print(f"8B staleness: agree cached/fresh "
              f"{(g['tok_cached'] == g['tok_fresh']).float().mean().item():.3f}, "
              f"k_cos min {kc.min():.4f} mean {kc.mean():.4f}", flush=True)
    finally:
        eng.close()


def test_sweep_by_age(tiny_engines):
    """The sweep probes every step; at age 0 (right after a refresh) the cached
    and fresh evaluations agree and the cache equals the fresh K/V."""
    from diffusion_lm_decoding_amd.diagnostics import by_age, staleness_sweep
    from diffusion_lm_decoding_amd.engine import Engine
    eng, _ = tiny_engines["f32"]
    pr = gen_prompt(TINY, 1, 32, 97)
    t, a = gen_bias(TINY, 1, 64, 98, 8.0)
    cfg = Engine.decode_cfg(1, 32, 64, 16, cache="dual")
    cv = eng.canvas(pr, t, a, 64)
    recs = staleness_sweep(eng, cv, cfg)
    assert len(recs) == 64 and (cv.tokens.cpu().numpy()[0, 32:] != TINY.mask_id).all()
    for r in recs:
        if r["age"] == 0:
            assert r["argmax_agree"] == 1.0 and r["conf_shift_max"] < 1e-5
            assert min(r["k_cos_cached_by_layer"]) > 1 - 1e-5
    ages = by_age(recs)
    assert ages[0]["age"] == 0 and ages[-1]["age"] == 15
