"""GPU parity on the two-layer model (fp32 and bf16), through the C ABI,
against the float64 oracle: independent full decodes and lock-step replays
over every cache mode and selection rule."""
import numpy as np
import pytest
import torch

from oracle import OracleDecoder, OracleModel
from workloads import TINY, gen_bias, gen_prompt, gen_weights, workload

from .parity import Tol, replay

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def engines():
    from diffusion_lm_decoding_amd.engine import Engine
    w32 = gen_weights(TINY, seed=0, gain_jitter=0.1)
    bshape = TINY.__class__(**{**TINY.__dict__, "dtype": "bf16", "name": "tiny_bf16"})
    wbf = gen_weights(bshape, seed=0, gain_jitter=0.1)
    e32 = Engine(TINY, w32, max_batch=4, max_seq=128)
    ebf = Engine(bshape, wbf, max_batch=4, max_seq=128)
    yield {"f32": (e32, OracleModel(TINY, w32)), "bf16": (ebf, OracleModel(bshape, wbf))}
    e32.close()
    ebf.close()


def _inputs(batch, P, L, seed, alpha_max):
    pr = gen_prompt(TINY, batch, P, seed)
    t, a = gen_bias(TINY, batch, L, seed + 1, alpha_max)
    return pr, t, a


def test_tiny_workload_full_decode_matches_oracle():
    """The tiny fp32 workload: tokens and per-position commit steps identical."""
    from diffusion_lm_decoding_amd.engine import Engine
    w = workload("tiny")
    weights = gen_weights(TINY, w.weight_seed)
    eng = Engine(TINY, weights, max_batch=1, max_seq=w.seq_len)
    pr = gen_prompt(TINY, 1, w.prompt_len, w.prompt_seed)
    t, a = gen_bias(TINY, 1, w.gen_len, w.bias_seed, w.alpha_max)
    cv = eng.canvas(pr, t, a, w.gen_len)
    stats = eng.decode(cv, Engine.cfg_from_workload(w))
    dec = OracleDecoder(OracleModel(TINY, weights), w.prompt_len, w.gen_len, w.block_len, w.cache, w.rule, w.tau)
    st = dec.decode(pr[0], t[0], a[0])
    got = cv.tokens.cpu().numpy()[0]
    assert np.array_equal(got, st.canvas)
    assert stats.steps == st.steps and stats.refreshes == st.refreshes
    cs = cv.commit_step.cpu().numpy()[0]
    for k, rec in enumerate(st.records):
        assert (cs[rec.selected - w.prompt_len] == k).all()
    eng.close()


@pytest.mark.parametrize("cache", ["dual", "prefix", "none", "block_causal"])
@pytest.mark.parametrize("rule,kw", [("threshold", dict(tau=0.9)), ("factor", dict(factor=1.0)),
                                     ("factor", dict(factor=2.0)), ("topk", dict(k=4)), ("budget", {}),
                                     ("steps", dict(k=5))])
def test_f32_lockstep(engines, cache, rule, kw):
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = engines["f32"]
    pr, t, a = _inputs(2, 32, 64, seed=21, alpha_max=16.0)
    cfg = Engine.decode_cfg(2, 32, 64, 16, cache=cache, rule=rule, **kw)
    cv = eng.canvas(pr, t, a, 64)
    rep = replay(eng, cv, cfg, om, pr, t, a, cache, rule, tol=Tol(fp32=True), seq=1, **kw)
    assert not rep.bad, rep.bad[:5]
    assert rep.steps >= 4 and rep.max_logit_err < 1e-4


@pytest.mark.parametrize("cache", ["dual", "prefix", "none", "block_causal"])
@pytest.mark.parametrize("rule,kw", [("threshold", dict(tau=0.9)), ("factor", dict(factor=1.0)),
                                     ("budget", {})])
def test_bf16_lockstep(engines, cache, rule, kw):
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = engines["bf16"]
    pr, t, a = _inputs(3, 40, 48, seed=31, alpha_max=16.0)
    cfg = Engine.decode_cfg(3, 40, 48, 16, cache=cache, rule=rule, **kw)
    cv = eng.canvas(pr, t, a, 48)
    rep = replay(eng, cv, cfg, om, pr, t, a, cache, rule, tol=Tol(fp32=False), seq=2, **kw)
    print(f"bf16 {cache}/{rule}: {rep.summary()}", flush=True)
    assert not rep.bad, rep.bad[:5]
    assert rep.max_logit_err < 5e-2 and rep.max_conf_err < 1e-2


@pytest.mark.parametrize("cache", ["dual", "prefix", "none"])
def test_bf16_lockstep_wide_attention(engines, cache):
    """128-row forwards (refresh and no-cache steps) take the wide-query
    attention kernel (4 query blocks share each key tile)."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = engines["bf16"]
    pr, t, a = _inputs(2, 64, 64, seed=33, alpha_max=16.0)
    cfg = Engine.decode_cfg(2, 64, 64, 16, cache=cache)
    cv = eng.canvas(pr, t, a, 64)
    rep = replay(eng, cv, cfg, om, pr, t, a, cache, "threshold", tol=Tol(fp32=False), seq=1, max_steps=12)
    assert not rep.bad, rep.bad[:5]
    assert rep.max_logit_err < 5e-2 and rep.max_conf_err < 1e-2


def test_batch_equals_single_runs(engines):
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = engines["f32"]
    pr, t, a = _inputs(4, 32, 64, seed=41, alpha_max=16.0)
    cfg = Engine.decode_cfg(4, 32, 64, 16, cache="dual")
    cv = eng.canvas(pr, t, a, 64)
    eng.decode(cv, cfg)
    full = cv.tokens.cpu().numpy()
    for b in range(4):
        c1 = eng.canvas(pr[b:b + 1], t[b:b + 1], a[b:b + 1], 64)
        eng.decode(c1, Engine.decode_cfg(1, 32, 64, 16, cache="dual"))
        assert np.array_equal(c1.tokens.cpu().numpy()[0], full[b])


def test_decode_is_deterministic(engines):
    from diffusion_lm_decoding_amd.engine import Engine
    eng, _ = engines["bf16"]
    pr, t, a = _inputs(2, 32, 64, seed=51, alpha_max=16.0)
    cfg = Engine.decode_cfg(2, 32, 64, 16, cache="dual")
    outs = []
    for _ in range(2):
        cv = eng.canvas(pr, t, a, 64)
        eng.decode(cv, cfg)
        outs.append((cv.tokens.cpu().numpy(), cv.commit_step.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_refresh_every_step_equals_uncached_on_gpu(engines):
    from diffusion_lm_decoding_amd.engine import Engine
    eng, _ = engines["f32"]
    pr, t, a = _inputs(1, 32, 64, seed=61, alpha_max=16.0)
    c1 = eng.canvas(pr, t, a, 64)
    eng.decode(c1, Engine.decode_cfg(1, 32, 64, 16, cache="none"))
    c2 = eng.canvas(pr, t, a, 64)
    eng.decode(c2, Engine.decode_cfg(1, 32, 64, 16, cache="dual", refresh_every=1))
    assert np.array_equal(c1.tokens.cpu().numpy(), c2.tokens.cpu().numpy())
    assert np.array_equal(c1.commit_step.cpu().numpy(), c2.commit_step.cpu().numpy())


@pytest.mark.parametrize("cache", ["dual", "prefix"])
@pytest.mark.parametrize("r", [2, 4])
def test_refresh_every_full_decode_matches_oracle(engines, cache, r):
    """Refresh interval r inside a block (reading notes sec. 11): whole
    dllm_decode runs (batch 2) give the oracle's tokens, per-position commit
    steps and, per sequence, step counts; the batch-1 refresh count is the
    oracle's."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = engines["f32"]
    pr, t, a = _inputs(2, 32, 64, seed=63 + r, alpha_max=16.0)
    cv = eng.canvas(pr, t, a, 64)
    stats = eng.decode(cv, Engine.decode_cfg(2, 32, 64, 16, cache=cache, refresh_every=r))
    toks, cs = cv.tokens.cpu().numpy(), cv.commit_step.cpu().numpy()
    dec = OracleDecoder(om, 32, 64, 16, cache=cache, refresh_every=r)
    steps = []
    for b in range(2):
        st = dec.decode(pr[b], t[b], a[b])
        assert np.array_equal(toks[b], st.canvas), f"sequence {b}"
        for k, rec in enumerate(st.records):
            assert (cs[b, rec.selected - 32] == k).all()
        steps.append(st.steps)
    assert stats.max_seq_steps == max(steps)
    c1 = eng.canvas(pr[:1], t[:1], a[:1], 64)
    s1 = eng.decode(c1, Engine.decode_cfg(1, 32, 64, 16, cache=cache, refresh_every=r))
    o1 = dec.decode(pr[0], t[0], a[0])
    assert s1.refreshes == o1.refreshes and s1.steps == o1.steps
    assert o1.refreshes > 4             # the interval fired inside blocks


@pytest.mark.parametrize("cache,r", [("dual", 0), ("prefix", 0), ("dual", 3), ("prefix", 5)])
def test_decode_shares_refresh_and_step_forward(engines, cache, r):
    """dllm_decode evaluates the step after each refresh from the refresh's
    own forward over the whole canvas; a loop driven through
    dllm_refresh_cache + dllm_block_step (a second forward, over the block or
    the suffix) commits the same tokens at the same steps (fp32), with the
    same step and refresh counts."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, _ = engines["f32"]
    pr, t, a = _inputs(2, 32, 64, seed=91 + r, alpha_max=16.0)
    cfg = Engine.decode_cfg(2, 32, 64, 16, cache=cache, refresh_every=r)
    c1 = eng.canvas(pr, t, a, 64)
    st = eng.decode(c1, cfg)
    c2 = eng.canvas(pr, t, a, 64)
    eng.begin(c2, cfg)
    steps = refreshes = 0
    for j in range(4):
        n = 0
        while True:
            if n == 0 or (r and n % r == 0):
                eng.refresh(c2, cfg, 0)
                refreshes += 1
            _, done, *_ = eng.step(c2, cfg, j)
            steps += 1
            n += 1
            if np.asarray(done).all():
                break
            assert n < 16, "block outlived its step bound"
    assert np.array_equal(c1.tokens.cpu().numpy(), c2.tokens.cpu().numpy())
    assert np.array_equal(c1.commit_step.cpu().numpy(), c2.commit_step.cpu().numpy())
    assert st.steps == steps and st.refreshes == refreshes
    assert steps > refreshes            # steps from the cache ran too


@pytest.mark.parametrize("cache", ["dual", "prefix"])
@pytest.mark.parametrize("r", [2, 4])
def test_refresh_every_lockstep_f32(engines, cache, r):
    """The same interval in lock-step: every step's logits within 1e-4 of the
    row scale and every decision identical (fp32: no exemption)."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = engines["f32"]
    pr, t, a = _inputs(2, 32, 64, seed=73 + r, alpha_max=16.0)
    cfg = Engine.decode_cfg(2, 32, 64, 16, cache=cache, refresh_every=r)
    cv = eng.canvas(pr, t, a, 64)
    rep = replay(eng, cv, cfg, om, pr, t, a, cache, "threshold", tol=Tol(fp32=True), seq=1, refresh_every=r)
    assert not rep.bad, rep.bad[:5]
    assert rep.steps >= 8 and rep.max_logit_err < 1e-4 and rep.exempt == 0


def test_schedules_on_gpu(engines):
    from diffusion_lm_decoding_amd.engine import Engine
    eng, _ = engines["f32"]
    pr, t, _ = _inputs(1, 32, 64, seed=71, alpha_max=8.0)
    a = np.full((1, 64), 30.0, np.float32)
    cv = eng.canvas(pr, t, a, 64)
    st = eng.decode(cv, Engine.decode_cfg(1, 32, 64, 16, cache="dual"))
    assert st.steps == 4 and np.array_equal(cv.tokens.cpu().numpy()[0, 32:], t[0])
    for k, expect in ((1, 64), (4, 16)):
        cv = eng.canvas(pr, t, a * 0, 64)
        st = eng.decode(cv, Engine.decode_cfg(1, 32, 64, 16, cache="dual", rule="topk", k=k))
        assert st.steps == expect and st.committed == 64
    # tau = 1: one position per step while no confidence rounds to 1.0 in fp32
    cv = eng.canvas(pr, t, a * 0 + 8.0, 64)
    st = eng.decode(cv, Engine.decode_cfg(1, 32, 64, 16, cache="dual", tau=1.0))
    assert st.steps == 64


@pytest.mark.parametrize("block,steps", [(64, 10), (16, 20)])
def test_fixed_steps_sampler_full_decode(engines, block, steps):
    """LLaDA's sampler: unblocked (one block, no cache) and with more steps
    than block positions (steps that commit nothing): tokens, commit steps
    and step counts identical to the oracle."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = engines["f32"]
    pr, t, a = _inputs(1, 32, 64, seed=81, alpha_max=8.0)
    cache = "none" if block == 64 else "dual"
    cv = eng.canvas(pr, t, a, 64)
    stats = eng.decode(cv, Engine.decode_cfg(1, 32, 64, block, cache=cache, rule="steps", k=steps))
    dec = OracleDecoder(om, 32, 64, block, cache=cache, rule="steps", k=steps)
    st = dec.decode(pr[0], t[0], a[0])
    assert np.array_equal(cv.tokens.cpu().numpy()[0], st.canvas)
    assert stats.steps == st.steps == steps * (64 // block)
    cs = cv.commit_step.cpu().numpy()[0]
    for k, rec in enumerate(st.records):
        assert (cs[rec.selected - 32] == k).all()


def test_bad_canvas_rejected(engines):
    from diffusion_lm_decoding_amd import _lib as L
    from diffusion_lm_decoding_amd.engine import Engine
    eng, _ = engines["f32"]
    pr, t, a = _inputs(1, 32, 64, seed=81, alpha_max=8.0)
    pr[0, 3] = TINY.mask_id
    cv = eng.canvas(pr, t, a, 64)
    with pytest.raises(L.DllmError) as e:
        eng.decode(cv, Engine.decode_cfg(1, 32, 64, 16))
    assert e.value.status == L.ERR_ARG
    with pytest.raises(L.DllmError):
        eng.decode(cv, Engine.decode_cfg(1, 32, 60, 16))


def test_nan_bias_reports_numeric_error_and_leaves_canvas(engines):
    from diffusion_lm_decoding_amd import _lib as L
    from diffusion_lm_decoding_amd.engine import Engine
    eng, _ = engines["f32"]
    pr, t, a = _inputs(1, 32, 64, seed=91, alpha_max=8.0)
    a[0, 5] = np.nan
    cv = eng.canvas(pr, t, a, 64)
    cfg = Engine.decode_cfg(1, 32, 64, 16)
    eng.refresh(cv, cfg)
    before = cv.tokens.clone()
    with pytest.raises(L.DllmError) as e:
        eng.step(cv, cfg, 0)
    assert e.value.status == L.ERR_NUMERIC
    assert torch.equal(before, cv.tokens)


@pytest.mark.parametrize("vocab", [8192, 65536])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grouped_head_partials_lockstep(vocab, dtype):
    """Vocabularies whose LM-head launch puts 2 (8192) or 4 (65536) vocabulary
    tiles in a workgroup: the workgroup combines its tiles' (max, sum,
    argmax) before the merge kernel.  Lock-step against the oracle."""
    from diffusion_lm_decoding_amd.engine import Engine
    shape = TINY.__class__(**{**TINY.__dict__, "vocab": vocab, "mask_id": vocab - 1, "dtype": dtype,
                              "name": f"tiny_v{vocab}_{dtype}"})
    w = gen_weights(shape, seed=5, gain_jitter=0.1)
    eng = Engine(shape, w, max_batch=2, max_seq=96)
    om = OracleModel(shape, w)
    pr = gen_prompt(shape, 2, 32, 71)
    t, a = gen_bias(shape, 2, 64, 72, 16.0)
    cfg = Engine.decode_cfg(2, 32, 64, 16, cache="dual", rule="threshold", tau=0.9)
    cv = eng.canvas(pr, t, a, 64)
    fp32 = dtype == "f32"
    rep = replay(eng, cv, cfg, om, pr, t, a, "dual", "threshold", tol=Tol(fp32=fp32), seq=1, tau=0.9)
    print(f"vocab {vocab} {dtype}: {rep.summary()}", flush=True)
    eng.close()
    assert not rep.bad, rep.bad[:5]
    assert rep.steps >= 4
    if fp32:
        assert rep.max_logit_err < 1e-4
    else:
        assert rep.max_logit_err < 5e-2 and rep.max_conf_err < 1e-2
