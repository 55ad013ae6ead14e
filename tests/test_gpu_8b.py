"""GPU parity at the LLaDA-8B shape (32 layers, d 4096, 32x128 heads, FFN
12288, vocab 126464, bf16) against the float64 oracle on sampled steps.

The oracle is expensive at this size (a 768-row refresh is ~12 TFLOP in
float64), so each test replays a few steps in lock-step: the oracle keeps
its own cache, refreshed at the same boundaries from the GPU's canvas, and
compares logits (5e-2 abs), confidences (1e-2 abs) and decisions (exempt only
near tau, near a rank tie, or with a top-2 probability gap <= 0.05).
Workloads are those of the benchmark or reduced-length versions of them;
alpha_max 24 variants put a share of positions above tau so that the
threshold branch is exercised (alpha_max 12 decodes one token per step).
"""
import numpy as np
import pytest
import torch

from oracle import OracleDecoder, OracleModel
from workloads import LLADA_8B, gen_bias, gen_prompt, gen_tensor, tensor_names, workload

from .parity import Report, Tol, compare_step, replay

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

MAX_BATCH, MAX_SEQ = 16, 3072


@pytest.fixture(scope="module")
def big():
    from diffusion_lm_decoding_amd.engine import Engine
    host = {n: gen_tensor(LLADA_8B, n, 0) for n, _ in tensor_names(LLADA_8B)}
    eng = Engine(LLADA_8B, host, max_batch=MAX_BATCH, max_seq=MAX_SEQ)
    om = OracleModel(LLADA_8B, host)
    om.materialize()
    yield eng, om
    eng.close()


def _inputs(batch, P, L, seed, alpha_max):
    pr = gen_prompt(LLADA_8B, batch, P, seed)
    t, a = gen_bias(LLADA_8B, batch, L, seed + 1, alpha_max)
    return pr, t, a


def _check(rep, what):
    print(f"{what}: steps={rep.steps} max|dlogit|={rep.max_logit_err:.3g} max|dconf|={rep.max_conf_err:.3g} "
          f"decisions={rep.decisions} exempt={rep.exempt}", flush=True)
    assert not rep.bad, rep.bad[:5]
    assert rep.steps >= 1


def test_dual_threshold_lockstep_p512(big):
    """Benchmark shape (P 512, L 256, B 32), DualCache, tau 0.9, alpha ~ U(0, 24)."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    pr, t, a = _inputs(1, 512, 256, seed=2001, alpha_max=24.0)
    cfg = Engine.decode_cfg(1, 512, 256, 32, cache="dual", rule="threshold", tau=0.9)
    cv = eng.canvas(pr, t, a, 256)
    _check(replay(eng, cv, cfg, om, pr, t, a, "dual", "threshold", tau=0.9, tol=Tol(fp32=False),
                  max_steps=3), "dual/threshold")


def test_benchmark_workload_block3_exact_point(big):
    """The benchmark workload decoded end to end on the GPU; then the first
    step of block 3 (right after a refresh, where the cache is exact) is
    recomputed from the decode's own canvas and checked against the oracle."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    w = workload("llada8b_p512_g256")
    pr, (t, a) = (gen_prompt(LLADA_8B, 1, w.prompt_len, w.prompt_seed),
                  gen_bias(LLADA_8B, 1, w.gen_len, w.bias_seed, w.alpha_max))
    cfg = Engine.cfg_from_workload(w)
    cv = eng.canvas(pr, t, a, w.gen_len)
    st = eng.decode(cv, cfg)
    final = cv.tokens.cpu().numpy()[0]
    assert (final != LLADA_8B.mask_id).all() and st.committed == w.gen_len
    assert st.steps <= w.gen_len and st.refreshes == w.n_blocks
    j = 3
    s = w.prompt_len + j * w.block_len
    canvas = final.copy()
    canvas[s:] = LLADA_8B.mask_id
    cv.tokens[0] = torch.from_numpy(canvas).to(cv.tokens.device)
    eng.refresh(cv, cfg)
    _, _, gconf, gtok, glog = eng.step(cv, cfg, j, debug=True, debug_logits=True)
    dec = OracleDecoder(om, w.prompt_len, w.gen_len, w.block_len, cache="dual")
    ost = dec.new_state(pr[0], t[0], a[0])
    ost.canvas[:] = canvas
    dec.refresh(ost)
    cand, y, c, l = dec.evaluate(ost, j)
    before = canvas.copy()
    after = cv.tokens.cpu().numpy()[0]
    rows = cand - s
    rep = Report()
    compare_step(rep, Tol(fp32=False), dec, cand, y, c, l, gconf.cpu().numpy()[rows].astype(np.float64),
                 gtok.cpu().numpy()[rows], glog.cpu().numpy()[rows].astype(np.float64), before, after,
                 tag="block 3 first step")
    _check(rep, "benchmark workload, block 3")


@pytest.mark.parametrize("cache", ["prefix", "none"])
def test_prefix_and_uncached_lockstep(big, cache):
    """Reduced length (P 64, L 128, B 32, batch 2): PrefixCache recomputes 128
    rows and no-cache 192 rows per step (tiled projections, LM head on a
    subset of the rows)."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    pr, t, a = _inputs(2, 64, 128, seed=2101, alpha_max=24.0)
    cfg = Engine.decode_cfg(2, 64, 128, 32, cache=cache)
    cv = eng.canvas(pr, t, a, 128)
    _check(replay(eng, cv, cfg, om, pr, t, a, cache, "threshold", tol=Tol(fp32=False), seq=1,
                  max_steps=2), cache)


@pytest.mark.parametrize("f", [1.0, 2.0])
def test_factor_rule_lockstep(big, f):
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    pr, t, a = _inputs(1, 256, 64, seed=2201, alpha_max=24.0)
    cfg = Engine.decode_cfg(1, 256, 64, 32, cache="dual", rule="factor", factor=f)
    cv = eng.canvas(pr, t, a, 64)
    _check(replay(eng, cv, cfg, om, pr, t, a, "dual", "factor", factor=f, tol=Tol(fp32=False),
                  max_steps=3), f"factor {f}")


def test_batch16_first_step(big):
    """Batch-16 shape (P 128, L 128, B 32): the step has 512 rows (tiled
    projections and LM head); sequences 0 and 15 are checked."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    w = workload("llada8b_p128_g128", alpha_max=24.0)
    pr = gen_prompt(LLADA_8B, 16, 128, w.prompt_seed)
    t, a = gen_bias(LLADA_8B, 16, 128, w.bias_seed, w.alpha_max)
    cfg = Engine.cfg_from_workload(w)
    cv = eng.canvas(pr, t, a, 128)
    eng.refresh(cv, cfg)
    before = cv.tokens.cpu().numpy()
    _, _, gconf, gtok, glog = eng.step(cv, cfg, 0, debug=True, debug_logits=True)
    after = cv.tokens.cpu().numpy()
    rep = Report()
    dec = OracleDecoder(om, 128, 128, 32, cache="dual")
    for b in (0, 15):
        st = dec.new_state(pr[b], t[b], a[b])
        st.canvas[:] = before[b]
        dec.refresh(st)
        cand, y, c, l = dec.evaluate(st, 0)
        rows = b * 32 + (cand - 128)
        compare_step(rep, Tol(fp32=False), dec, cand, y, c, l, gconf.cpu().numpy()[rows].astype(np.float64),
                     gtok.cpu().numpy()[rows], glog.cpu().numpy()[rows].astype(np.float64), before[b], after[b],
                     tag=f"sequence {b}")
    _check(rep, "batch 16")


def test_block_causal_lockstep(big):
    """Block diffusion (blocks of 256, batch 2, P 256, L 512): prompt pass,
    block-causal steps of 512 rows, commit pass after the block."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    pr, t, a = _inputs(2, 256, 512, seed=2301, alpha_max=24.0)
    cfg = Engine.decode_cfg(2, 256, 512, 256, cache="block_causal")
    cv = eng.canvas(pr, t, a, 512)
    _check(replay(eng, cv, cfg, om, pr, t, a, "block_causal", "threshold", tol=Tol(fp32=False), seq=1,
                  max_steps=2), "block_causal")


def test_block_causal_sliced_attention_lockstep(big):
    """Block diffusion with blocks of 32 (batch 3, P 192, L 64, top-8 per
    step): the block steps' 32 queries attend 224 or 256 keys, which runs the
    output-dim-sliced attention (two slices per head at this batch) under the
    block-causal key limit; the last sequence is followed."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    pr, t, a = _inputs(3, 192, 64, seed=2311, alpha_max=24.0)
    cfg = Engine.decode_cfg(3, 192, 64, 32, cache="block_causal", rule="topk", k=8)
    cv = eng.canvas(pr, t, a, 64)
    _check(replay(eng, cv, cfg, om, pr, t, a, "block_causal", "topk", k=8, tol=Tol(fp32=False), seq=2,
                  max_steps=8), "block_causal, sliced attention")


def test_block_diffusion_full_size_first_step(big):
    """The block-diffusion workload at full size (batch 8, P 2048, L 1024,
    blocks of 256): the GPU's prompt pass over 8 x 2048 rows and first
    block-causal step over 8 x 256 rows; sequence 0 checked against the
    oracle's own prompt pass and step."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    w = workload("llada8b_blockdiff")
    pr = gen_prompt(LLADA_8B, w.batch, w.prompt_len, w.prompt_seed)
    t, a = gen_bias(LLADA_8B, w.batch, w.gen_len, w.bias_seed, w.alpha_max)
    cfg = Engine.cfg_from_workload(w)
    assert (cfg.batch, cfg.prompt_len, cfg.gen_len, cfg.block_len) == (8, 2048, 1024, 256)
    cv = eng.canvas(pr, t, a, w.gen_len)
    _check(replay(eng, cv, cfg, om, pr, t, a, "block_causal", w.rule, tau=w.tau, tol=Tol(fp32=False), seq=0,
                  max_steps=1), "block diffusion, full size")


def test_long_canvas_decode_properties(big):
    """Long-canvas shape (P 1024, L 1024, B 32), GPU only: every position is
    committed, each block finishes within B steps, and two decodes are
    bitwise identical (tokens and commit steps)."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, _ = big
    w = workload("llada8b_p1024_g1024")
    pr = gen_prompt(LLADA_8B, 1, w.prompt_len, w.prompt_seed)
    t, a = gen_bias(LLADA_8B, 1, w.gen_len, w.bias_seed, w.alpha_max)
    cfg = Engine.cfg_from_workload(w)
    outs = []
    for _ in range(2):
        cv = eng.canvas(pr, t, a, w.gen_len)
        st = eng.decode(cv, cfg)
        outs.append((cv.tokens.cpu().numpy(), cv.commit_step.cpu().numpy(), st.steps))
    toks, cs, steps = outs[0]
    assert (toks != LLADA_8B.mask_id).all() and steps <= w.gen_len
    assert (cs >= 0).all() and cs.max() == steps - 1
    for j in range(w.n_blocks):
        blk = cs[0, j * 32:(j + 1) * 32]
        assert blk.max() - blk.min() < 32
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("k", [1, 4])
def test_fixed_count_rules_lockstep(big, k):
    """Benchmark shape (P 512, L 256, B 32), DualCache, a fixed k tokens per
    step (top-k by confidence)."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    pr, t, a = _inputs(1, 512, 256, seed=2401 + k, alpha_max=12.0)
    cfg = Engine.decode_cfg(1, 512, 256, 32, cache="dual", rule="topk", k=k)
    cv = eng.canvas(pr, t, a, 256)
    _check(replay(eng, cv, cfg, om, pr, t, a, "dual", "topk", k=k, tol=Tol(fp32=False), max_steps=2),
           f"top-{k}")


@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_batch_1_to_8_first_step(big, batch):
    """Batch shapes below 16 (P 128, L 128, B 32): the step has batch x 32
    rows; the first and last sequences are checked.  Batches 1 and 2 run the
    attention as output-dim slices of one 32-dim tile, batch 4 of two."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    w = workload("llada8b_p128_g128", alpha_max=24.0)
    pr = gen_prompt(LLADA_8B, batch, 128, w.prompt_seed + batch)
    t, a = gen_bias(LLADA_8B, batch, 128, w.bias_seed + batch, w.alpha_max)
    cfg = Engine.decode_cfg(batch, 128, 128, 32, cache="dual")
    cv = eng.canvas(pr, t, a, 128)
    eng.refresh(cv, cfg)
    before = cv.tokens.cpu().numpy()
    _, _, gconf, gtok, glog = eng.step(cv, cfg, 0, debug=True, debug_logits=True)
    after = cv.tokens.cpu().numpy()
    rep = Report()
    dec = OracleDecoder(om, 128, 128, 32, cache="dual")
    for b in sorted({0, batch - 1}):
        st = dec.new_state(pr[b], t[b], a[b])
        st.canvas[:] = before[b]
        dec.refresh(st)
        cand, y, c, l = dec.evaluate(st, 0)
        rows = b * 32 + (cand - 128)
        compare_step(rep, Tol(fp32=False), dec, cand, y, c, l, gconf.cpu().numpy()[rows].astype(np.float64),
                     gtok.cpu().numpy()[rows], glog.cpu().numpy()[rows].astype(np.float64), before[b], after[b],
                     tag=f"batch {batch} sequence {b}")
    _check(rep, f"batch {batch}")


def test_long_canvas_block0_exact_point(big):
    """Long canvas (P 1024, L 1024, B 32), right after the first refresh:
    the DualCache step under threshold 0.9 and the factor rule with f = 1 and
    2, and the PrefixCache step (1024 recomputed rows), each from the same
    refreshed canvas, against one oracle refresh."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    w = workload("llada8b_p1024_g1024", alpha_max=24.0)
    pr = gen_prompt(LLADA_8B, 1, w.prompt_len, w.prompt_seed)
    t, a = gen_bias(LLADA_8B, 1, w.gen_len, w.bias_seed, w.alpha_max)
    P, Lg = w.prompt_len, w.gen_len
    cv = eng.canvas(pr, t, a, Lg)
    start = cv.tokens.clone()
    dual = OracleDecoder(om, P, Lg, 32, cache="dual")
    st = dual.new_state(pr[0], t[0], a[0])
    dual.refresh(st)
    cand, y, c, l = dual.evaluate(st, 0)
    rep = Report()
    for rule, kw in (("threshold", dict(tau=0.9)), ("factor", dict(factor=1.0)), ("factor", dict(factor=2.0))):
        cv.tokens.copy_(start)
        cfg = Engine.decode_cfg(1, P, Lg, 32, cache="dual", rule=rule, **kw)
        eng.begin(cv, cfg)
        eng.refresh(cv, cfg)
        before = cv.tokens.cpu().numpy()[0]
        _, _, gconf, gtok, glog = eng.step(cv, cfg, 0, debug=True, debug_logits=True)
        after = cv.tokens.cpu().numpy()[0]
        rows = cand - P
        dec = OracleDecoder(om, P, Lg, 32, cache="dual", rule=rule, **kw)
        compare_step(rep, Tol(fp32=False), dec, cand, y, c, l, gconf.cpu().numpy()[rows].astype(np.float64),
                     gtok.cpu().numpy()[rows], glog.cpu().numpy()[rows].astype(np.float64), before, after,
                     tag=f"dual {rule} {kw}")
    prefix = OracleDecoder(om, P, Lg, 32, cache="prefix")
    cand, y, c, l = prefix.evaluate(st, 0)
    cv.tokens.copy_(start)
    cfg = Engine.decode_cfg(1, P, Lg, 32, cache="prefix")
    eng.begin(cv, cfg)
    eng.refresh(cv, cfg)
    before = cv.tokens.cpu().numpy()[0]
    _, _, gconf, gtok, glog = eng.step(cv, cfg, 0, debug=True, debug_logits=True)
    after = cv.tokens.cpu().numpy()[0]
    rows = cand - P
    compare_step(rep, Tol(fp32=False), prefix, cand, y, c, l, gconf.cpu().numpy()[rows].astype(np.float64),
                 gtok.cpu().numpy()[rows], glog.cpu().numpy()[rows].astype(np.float64), before, after,
                 tag="prefix threshold")
    _check(rep, "long canvas, block 0")
    assert rep.steps == 4
