"""GPU parity at the LLaDA-8B shape (32 layers, d 4096, 32x128 heads, FFN
12288, vocab 126464, bf16) against the float64 oracle on sampled steps.

The oracle is expensive at this size (a 768-row refresh is ~12 TFLOP in
float64), so each test replays a few steps in lock-step: the oracle keeps
its own cache, refreshed at the same boundaries from the GPU's canvas, and
compares logits (5e-2 abs), confidences (1e-2 abs) and decisions (the GPU's
selection must be its rule on its own confidences; a difference from the
oracle is exempt only at the rule's cut, a token difference only with a top-2
probability gap <= 0.05; at most 1% of the decisions exempt).
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
    rep.check_exemptions()
    print(f"{what}: {rep.summary()}", flush=True)
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


def _cmp(rep, dec, eng, cv, cfg, st, j, seq, B, tag, k_in_block=0):
    """One GPU debug step on block j, compared for sequence `seq` with the
    oracle's evaluation of the same canvas from its own cache `st`."""
    s = dec.block_range(j)[0]
    before_all = cv.tokens.cpu().numpy()
    st.canvas[:] = before_all[seq]
    cand, y, c, l = dec.evaluate(st, j)
    _, _, gconf, gtok, glog = eng.step(cv, cfg, j, debug=True, debug_logits=True)
    after = cv.tokens.cpu().numpy()[seq]
    rows = seq * B + (cand - s)
    compare_step(rep, Tol(fp32=False), dec, cand, y, c, l, gconf.cpu().numpy()[rows].astype(np.float64),
                 gtok.cpu().numpy()[rows], glog.cpu().numpy()[rows].astype(np.float64), before_all[seq], after,
                 k_in_block, tag=tag)


def test_block_diffusion_full_size_two_blocks(big):
    """The block-diffusion workload at full size (batch 8, P 2048, L 1024,
    blocks of 256), sequence 0 against the oracle: the prompt pass, the first
    block-causal step of block 0, then (after the GPU finishes block 0 in
    every sequence) the commit pass of block 0 from the GPU's final block and
    the first step of block 1, whose keys [0, 2560) include that commit
    pass's K/V."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    w = workload("llada8b_blockdiff")
    pr = gen_prompt(LLADA_8B, w.batch, w.prompt_len, w.prompt_seed)
    t, a = gen_bias(LLADA_8B, w.batch, w.gen_len, w.bias_seed, w.alpha_max)
    cfg = Engine.cfg_from_workload(w)
    assert (cfg.batch, cfg.prompt_len, cfg.gen_len, cfg.block_len) == (8, 2048, 1024, 256)
    B, P = w.block_len, w.prompt_len
    cv = eng.canvas(pr, t, a, w.gen_len)
    dec = OracleDecoder(om, P, w.gen_len, B, cache="block_causal", rule=w.rule, tau=w.tau)
    st = dec.new_state(pr[0], t[0], a[0])
    rep = Report()
    eng.begin(cv, cfg)
    eng.refresh(cv, cfg, -1)
    dec.prefill(st)
    _cmp(rep, dec, eng, cv, cfg, st, 0, 0, B, "block 0, step 0")
    n = 1
    while (cv.tokens[:, P:P + B] == LLADA_8B.mask_id).any().item():
        eng.step(cv, cfg, 0)
        n += 1
        assert n <= B
    eng.refresh(cv, cfg, 0)                      # commit pass of block 0
    st.canvas[:] = cv.tokens[0].cpu().numpy()
    dec.commit_pass(st, 0)
    _cmp(rep, dec, eng, cv, cfg, st, 1, 0, B, "block 1, step 0")
    _check(rep, f"block diffusion, full size (block 0 took {n} steps)")
    assert rep.steps == 2


def test_benchmark_workload_all_blocks_sampled(big):
    """The benchmark workload itself (P 512, L 256, blocks of 32, DualCache,
    tau 0.9, alpha ~ U(0, 12)) decoded step by step on the GPU over all 8
    blocks.  At each block start both sides refresh from the GPU's canvas;
    the first two steps of every block and a seeded 10% of the later ones
    are compared, the oracle evaluating the GPU's canvas from its block-start
    cache: a DualCache step rewrites the block's K/V rows before any layer
    reads them, so this equals the oracle's own lock-step replay."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    w = workload("llada8b_p512_g256")
    pr = gen_prompt(LLADA_8B, 1, w.prompt_len, w.prompt_seed)
    t, a = gen_bias(LLADA_8B, 1, w.gen_len, w.bias_seed, w.alpha_max)
    cfg = Engine.cfg_from_workload(w)
    B, P = w.block_len, w.prompt_len
    cv = eng.canvas(pr, t, a, w.gen_len)
    dec = OracleDecoder(om, P, w.gen_len, B, cache=w.cache, rule=w.rule, tau=w.tau)
    st = dec.new_state(pr[0], t[0], a[0])
    rng = np.random.default_rng(20251)
    rep = Report()
    total = 0
    eng.begin(cv, cfg)
    for j in range(w.n_blocks):
        eng.refresh(cv, cfg, 0)
        st.canvas[:] = cv.tokens[0].cpu().numpy()
        dec.refresh(st)
        s, e = dec.block_range(j)
        k = 0
        while (cv.tokens[0, s:e] == LLADA_8B.mask_id).any().item():
            if k < 2 or rng.random() < 0.10:
                _cmp(rep, dec, eng, cv, cfg, st, j, 0, B, f"block {j}, step {k}")
            else:
                eng.step(cv, cfg, j)
            k += 1
            total += 1
            assert k <= B
    final = cv.tokens.cpu().numpy()[0]
    assert (final != LLADA_8B.mask_id).all() and total <= w.gen_len
    _check(rep, f"benchmark workload, all blocks ({rep.steps} of {total} steps compared)")
    assert rep.steps >= 2 * w.n_blocks


def test_long_canvas_uncached_step(big):
    """The long canvas (P 1024, L 1024) without a cache: one step over all
    2048 rows at block 16, on a canvas whose first 16 blocks hold the GPU's
    own DualCache decode and whose later blocks are masked again."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    w = workload("llada8b_p1024_g1024")
    pr = gen_prompt(LLADA_8B, 1, w.prompt_len, w.prompt_seed)
    t, a = gen_bias(LLADA_8B, 1, w.gen_len, w.bias_seed, w.alpha_max)
    cv = eng.canvas(pr, t, a, w.gen_len)
    eng.decode(cv, Engine.cfg_from_workload(w))
    j = 16
    P, B = w.prompt_len, w.block_len
    s = P + j * B
    cv.tokens[0, s:] = LLADA_8B.mask_id
    cfg = Engine.cfg_from_workload(w, cache="none")
    dec = OracleDecoder(om, P, w.gen_len, B, cache="none", rule=w.rule, tau=w.tau)
    st = dec.new_state(pr[0], t[0], a[0])
    rep = Report()
    _cmp(rep, dec, eng, cv, cfg, st, j, 0, B, "no cache, block 16")
    _check(rep, "long canvas, uncached step over 2048 rows")


def test_batch16_step_10(big):
    """The batch-16 workload (P 128, L 128, blocks of 32, alpha ~ U(0, 12)):
    ten plain DualCache steps of block 0, then the eleventh step compared for
    sequences 0 and 15, the oracle evaluating the GPU's canvas from its own
    refresh of the block-start canvas (cache age 10)."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    w = workload("llada8b_p128_g128")
    pr = gen_prompt(LLADA_8B, 16, 128, w.prompt_seed)
    t, a = gen_bias(LLADA_8B, 16, 128, w.bias_seed, w.alpha_max)
    cfg = Engine.cfg_from_workload(w)
    cv = eng.canvas(pr, t, a, 128)
    eng.begin(cv, cfg)
    eng.refresh(cv, cfg)
    start = cv.tokens.cpu().numpy()
    for _ in range(10):
        eng.step(cv, cfg, 0)
    before = cv.tokens.cpu().numpy()
    _, _, gconf, gtok, glog = eng.step(cv, cfg, 0, debug=True, debug_logits=True)
    after = cv.tokens.cpu().numpy()
    dec = OracleDecoder(om, 128, 128, 32, cache="dual", rule=w.rule, tau=w.tau)
    rep = Report()
    for b in (0, 15):
        assert (before[b, 128:160] == LLADA_8B.mask_id).any()
        st = dec.new_state(pr[b], t[b], a[b])
        st.canvas[:] = start[b]
        dec.refresh(st)
        st.canvas[:] = before[b]
        cand, y, c, l = dec.evaluate(st, 0)
        rows = b * 32 + (cand - 128)
        compare_step(rep, Tol(fp32=False), dec, cand, y, c, l, gconf.cpu().numpy()[rows].astype(np.float64),
                     gtok.cpu().numpy()[rows], glog.cpu().numpy()[rows].astype(np.float64), before[b], after[b],
                     tag=f"sequence {b}, step 10")
    _check(rep, "batch 16, step 10")


def test_refresh_every_4_lockstep(big):
    """Refresh interval 4 inside a block at the 8B shape (P 256, L 64,
    DualCache, alpha ~ U(0, 12): about one commit per step, so block 0 is
    still open at step 4): steps 0-5 of block 0 in lock-step, both sides
    refreshing before step 4."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = big
    pr, t, a = _inputs(1, 256, 64, seed=2501, alpha_max=12.0)
    cfg = Engine.decode_cfg(1, 256, 64, 32, cache="dual", refresh_every=4)
    cv = eng.canvas(pr, t, a, 64)
    _check(replay(eng, cv, cfg, om, pr, t, a, "dual", "threshold", tol=Tol(fp32=False), max_steps=6,
                  refresh_every=4), "refresh every 4 steps")


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
