"""GPU edge cases through the C ABI on the two-layer model, against the float64
oracle: ragged sizes (no row, key or block count a multiple of 16), degenerate
blocks (one position per block; one block for the whole answer), the largest
batch and canvas a context was created for, and argument errors that must be
rejected before any device work."""
import numpy as np
import pytest

from oracle import OracleDecoder, OracleModel
from workloads import TINY, gen_bias, gen_prompt, gen_weights

from .parity import Tol, replay

pytestmark = pytest.mark.gpu

MAX_BATCH, MAX_SEQ = 4, 128


@pytest.fixture(scope="module")
def engines():
    from diffusion_lm_decoding_amd.engine import Engine
    w32 = gen_weights(TINY, seed=0, gain_jitter=0.1)
    bshape = TINY.__class__(**{**TINY.__dict__, "dtype": "bf16", "name": "tiny_bf16"})
    wbf = gen_weights(bshape, seed=0, gain_jitter=0.1)
    e32 = Engine(TINY, w32, max_batch=MAX_BATCH, max_seq=MAX_SEQ)
    ebf = Engine(bshape, wbf, max_batch=MAX_BATCH, max_seq=MAX_SEQ)
    yield {"f32": (e32, OracleModel(TINY, w32)), "bf16": (ebf, OracleModel(bshape, wbf))}
    e32.close()
    ebf.close()


def _inputs(batch, P, L, seed, alpha_max):
    pr = gen_prompt(TINY, batch, P, seed)
    t, a = gen_bias(TINY, batch, L, seed + 1, alpha_max)
    return pr, t, a


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cache", ["dual", "prefix", "none", "block_causal"])
def test_ragged_sizes_lockstep(engines, dtype, cache):
    """Batch 3, prompt 13, answer 21 in blocks of 7: 21-row steps (two
    partly filled 16-row tiles), key counts 13..34, a last key tile of 2."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = engines[dtype]
    pr, t, a = _inputs(3, 13, 21, seed=401, alpha_max=16.0)
    cfg = Engine.decode_cfg(3, 13, 21, 7, cache=cache)
    cv = eng.canvas(pr, t, a, 21)
    fp32 = dtype == "f32"
    rep = replay(eng, cv, cfg, om, pr, t, a, cache, "threshold", tol=Tol(fp32=fp32), seq=2)
    print(f"{dtype}/{cache}: {rep.summary()}", flush=True)
    assert not rep.bad, rep.bad[:5]
    assert rep.steps >= 3
    if fp32:
        assert rep.max_logit_err < 1e-4
    else:
        assert rep.max_logit_err < 5e-2 and rep.max_conf_err < 1e-2


def _full_decode_matches(eng, om, pr, t, a, P, L, B, cache, rule="threshold", **kw):
    from diffusion_lm_decoding_amd.engine import Engine
    batch = pr.shape[0]
    cv = eng.canvas(pr, t, a, L)
    stats = eng.decode(cv, Engine.decode_cfg(batch, P, L, B, cache=cache, rule=rule, **kw))
    toks, cs = cv.tokens.cpu().numpy(), cv.commit_step.cpu().numpy()
    steps = []
    for b in range(batch):
        dec = OracleDecoder(om, P, L, B, cache=cache, rule=rule, **kw)
        st = dec.decode(pr[b], t[b], a[b])
        assert np.array_equal(toks[b], st.canvas), f"sequence {b}: tokens differ"
        for k, rec in enumerate(st.records):
            assert (cs[b, rec.selected - P] == k).all(), f"sequence {b}: commit step {k} differs"
        steps.append(st.steps)
    assert stats.committed == batch * L and (toks[:, P:] != TINY.mask_id).all()
    assert stats.max_seq_steps == max(steps)
    return stats


@pytest.mark.parametrize("cache", ["dual", "prefix", "none", "block_causal"])
def test_one_position_blocks(engines, cache):
    """Blocks of one position: every block takes exactly one step."""
    eng, om = engines["f32"]
    pr, t, a = _inputs(2, 5, 8, seed=411, alpha_max=8.0)
    stats = _full_decode_matches(eng, om, pr, t, a, 5, 8, 1, cache)
    assert stats.max_seq_steps == 8


@pytest.mark.parametrize("cache", ["dual", "prefix", "none"])
def test_single_block_answer(engines, cache):
    """One block spans the whole answer (24 positions, prompt 9)."""
    eng, om = engines["f32"]
    pr, t, a = _inputs(2, 9, 24, seed=421, alpha_max=16.0)
    stats = _full_decode_matches(eng, om, pr, t, a, 9, 24, 24, cache)
    expect_refreshes = {"dual": 1, "prefix": 1, "none": 0}[cache]
    assert stats.refreshes == expect_refreshes


@pytest.mark.parametrize("cache", ["dual", "block_causal"])
def test_largest_batch_and_canvas(engines, cache):
    """batch = max_batch (4) and prompt + answer = max_seq (62 + 66, blocks
    of 11): every sequence equals its own oracle decode."""
    eng, om = engines["f32"]
    pr, t, a = _inputs(MAX_BATCH, 62, 66, seed=431, alpha_max=16.0)
    _full_decode_matches(eng, om, pr, t, a, 62, 66, 11, cache)


def test_argument_errors_rejected(engines):
    """Invalid configurations fail with DLLM_ERR_ARG before any device work,
    and the context still decodes afterwards."""
    from diffusion_lm_decoding_amd import _lib as L
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = engines["f32"]
    pr, t, a = _inputs(1, 32, 64, seed=441, alpha_max=8.0)
    cv = eng.canvas(pr, t, a, 64)
    bad = [
        dict(batch=0), dict(batch=MAX_BATCH + 1), dict(prompt_len=0), dict(gen_len=0), dict(block_len=0),
        dict(gen_len=60), dict(prompt_len=MAX_SEQ - 63), dict(block_len=320, gen_len=320),
        dict(tau=0.0), dict(tau=1.5), dict(rule="factor", factor=0.0), dict(rule="topk", k=0),
        dict(rule="steps", k=0), dict(refresh_every=-1),
    ]
    for kw in bad:
        args = dict(batch=1, prompt_len=32, gen_len=64, block_len=16)
        args.update(kw)
        cfg = Engine.decode_cfg(**args)
        for call in (lambda: eng.decode(cv, cfg), lambda: eng.begin(cv, cfg), lambda: eng.refresh(cv, cfg, 0)):
            with pytest.raises(L.DllmError) as e:
                call()
            assert e.value.status == L.ERR_ARG, kw
    good = Engine.decode_cfg(1, 32, 64, 16)
    for j in (-1, 4):
        eng.begin(cv, good)
        with pytest.raises(L.DllmError) as e:
            eng.step(cv, good, j)
        assert e.value.status == L.ERR_ARG
    raw = Engine.decode_cfg(1, 32, 64, 16)
    for field, value in (("cache", 9), ("rule", 9)):
        setattr(raw, field, value)
        with pytest.raises(L.DllmError) as e:
            eng.decode(cv, raw)
        assert e.value.status == L.ERR_ARG
        raw = Engine.decode_cfg(1, 32, 64, 16)
    _full_decode_matches(eng, om, pr, t, a, 32, 64, 16, "dual")


@pytest.mark.parametrize("cache", ["dual", "prefix", "none", "block_causal"])
def test_masked_row_lm_head_full_decode(engines, cache):
    """Batch 4 x blocks of 32 = 128 block rows: the LM head runs only on the
    still-masked rows (gathered in row order).  Full decodes equal the
    oracle's tokens and commit steps per sequence."""
    eng, om = engines["f32"]
    pr, t, a = _inputs(4, 16, 64, seed=451, alpha_max=16.0)
    _full_decode_matches(eng, om, pr, t, a, 16, 64, 32, cache)


@pytest.mark.parametrize("cache", ["dual", "block_causal"])
def test_masked_row_lm_head_lockstep_bf16(engines, cache):
    """The same gathered LM head in bf16, lock-step: logits of the masked rows
    of partly committed blocks against the oracle."""
    from diffusion_lm_decoding_amd.engine import Engine
    eng, om = engines["bf16"]
    pr, t, a = _inputs(4, 16, 64, seed=461, alpha_max=16.0)
    cfg = Engine.decode_cfg(4, 16, 64, 32, cache=cache)
    cv = eng.canvas(pr, t, a, 64)
    rep = replay(eng, cv, cfg, om, pr, t, a, cache, "threshold", tol=Tol(fp32=False), seq=3, max_steps=12)
    print(f"bf16/{cache}: {rep.summary()}", flush=True)
    assert not rep.bad, rep.bad[:5]
    assert rep.steps >= 3 and rep.max_logit_err < 5e-2
