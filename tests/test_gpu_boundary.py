"""The C ABI's state, memory and range checks on the two-layer model: a step
or commit pass with no cache pass gives DLLM_ERR_STATE; a device-memory cap
gives DLLM_ERR_OOM at init; a bf16 weight outside the fp16 range the model is
computed in is rejected at init; an fp16 overflow in the activations gives
DLLM_ERR_NUMERIC with the canvas unchanged; and the decode statistics split
the device time as eq. (15) of the reading notes does (steps, refreshes,
selection).  Every error is raised from the host before or after complete
kernels; nothing here faults or stalls the GPU."""
import json

import numpy as np
import pytest
import torch

from workloads import TINY, gen_bias, gen_prompt, gen_weights, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

BF16 = TINY.__class__(**{**TINY.__dict__, "dtype": "bf16", "name": "tiny_bf16"})


def _inputs(batch=1, P=32, L=64, seed=501, alpha_max=8.0):
    pr = gen_prompt(TINY, batch, P, seed)
    t, a = gen_bias(TINY, batch, L, seed + 1, alpha_max)
    return pr, t, a


@pytest.fixture(scope="module")
def eng32():
    from diffusion_lm_decoding_amd.engine import Engine
    e = Engine(TINY, gen_weights(TINY, seed=0), max_batch=2, max_seq=128)
    yield e
    e.close()


@pytest.mark.parametrize("cache", ["dual", "prefix", "block_causal"])
def test_step_without_cache_pass_is_state_error(eng32, cache):
    from diffusion_lm_decoding_amd import _lib as L
    from diffusion_lm_decoding_amd.engine import Engine
    pr, t, a = _inputs()
    cv = eng32.canvas(pr, t, a, 64)
    cfg = Engine.decode_cfg(1, 32, 64, 16, cache=cache)
    eng32.begin(cv, cfg)
    before = cv.tokens.clone()
    with pytest.raises(L.DllmError) as e:
        eng32.step(cv, cfg, 0)
    assert e.value.status == L.ERR_STATE
    if cache == "block_causal":
        with pytest.raises(L.DllmError) as e:      # commit pass before the prompt pass
            eng32.refresh(cv, cfg, 0)
        assert e.value.status == L.ERR_STATE
        eng32.refresh(cv, cfg, -1)
    else:
        eng32.refresh(cv, cfg, 0)
    assert torch.equal(before, cv.tokens)
    # a cache pass over another geometry does not count
    other = Engine.decode_cfg(2, 32, 64, 16, cache=cache)
    cv2 = eng32.canvas(np.repeat(pr, 2, 0), np.repeat(t, 2, 0), np.repeat(a, 2, 0), 64)
    with pytest.raises(L.DllmError) as e:
        eng32.step(cv2, other, 0)
    assert e.value.status == L.ERR_STATE
    nc, _, _, _, _ = eng32.step(cv, cfg, 0)
    assert nc[0] >= 1


def test_uncached_step_needs_no_cache_pass(eng32):
    from diffusion_lm_decoding_amd.engine import Engine
    pr, t, a = _inputs()
    cv = eng32.canvas(pr, t, a, 64)
    cfg = Engine.decode_cfg(1, 32, 64, 16, cache="none")
    eng32.begin(cv, cfg)
    nc, _, _, _, _ = eng32.step(cv, cfg, 0)
    assert nc[0] >= 1


def test_device_limit_gives_oom_at_init():
    from diffusion_lm_decoding_amd import _lib as L
    from diffusion_lm_decoding_amd.engine import Engine
    w = gen_weights(TINY, seed=0)
    L.dllm_set_device_limit(1 << 20)          # the tiny context needs ~13 MB
    try:
        with pytest.raises(L.DllmError) as e:
            Engine(TINY, w, max_batch=1, max_seq=96)
        assert e.value.status == L.ERR_OOM
        assert "dllm_set_device_limit" in str(e.value)
    finally:
        L.dllm_set_device_limit(0)
    eng = Engine(TINY, w, max_batch=1, max_seq=96)
    pr, t, a = _inputs()
    cv = eng.canvas(pr, t, a, 64)
    st = eng.decode(cv, Engine.decode_cfg(1, 32, 64, 16))
    assert st.committed == 64
    eng.close()


def test_bf16_weight_beyond_fp16_range_is_rejected():
    from diffusion_lm_decoding_amd import _lib as L
    from diffusion_lm_decoding_amd.engine import Engine
    w = gen_weights(BF16, seed=0)
    wq = w["l1.wq"].copy()
    wq[3, 5] = f32_to_bf16_bits(np.array([1.0e6], np.float32))[0]   # finite in bf16, inf in fp16
    w["l1.wq"] = wq
    with pytest.raises(L.DllmError) as e:
        Engine(BF16, w, max_batch=1, max_seq=96)
    assert e.value.status == L.ERR_ARG and "65504" in str(e.value)


def test_fp16_activation_overflow_is_numeric_error():
    """Planted gains of 1e7 on the first norm push the fp16 copy of x * gain
    past 65504: the step reports DLLM_ERR_NUMERIC and commits nothing."""
    from diffusion_lm_decoding_amd import _lib as L
    from diffusion_lm_decoding_amd.engine import Engine
    w = gen_weights(BF16, seed=0)
    w["l0.attn_norm"] = f32_to_bf16_bits(np.full(BF16.d_model, 1.0e7, np.float32))
    eng = Engine(BF16, w, max_batch=1, max_seq=96)
    pr, t, a = _inputs()
    cv = eng.canvas(pr, t, a, 64)
    cfg = Engine.decode_cfg(1, 32, 64, 16)
    eng.begin(cv, cfg)
    eng.refresh(cv, cfg)
    before = cv.tokens.clone()
    with pytest.raises(L.DllmError) as e:
        eng.step(cv, cfg, 0)
    assert e.value.status == L.ERR_NUMERIC
    assert torch.equal(before, cv.tokens)
    eng.close()


def test_stats_split_device_time(eng32):
    from diffusion_lm_decoding_amd.engine import Engine
    pr, t, a = _inputs()
    cv = eng32.canvas(pr, t, a, 64)
    st = eng32.decode(cv, Engine.decode_cfg(1, 32, 64, 16))
    # each block's first step is its refresh pass; the others split the time
    assert st.refreshes == 4 and st.committed == 64 and st.steps > st.refreshes
    assert st.ms_step > 0 and st.ms_select > 0 and st.ms_refresh > 0
    assert st.ms_step + st.ms_select + st.ms_refresh <= st.ms_total


def test_trace_log_matches_stats(eng32, tmp_path, monkeypatch):
    """DLLM_TRACE: one line per cache pass and per step, whose counts add up
    to the decode's statistics; an unopenable path is an argument error."""
    from diffusion_lm_decoding_amd import _lib as L
    from diffusion_lm_decoding_amd.engine import Engine
    pr, t, a = _inputs(batch=2)
    cfg = Engine.decode_cfg(2, 32, 64, 16)
    path = tmp_path / "trace.jsonl"
    monkeypatch.setenv("DLLM_TRACE", str(path))
    cv = eng32.canvas(pr, t, a, 64)
    st = eng32.decode(cv, cfg)
    lines = [json.loads(x) for x in path.read_text().splitlines()]
    steps = [x for x in lines if x["event"] == "step"]
    refreshes = [x for x in lines if x["event"] == "refresh"]
    assert lines[-1] == {"event": "decode", "steps": st.steps, "refreshes": st.refreshes, "committed": st.committed}
    assert len(steps) == st.steps and len(refreshes) == st.refreshes == 4
    assert sum(sum(x["committed"]) for x in steps) == st.committed == 128
    assert [x["step"] for x in steps] == list(range(st.steps))
    for j in range(4):
        blk = [x for x in steps if x["block"] == j]
        assert [x["in_block"] for x in blk] == list(range(len(blk)))
        assert blk[-1]["done"] == [1, 1]
        assert sum(sum(x["committed"]) for x in blk) == 2 * 16
    # each block's first step is a cache pass, logged right after its refresh
    # line; the forward / selection split is sampled on every 8th other step
    passes = [x for x in steps if x.get("cache_pass")]
    assert [(x["block"], x["in_block"]) for x in passes] == [(j, 0) for j in range(4)]
    for i, x in enumerate(lines):
        if x.get("cache_pass"):
            assert lines[i - 1]["event"] == "refresh"
            assert (lines[i - 1]["block"], lines[i - 1]["in_block"]) == (x["block"], x["in_block"])
    plain = [x for x in steps if not x.get("cache_pass")]
    assert plain and all(("ms_forward" in x) == (k % 8 == 0) for k, x in enumerate(plain))
    assert not any("ms_forward" in x for x in passes)
    assert all(x["ms"] > 0 for x in refreshes)
    monkeypatch.setenv("DLLM_TRACE", str(tmp_path / "no_such_dir" / "trace.jsonl"))
    cv = eng32.canvas(pr, t, a, 64)
    with pytest.raises(L.DllmError) as e:
        eng32.decode(cv, cfg)
    assert e.value.status == L.ERR_ARG and "DLLM_TRACE" in str(e.value)
