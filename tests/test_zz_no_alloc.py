"""dllm_block_step_noalloc (a block step whose workspaces are the library's
static device scratch, for callers that cannot allocate) against
dllm_block_step on identical states: two calls in a row, the second with a
smaller input, must give bitwise the same canvas, commit steps, counts,
confidences, tokens and logits; a step larger than the scratch serves is
rejected before any device work."""
import ctypes as C

import numpy as np
import pytest
import torch

from workloads import LLADA_8B, TINY, gen_bias, gen_prompt, gen_tensor, gen_weights, tensor_names

pytestmark = pytest.mark.gpu

BF16 = TINY.__class__(**{**TINY.__dict__, "dtype": "bf16", "name": "tiny_bf16"})


def _call(eng, cv, cfg, j, noalloc):
    from diffusion_lm_decoding_amd import _lib as L
    b, B = cfg.batch, cfg.block_len
    nc, dn = (C.c_int32 * b)(), (C.c_int32 * b)()
    conf = torch.empty(b * B, dtype=torch.float32, device=eng.device)
    tok = torch.empty(b * B, dtype=torch.int32, device=eng.device)
    logits = torch.empty(b * B, eng.shape.vocab, dtype=torch.float32, device=eng.device)
    fn = L.dllm_block_step_noalloc if noalloc else L.dllm_block_step
    fn(eng.ctx, cv.c_struct(), cfg, j, nc, dn, logits.data_ptr(), conf.data_ptr(), tok.data_ptr())
    torch.cuda.synchronize()
    return dict(nc=np.array(nc[:]), done=np.array(dn[:]), conf=conf.cpu().numpy(), tok=tok.cpu().numpy(),
                logits=logits.cpu().numpy(), tokens=cv.tokens.cpu().numpy(), cs=cv.commit_step.cpu().numpy())


def _run(eng, shape, batch, P, Lg, B, cache, n_steps, seed, noalloc):
    from diffusion_lm_decoding_amd.engine import Engine
    pr = gen_prompt(shape, batch, P, seed)
    t, a = gen_bias(shape, batch, Lg, seed + 1, 16.0)
    cv = eng.canvas(pr, t, a, Lg)
    cfg = Engine.decode_cfg(batch, P, Lg, B, cache=cache)
    eng.begin(cv, cfg)
    if cache == "block_causal":
        eng.refresh(cv, cfg, -1)
    elif cache != "none":
        eng.refresh(cv, cfg, 0)
    return [_call(eng, cv, cfg, 0, noalloc) for _ in range(n_steps)]


def _same(ref, got, what):
    assert len(ref) == len(got)
    for k, (r, g) in enumerate(zip(ref, got)):
        for key in r:
            assert np.array_equal(r[key], g[key], equal_nan=True), f"{what}: step {k} {key} differs"


def _check_pair(eng, shape, big, small):
    """big then small through dllm_block_step, then the same two through the
    static-scratch entry point, in a row."""
    ref = [_run(eng, shape, *big, noalloc=False), _run(eng, shape, *small, noalloc=False)]
    got = [_run(eng, shape, *big, noalloc=True), _run(eng, shape, *small, noalloc=True)]
    _same(ref[0], got[0], f"{shape.name} {big}")
    _same(ref[1], got[1], f"{shape.name} {small}")
    assert ref[0][0]["nc"].sum() >= 1


@pytest.mark.parametrize("cache", ["dual", "prefix", "none", "block_causal"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_step_equals_block_step_tiny(cache, dtype):
    from diffusion_lm_decoding_amd.engine import Engine
    shape = TINY if dtype == "f32" else BF16
    eng = Engine(shape, gen_weights(shape, seed=0, gain_jitter=0.1), max_batch=2, max_seq=64)
    batch = 2 if cache in ("dual", "block_causal") else 1
    _check_pair(eng, shape, (batch, 24, 32, 16, cache, 3, 601), (1, 8, 16, 8, cache, 2, 611))
    eng.close()


def test_noalloc_step_equals_block_step_llada8b():
    """LLaDA-8B shape: the benchmark's step (P 512, L 256, 32 rows, 8 key
    shares of attention, 6 MB of LM-head partials), then a shorter canvas
    (P 128, L 128)."""
    from diffusion_lm_decoding_amd.engine import Engine
    host = {n: gen_tensor(LLADA_8B, n, 0) for n, _ in tensor_names(LLADA_8B)}
    eng = Engine(LLADA_8B, host, max_batch=2, max_seq=768)
    del host
    _check_pair(eng, LLADA_8B, (1, 512, 256, 32, "dual", 2, 621), (1, 128, 128, 32, "dual", 2, 631))
    eng.close()


def test_noalloc_rejects_steps_beyond_the_scratch():
    from diffusion_lm_decoding_amd import _lib as L
    from diffusion_lm_decoding_amd.engine import Engine
    eng = Engine(TINY, gen_weights(TINY, seed=0), max_batch=4, max_seq=96)
    pr = gen_prompt(TINY, 4, 32, 641)
    t, a = gen_bias(TINY, 4, 64, 642, 8.0)
    cv = eng.canvas(pr, t, a, 64)
    cfg = Engine.decode_cfg(4, 32, 64, 32, cache="dual")      # 128 block rows
    eng.begin(cv, cfg)
    eng.refresh(cv, cfg, 0)
    before = cv.tokens.clone()
    with pytest.raises(L.DllmError) as e:
        _call(eng, cv, cfg, 0, noalloc=True)
    assert e.value.status == L.ERR_ARG and "64" in str(e.value)
    assert torch.equal(before, cv.tokens)
    eng.close()
