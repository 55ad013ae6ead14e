"""The shared synthetic-input generator: determinism, slice independence,
ranges, moments, and bf16 rounding against torch's float->bfloat16 cast."""
import numpy as np
import torch

from workloads import (LLADA_8B, TINY, bf16_bits_to_f32, f32_to_bf16_bits, gen_bias,
                       gen_prompt, gen_tensor, gen_weights, tensor_names)


def test_deterministic_and_seed_sensitive():
    a = gen_tensor(TINY, "l0.wq", seed=0)
    assert np.array_equal(a, gen_tensor(TINY, "l0.wq", seed=0))
    assert not np.array_equal(a, gen_tensor(TINY, "l0.wq", seed=1))
    assert not np.array_equal(a, gen_tensor(TINY, "l0.wk", seed=0))


def test_moments_and_gains():
    w = gen_weights(TINY, seed=0)
    x = np.concatenate([w[n].ravel() for n, _ in tensor_names(TINY) if not n.endswith("norm")])
    assert abs(x.std() - 0.02) < 2e-4 and abs(x.mean()) < 2e-4
    assert np.abs(x).max() <= 0.02 * 3.47
    assert all((w[n] == 1).all() for n, _ in tensor_names(TINY) if n.endswith("norm"))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=10000).astype(np.float32),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8], np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_8b_tensor_is_bf16_of_f32():
    f = gen_tensor(LLADA_8B, "l3.wo", seed=0, as_bf16=False)
    b = gen_tensor(LLADA_8B, "l3.wo", seed=0)
    assert b.dtype == np.uint16 and b.shape == (4096, 4096)
    assert np.array_equal(b, f32_to_bf16_bits(f))


def test_prompt_and_bias_ranges():
    p = gen_prompt(LLADA_8B, 4, 512, seed=2001)
    assert p.min() >= 0 and p.max() <= LLADA_8B.vocab - 2
    t, a = gen_bias(LLADA_8B, 4, 256, seed=2002, alpha_max=12.0)
    assert t.shape == (4, 256) and t.max() <= LLADA_8B.vocab - 2
    assert a.dtype == np.float32 and a.min() >= 0 and a.max() < 12.0
    assert abs(a.mean() - 6.0) < 0.5
