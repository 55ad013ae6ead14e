"""Pins of the oracle's transformer forward: transformers' LLaMA (same
architecture family) driven with a bidirectional or block-causal additive
4-D mask; component reductions to torch library routines; RoPE against a
complex-number formulation; and a check that planted mistakes are caught."""
import numpy as np
import pytest
import torch

from oracle import OracleModel, KVCache
from oracle import model as OM
from workloads import TINY, gen_prompt, gen_weights

transformers = pytest.importorskip("transformers")


def _hf_model(shape, tensors):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(vocab_size=shape.vocab, hidden_size=shape.d_model,
                      intermediate_size=shape.d_ffn, num_hidden_layers=shape.n_layers,
                      num_attention_heads=shape.n_heads, num_key_value_heads=shape.n_heads,
                      head_dim=shape.head_dim, rms_norm_eps=shape.rms_eps,
                      rope_theta=shape.rope_theta, max_position_embeddings=4096,
                      attention_bias=False, mlp_bias=False, tie_word_embeddings=False,
                      attn_implementation="eager")
    m = LlamaForCausalLM(cfg).double().eval()
    sd = {"model.embed_tokens.weight": tensors["emb"], "model.norm.weight": tensors["final_norm"],
          "lm_head.weight": tensors["lm_head"]}
    names = {"attn_norm": "input_layernorm", "ffn_norm": "post_attention_layernorm",
             "wq": "self_attn.q_proj", "wk": "self_attn.k_proj", "wv": "self_attn.v_proj",
             "wo": "self_attn.o_proj", "wg": "mlp.gate_proj", "wu": "mlp.up_proj",
             "wd": "mlp.down_proj"}
    for l in range(shape.n_layers):
        for a, b in names.items():
            sd[f"model.layers.{l}.{b}.weight"] = tensors[f"l{l}.{a}"]
    m.load_state_dict({k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in sd.items()},
                      strict=True)
    return m


def _hf_logits(hf, tokens, key_limit):
    T = len(tokens)
    vis = np.arange(T)[None, :] < np.asarray(key_limit)[:, None]
    mask = torch.from_numpy(np.where(vis, 0.0, -np.inf))[None, None]
    with torch.no_grad():
        out = hf(input_ids=torch.from_numpy(np.asarray(tokens, np.int64))[None], attention_mask=mask)
    return out.logits[0].numpy()


def _oracle_logits(om, tokens, key_limit):
    N = len(tokens)
    kv = KVCache(om.shape.n_layers, N, om.shape.n_heads, om.shape.head_dim)
    h = om.forward_rows(np.asarray(tokens), np.arange(N), kv, np.asarray(key_limit))
    return om.logits(h)


def _rel_err(a, b):
    return float(np.abs(a - b).max() / np.abs(b).max())


@pytest.fixture(scope="module")
def tiny():
    t = gen_weights(TINY, seed=0, gain_jitter=0.1)
    toks = gen_prompt(TINY, 1, 48, seed=11)[0]
    return t, toks, _hf_model(TINY, t)


# transformers' LLaMA runs its norms and rotary tables in float32
TOL = 2e-5


def test_forward_matches_llama_bidirectional(tiny):
    t, toks, hf = tiny
    om = OracleModel(TINY, t)
    lim = np.full(len(toks), len(toks))
    assert _rel_err(_oracle_logits(om, toks, lim), _hf_logits(hf, toks, lim)) < TOL


def test_forward_matches_llama_block_causal(tiny):
    t, toks, hf = tiny
    om = OracleModel(TINY, t)
    P, B = 16, 8
    rows = np.arange(len(toks))
    lim = np.where(rows < P, P, P + ((rows - P) // B + 1) * B)
    assert _rel_err(_oracle_logits(om, toks, lim), _hf_logits(hf, toks, lim)) < TOL


@pytest.mark.parametrize("mutation", ["rope_interleaved", "attn_scale", "no_gain", "wo_transposed",
                                      "swap_gate_up", "no_mask"])
def test_planted_mistakes_are_caught(tiny, monkeypatch, mutation):
    t, toks, hf = tiny
    P, B = 16, 8
    rows = np.arange(len(toks))
    lim = np.where(rows < P, P, P + ((rows - P) // B + 1) * B)
    ref = _hf_logits(hf, toks, lim)
    tt = dict(t)
    if mutation == "rope_interleaved":
        def bad_rope(x, positions, theta):
            y = x.copy()
            y[..., 0::2], y[..., 1::2] = x[..., : x.shape[-1] // 2], x[..., x.shape[-1] // 2:]
            y = OM.__dict__["_orig_rope"](y, positions, theta)
            z = y.copy()
            z[..., : x.shape[-1] // 2], z[..., x.shape[-1] // 2:] = y[..., 0::2], y[..., 1::2]
            return z
        monkeypatch.setitem(OM.__dict__, "_orig_rope", OM.rope)
        monkeypatch.setattr(OM, "rope", bad_rope)
    elif mutation == "attn_scale":
        orig = OM.attention
        monkeypatch.setattr(OM, "attention", lambda q, k, v, lim: orig(q / np.sqrt(q.shape[-1]), k, v, lim))
    elif mutation == "no_gain":
        tt["l1.ffn_norm"] = np.ones_like(t["l1.ffn_norm"])
    elif mutation == "wo_transposed":
        tt["l0.wo"] = np.ascontiguousarray(t["l0.wo"].T)
    elif mutation == "swap_gate_up":
        tt["l0.wg"], tt["l0.wu"] = t["l0.wu"], t["l0.wg"]
    elif mutation == "no_mask":
        lim = np.full(len(toks), len(toks))
    om = OracleModel(TINY, tt)
    assert _rel_err(_oracle_logits(om, toks, lim), ref) > 100 * TOL


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(0)
    x, g = rng.normal(size=(7, 64)), rng.normal(size=64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-5)
    assert np.allclose(OM.rms_norm(x, g, 1e-5), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(1)
    Tq, Tk, H, dh = 5, 11, 3, 16
    q, k, v = (rng.normal(size=(T, H, dh)) for T in (Tq, Tk, Tk))
    lim = np.array([11, 4, 7, 11, 1])
    mask = torch.from_numpy(np.arange(Tk)[None, :] < lim[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).transpose(0, 1), torch.from_numpy(k).transpose(0, 1),
        torch.from_numpy(v).transpose(0, 1), attn_mask=mask).transpose(0, 1)
    assert np.allclose(OM.attention(q, k, v, lim), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_rope_is_complex_rotation_and_relative():
    rng = np.random.default_rng(2)
    T, H, dh, theta = 9, 2, 16, 10000.0
    x = rng.normal(size=(T, H, dh))
    pos = rng.integers(0, 3000, T)
    half = dh // 2
    z = x[..., :half] + 1j * x[..., half:]
    w = np.exp(1j * pos[:, None, None] * theta ** (-np.arange(half) * 2.0 / dh))[:, :, :]
    zr = z * w
    ref = np.concatenate([zr.real, zr.imag], axis=-1)
    assert np.allclose(OM.rope(x, pos, theta), ref, atol=1e-12)
    # relative position: <R_m q, R_n k> depends only on m - n
    q, k = rng.normal(size=(1, 1, dh)), rng.normal(size=(1, 1, dh))
    d1 = np.sum(OM.rope(q, np.array([17]), theta) * OM.rope(k, np.array([5]), theta))
    d2 = np.sum(OM.rope(q, np.array([112]), theta) * OM.rope(k, np.array([100]), theta))
    assert abs(d1 - d2) < 1e-12
    assert np.allclose(OM.rope(x, np.zeros(T, int), theta), x)


def test_bf16_weights_widen_exactly():
    from workloads import f32_to_bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(3)
    a = rng.normal(size=100).astype(np.float32)
    b = f32_to_bf16_bits(a)
    assert np.array_equal(OM._as_f64(b), bf16_bits_to_f32(b).astype(np.float64))
