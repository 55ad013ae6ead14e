"""Pins of the oracle's cache geometry: which K/V rows each cache mode's step
rewrites, the block-causal attention pattern of block diffusion, and the
in-block refresh schedule.

  * Fast-dLLM reading notes, sec. 3 and Algorithm 1: PrefixCache reuses the
    prompt and the finished blocks and recomputes the current block and the
    suffix; DualCache also reuses the suffix and recomputes only the block;
    without a cache every position is recomputed.
  * Decoding-and-speed page, KV-cache section: block diffusion is
    bidirectional inside a block and causal across blocks, and a block size
    of one is plain autoregressive decoding.
  * Reading notes, sec. 11: the refresh interval decoupled from the block
    size (a refresh every r steps inside a block).

Each test is chosen so that a plausible slip in `OracleDecoder` (the row set
of one mode, token-causal instead of block-bidirectional rows, an off-by-one
in the refresh condition) fails it."""
import numpy as np
import pytest

from oracle import KVCache, OracleDecoder, OracleModel
from workloads import TINY, gen_bias, gen_prompt, gen_weights

SENTINEL = 7.25   # finite, so attention over poisoned rows stays finite


@pytest.fixture(scope="module")
def tiny_model():
    return OracleModel(TINY, gen_weights(TINY, seed=0, gain_jitter=0.1))


def _inputs(P=32, L=64, seed=1, alpha_max=16.0):
    pr = gen_prompt(TINY, 1, P, seed)
    t, a = gen_bias(TINY, 1, L, seed + 1, alpha_max)
    return pr[0], t[0], a[0]


def _rows_written(kv: KVCache) -> list:
    """Per layer, the sorted canvas rows whose K or V no longer hold the sentinel."""
    out = []
    for l in range(kv.k.shape[0]):
        hit = (kv.k[l] != SENTINEL).any(axis=(1, 2)) | (kv.v[l] != SENTINEL).any(axis=(1, 2))
        out.append(np.nonzero(hit)[0])
    return out


@pytest.mark.parametrize("cache", ["dual", "prefix", "none", "block_causal"])
def test_step_rewrites_exactly_the_modes_rows(tiny_model, cache):
    """Block 1 of P 32 / L 64 / B 16 (prefix, block and suffix all non-empty):
    after the cache passes the whole cache is overwritten with a sentinel,
    one step is evaluated, and the rows it wrote are read back per layer."""
    pr, t, a = _inputs()
    dec = OracleDecoder(tiny_model, 32, 64, 16, cache=cache)
    st = dec.new_state(pr, t, a)
    rng = np.random.default_rng(5)
    st.canvas[32:48] = rng.integers(0, TINY.mask_id, 16)      # block 0 finished
    st.canvas[50] = 7                                         # one committed position in block 1
    if cache == "block_causal":
        dec.prefill(st)
        dec.commit_pass(st, 0)
    elif cache != "none":
        dec.refresh(st)
    st.kv.k[:] = SENTINEL
    st.kv.v[:] = SENTINEL
    dec.evaluate(st, 1)
    s, e, N = 48, 64, 96
    expect = {"dual": np.arange(s, e), "block_causal": np.arange(s, e), "prefix": np.arange(s, N),
              "none": np.arange(0, N)}[cache]
    for l, rows in enumerate(_rows_written(st.kv)):
        assert np.array_equal(rows, expect), (cache, l, rows)


def test_block_size_one_is_autoregressive(tiny_model):
    """Block diffusion with a one-token prompt and blocks of one position is
    causal attention: the decoder's key limits drive the oracle forward to
    the logits of transformers' LLaMA under its own default causal mask."""
    torch = pytest.importorskip("torch")
    pytest.importorskip("transformers")
    from transformers import LlamaConfig, LlamaForCausalLM
    t = tiny_model.tensors
    cfg = LlamaConfig(vocab_size=TINY.vocab, hidden_size=TINY.d_model, intermediate_size=TINY.d_ffn,
                      num_hidden_layers=TINY.n_layers, num_attention_heads=TINY.n_heads,
                      num_key_value_heads=TINY.n_heads, head_dim=TINY.head_dim, rms_norm_eps=TINY.rms_eps,
                      rope_theta=TINY.rope_theta, max_position_embeddings=256, attention_bias=False,
                      mlp_bias=False, tie_word_embeddings=False, attn_implementation="eager")
    hf = LlamaForCausalLM(cfg).double().eval()
    sd = {"model.embed_tokens.weight": t["emb"], "model.norm.weight": t["final_norm"], "lm_head.weight": t["lm_head"]}
    names = {"attn_norm": "input_layernorm", "ffn_norm": "post_attention_layernorm", "wq": "self_attn.q_proj",
             "wk": "self_attn.k_proj", "wv": "self_attn.v_proj", "wo": "self_attn.o_proj", "wg": "mlp.gate_proj",
             "wu": "mlp.up_proj", "wd": "mlp.down_proj"}
    for l in range(TINY.n_layers):
        for a_, b_ in names.items():
            sd[f"model.layers.{l}.{b_}.weight"] = t[f"l{l}.{a_}"]
    hf.load_state_dict({k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in sd.items()}, strict=True)
    N = 24
    toks = gen_prompt(TINY, 1, N, seed=77)[0]
    dec = OracleDecoder(tiny_model, 1, N - 1, 1, cache="block_causal")
    rows = np.arange(N)
    kv = KVCache(TINY.n_layers, N, TINY.n_heads, TINY.head_dim)
    got = tiny_model.logits(tiny_model.forward_rows(toks, rows, kv, dec.key_limit(rows)))
    with torch.no_grad():
        ref = hf(input_ids=torch.from_numpy(toks.astype(np.int64))[None]).logits[0].numpy()
    # transformers computes its rotary tables and norms in float32
    assert np.abs(got - ref).max() / np.abs(ref).max() < 2e-5


def _block1_logits(dec, pr, t, a, canvas):
    """Block diffusion: prompt pass, commit pass of block 0, then the logits
    of block 1's masked rows (P 32, blocks of 16: block 1 is rows 48..63)."""
    st = dec.new_state(pr, t, a)
    st.canvas[:] = canvas
    dec.prefill(st)
    dec.commit_pass(st, 0)
    cand, _, _, l = dec.evaluate(st, 1)
    return cand, l


def test_block_diffusion_is_bidirectional_inside_a_block(tiny_model):
    pr, t, a = _inputs()
    dec = OracleDecoder(tiny_model, 32, 64, 16, cache="block_causal")
    rng = np.random.default_rng(9)
    canvas = np.concatenate([pr, rng.integers(0, TINY.mask_id, 64).astype(np.int32)])
    canvas[48:56] = TINY.mask_id                  # block 1: rows 48..55 masked, 56..63 filled
    canvas[64:] = TINY.mask_id                    # later blocks still masked
    cand, ref = _block1_logits(dec, pr, t, a, canvas)
    assert np.array_equal(cand, np.arange(48, 56))
    # a LATER token of the same block changes the earlier rows' logits
    c2 = canvas.copy()
    c2[61] = (c2[61] + 1) % TINY.mask_id
    _, l2 = _block1_logits(dec, pr, t, a, c2)
    fin = np.isfinite(ref)
    assert (np.abs(l2[fin] - ref[fin]).reshape(len(cand), -1).max(axis=1) > 1e-6).all()
    # a token of a later block changes nothing
    c3 = canvas.copy()
    c3[70] = 5
    _, l3 = _block1_logits(dec, pr, t, a, c3)
    assert np.array_equal(l3, ref)
    # an earlier block's token does reach block 1 (causal across blocks)
    c4 = canvas.copy()
    c4[40] = (c4[40] + 1) % TINY.mask_id
    _, l4 = _block1_logits(dec, pr, t, a, c4)
    assert np.abs(l4[fin] - ref[fin]).max() > 1e-6


def _canvas_before(rec_list, prompt, L, m):
    """Canvas before step m of a decode, rebuilt from the step records."""
    c = np.concatenate([prompt, np.full(L, TINY.mask_id, np.int32)])
    for r in rec_list[:m]:
        idx = np.searchsorted(r.cand, r.selected)
        c[r.selected] = r.tok[idx]
    return c


@pytest.mark.parametrize("cache,r", [("dual", 4), ("dual", 3), ("prefix", 2)])
def test_refresh_every_schedule(tiny_model, cache, r):
    """Top-1 per step, blocks of 16: every block takes 16 steps and refreshes
    at its start and before in-block steps r, 2r, ... < 16, i.e.
    1 + floor(15 / r) refreshes per block; exactly the steps that follow a
    refresh see an exact cache (their logits equal the uncached step's on
    the same canvas) and the others do not."""
    pr, t, a = _inputs()
    dec = OracleDecoder(tiny_model, 32, 64, 16, cache=cache, rule="topk", k=1, keep_logits=True,
                        refresh_every=r)
    st = dec.decode(pr, t, a)
    assert st.steps == 64
    assert st.refreshes == 4 * (1 + 15 // r)
    nc = OracleDecoder(tiny_model, 32, 64, 16, cache="none", rule="topk", k=1)
    for m, rec in enumerate(st.records):
        if rec.block != 1:
            continue
        s0 = nc.new_state(pr, t, a)
        s0.canvas[:] = _canvas_before(st.records, pr, 64, m)
        cand, _, _, l = nc.evaluate(s0, rec.block)
        assert np.array_equal(cand, rec.cand)
        fin = np.isfinite(l)
        err = np.abs(l[fin] - rec.logits[fin]).max()
        if rec.step % r == 0:
            assert err < 1e-10, (m, rec.step, err)
        else:
            assert err > 1e-8, (m, rec.step, err)


def test_dual_cache_step_is_stale_after_a_commit(tiny_model):
    """After one committed step the DualCache step reads a suffix cache that
    predates the commit: on the same canvas its confidences differ from the
    uncached step's (the approximation the pages accept)."""
    pr, t, a = _inputs()
    dual = OracleDecoder(tiny_model, 32, 64, 16, cache="dual")
    nc = OracleDecoder(tiny_model, 32, 64, 16, cache="none")
    st = dual.new_state(pr, t, a)
    dual.refresh(st)
    rec = dual.step(st, 0)
    assert len(rec.selected) >= 1
    c1, y1, cf1, _ = dual.evaluate(st, 0)
    s2 = nc.new_state(pr, t, a)
    s2.canvas[:] = st.canvas
    c2, y2, cf2, _ = nc.evaluate(s2, 0)
    assert np.array_equal(c1, c2)
    assert np.abs(cf1 - cf2).max() > 1e-9
