"""Why the bf16 model computes with fp16 activations: a CPU replay of the HIP
path's rounding points at reduced depth.

The HIP path for a bf16 model keeps the residual stream, the norms, softmax
and every MFMA accumulator in fp32, and rounds to a 16-bit type T at these
points: each projection input (x * gain, the norm's 1/rms applied to the fp32
result), q / k / v (the KV cache), the attention probabilities entering the
P V product, the attention output, the SwiGLU output, and the final-norm
input of the LM head.  The weights are the bf16 values themselves.  This test
runs that forward twice, T = bf16 (8-bit significand) and T = fp16 (11 bits),
on an 8-layer model of the LLaDA-8B width (d 4096, 32 heads of 128, FFN
12288; vocabulary cut to 16384 to bound the CPU time) over a 128-position
canvas, and compares the last 32 rows' logits with the float64 oracle
forward.  The logit bound of the parity rule is 5e-2: bf16 rounding already
crosses it at a quarter of the model's depth, fp16 stays well inside.  fp16
range: the largest magnitude stored at a rounding point is reported and must
leave a wide margin below 65504."""
import numpy as np
import pytest

from oracle import KVCache, OracleModel
from workloads import ModelShape, bf16_bits_to_f32, f32_to_bf16_bits, gen_prompt, gen_tensor, tensor_names

SHAPE = ModelShape("llada8b_depth8", n_layers=8, d_model=4096, n_heads=32, head_dim=128, d_ffn=12288,
                   vocab=16384, mask_id=16383, dtype="bf16")
N_ROWS, HEAD_ROWS = 128, 32


def _round_bf16(x):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, np.float32)))


def _round_f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def _rope32(x, pos, theta):
    dh = x.shape[-1]
    half = dh // 2
    inv = theta ** (-(2.0 * np.arange(half)) / dh)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]
    cos = np.cos(ang).astype(np.float32)[:, None, :]
    sin = np.sin(ang).astype(np.float32)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def _replay(w, toks, rnd, peak):
    """The HIP path's arithmetic with rounding function `rnd` at its 16-bit
    points; fp32 everywhere else.  Returns the last HEAD_ROWS rows' logits."""
    m = SHAPE
    H, dh, eps = m.n_heads, m.head_dim, np.float32(m.rms_eps)
    pos = np.arange(N_ROWS)

    def store(a):
        peak[0] = max(peak[0], float(np.abs(a).max()))
        return rnd(a)

    def proj_in(x, gain):
        # packed x * gain in T; the fp32 result row is scaled by 1/rms afterwards
        rstd = np.float32(1.0) / np.sqrt((x * x).mean(axis=1, keepdims=True, dtype=np.float32) + eps)
        return store(x * gain), rstd

    x = w["emb"][toks].astype(np.float32)
    for l in range(m.n_layers):
        p = f"l{l}."
        xi, rstd = proj_in(x, w[p + "attn_norm"])
        q = (xi @ w[p + "wq"].T) * rstd
        k = (xi @ w[p + "wk"].T) * rstd
        v = (xi @ w[p + "wv"].T) * rstd
        q = store(_rope32(q.reshape(-1, H, dh), pos, m.rope_theta))
        k = store(_rope32(k.reshape(-1, H, dh), pos, m.rope_theta))
        v = store(v.reshape(-1, H, dh))
        s = np.einsum("qhd,khd->hqk", q, k) * np.float32(1.0 / np.sqrt(dh))
        s = np.exp(s - s.max(axis=-1, keepdims=True))
        lsum = s.sum(axis=-1, keepdims=True)
        o = np.einsum("hqk,khd->qhd", rnd(s), v) / lsum.transpose(1, 0, 2)
        o = store(o.reshape(-1, H * dh))
        x = x + o @ w[p + "wo"].T
        xi, rstd = proj_in(x, w[p + "ffn_norm"])
        g = (xi @ w[p + "wg"].T) * rstd
        u = (xi @ w[p + "wu"].T) * rstd
        act = store(g / (np.float32(1.0) + np.exp(-g)) * u)
        x = x + act @ w[p + "wd"].T
    xh, rstd = proj_in(x[-HEAD_ROWS:], w["final_norm"])
    return ((xh @ w["lm_head"].T) * rstd).astype(np.float64)


@pytest.mark.slow
def test_fp16_activations_stay_inside_the_logit_bound_and_bf16_do_not():
    # weights: the bf16 values, widened exactly to float32
    w = {n: bf16_bits_to_f32(gen_tensor(SHAPE, n, 0)) for n, _ in tensor_names(SHAPE)}
    toks = gen_prompt(SHAPE, 1, N_ROWS, seed=4242)[0]
    om = OracleModel(SHAPE, w, keep_f64=False)
    rows = np.arange(N_ROWS)
    kv = KVCache(SHAPE.n_layers, N_ROWS, SHAPE.n_heads, SHAPE.head_dim)
    ref = om.logits(om.forward_rows(toks, rows, kv, np.full(N_ROWS, N_ROWS))[-HEAD_ROWS:])
    err = {}
    peak = {}
    for name, rnd in (("fp16", _round_f16), ("bf16", _round_bf16)):
        pk = [0.0]
        got = _replay(w, toks, rnd, pk)
        d = np.abs(got - ref)
        err[name] = (float(d.max()), float(np.sqrt((d ** 2).mean())))
        peak[name] = pk[0]
    print(f"8 layers, {HEAD_ROWS} x {SHAPE.vocab} logits: fp16 max {err['fp16'][0]:.4f} rms {err['fp16'][1]:.5f}; "
          f"bf16 max {err['bf16'][0]:.4f} rms {err['bf16'][1]:.5f}; largest stored |value| {peak['fp16']:.1f}")
    assert err["fp16"][0] < 0.5 * 5e-2
    assert err["bf16"][0] > 5e-2
    assert err["bf16"][1] > 4 * err["fp16"][1]
    assert peak["fp16"] < 65504 / 100
