"""The teaching cost model reproduces every number the decoding-and-speed
page prints in its 'hand-computed cost' section (tests/golden/teaching_roofline.json)."""
import json
import os

from diffusion_lm_decoding_amd.roofline import Teaching, step_bytes_8b
from workloads import LLADA_8B

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "teaching_roofline.json")))


def test_teaching_numbers():
    t = Teaching(G["weight_bytes"], G["hbm_bytes_per_s"], G["flops_per_s"])
    assert round(t.W_ms, 2) == G["W_ms"]
    assert round(t.C_ms, 5) == G["C_ms"]
    assert round(t.crossover) == G["crossover_positions"]
    pre = t.step_ms(512)
    assert round(pre, 2) == G["prefill_512_ms"]
    assert round(pre + 256 * t.step_ms(1)) == G["ar_total_ms"]
    assert round(256 * t.step_ms(768)) == G["diff_uncached_1perstep_ms"]
    assert round(64 * t.step_ms(768)) == G["diff_uncached_4perstep_ms"]
    assert round(pre + 64 * t.step_ms(32)) == G["block_cache_4perstep_ms"]
    assert round(pre + 72 * t.step_ms(32)) == G["block_cache_with_writes_ms"]
    big = 10000
    assert round(big / t.step_ms(big) * 1e3) == G["ar_cap_tok_s"]
    assert round(4 * big / t.step_ms(32 * big) * 1e3) == G["diffusion_cap_tok_s"]
    # diffusion (G=32, 4 tokens/step) saturates compute near 9 concurrent requests
    assert min(b for b in range(1, 100) if 32 * b * t.C_ms >= t.W_ms) - 1 == G["diffusion_saturating_concurrency"]
    # AR catches up with the diffusion cap near 37 concurrent requests
    ar = lambda b: b / t.step_ms(b) * 1e3
    assert min(b for b in range(1, 400) if ar(b) >= G["diffusion_cap_tok_s"]) == G["ar_catches_up_concurrency"]


def test_8b_step_bytes():
    b = step_bytes_8b(LLADA_8B, n_keys=768, rows=32)
    assert b["weights"] == 2 * (32 * (4 * 4096 ** 2 + 3 * 4096 * 12288) + 126464 * 4096)
    assert abs(b["total"] / 1e9 - 15.41) < 0.01
