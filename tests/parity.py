"""Helpers for GPU-vs-oracle parity: lock-step replay of a decode.

At every step the oracle evaluates the GPU's current canvas with its own
float64 cache (refreshed at the same boundaries), then the GPU step runs; the
two are compared on logits, confidences and decisions, and the replay
continues from the GPU's canvas.

Decision rule (bf16): a selection difference at position i is allowed only
when its oracle confidence is within 0.02 of tau (threshold rule), within
0.02 of another candidate's (rank tie), or, for the factor rule, when some
candidate's (n+1)(1-c) sits within 0.02 (n+1) of f; a token difference only
when the oracle's top-2 probability gap is <= 0.05.  fp32 allows none."""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from oracle import OracleDecoder, OracleModel


@dataclass
class Tol:
    fp32: bool
    logit_abs: float = 5e-2        # bf16: absolute
    logit_rel: float = 1e-4        # fp32: relative to the row's max |logit|
    conf_abs: float = 1e-2
    near_tau: float = 0.02
    near_rank: float = 0.02
    top2_gap: float = 0.05


@dataclass
class Report:
    steps: int = 0
    max_logit_err: float = 0.0
    max_conf_err: float = 0.0
    decisions: int = 0
    exempt: int = 0
    bad: List[str] = field(default_factory=list)


def top2_gap(l: np.ndarray) -> np.ndarray:
    z = np.where(np.isfinite(l), l, -np.inf)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    s = np.sort(p, axis=1)
    return s[:, -1] - s[:, -2]


def _exempt_sel(i, conf, rule, tau, factor, tol: Tol) -> bool:
    c = conf[i]
    if rule == "threshold" and abs(c - tau) <= tol.near_tau:
        return True
    others = np.delete(conf, i)
    if others.size and np.min(np.abs(others - c)) <= tol.near_rank:
        return True
    if rule == "factor":
        order = np.argsort(-conf, kind="stable")
        for r, j in enumerate(order):
            if abs((r + 2) * (1 - conf[j]) - factor) <= tol.near_rank * (r + 2):
                return True
    if rule == "budget":
        eps = 1.0 - np.sort(conf)[::-1]
        lhs = np.cumsum(eps) + eps
        if np.any(np.abs(lhs - 1.0) <= tol.near_rank * (np.arange(eps.size) + 2)):
            return True
    return False


def compare_step(rep: Report, tol: Tol, dec: OracleDecoder, cand, y, c, l, gc, gt, gl, before, after,
                 k_in_block: int = 0, tag: str = "") -> None:
    """Compare one step: oracle (cand, y, c, l) against the GPU's confidences
    gc, tokens gt, logits gl (rows of cand; gl may be None) and the canvas
    before/after the GPU step."""
    rep.steps += 1
    tag = tag or f"step {rep.steps}"
    rep.max_conf_err = max(rep.max_conf_err, float(np.abs(gc - c).max()))
    if not tol.fp32 and np.abs(gc - c).max() > tol.conf_abs:
        rep.bad.append(f"{tag}: conf err {np.abs(gc - c).max():.3g}")
    if gl is not None:
        fin = np.isfinite(l)
        if not np.array_equal(fin, np.isfinite(gl)):
            rep.bad.append(f"{tag}: -inf pattern differs")
        err = np.abs(np.where(fin, gl, 0.0) - np.where(fin, l, 0.0))
        if tol.fp32:
            scale = np.abs(np.where(fin, l, 0.0)).max(axis=1, keepdims=True)
            rel = float((err / scale).max())
            rep.max_logit_err = max(rep.max_logit_err, rel)
            if rel > tol.logit_rel:
                rep.bad.append(f"{tag}: logit rel err {rel:.3g}")
        else:
            rep.max_logit_err = max(rep.max_logit_err, float(err.max()))
            if err.max() > tol.logit_abs:
                d = np.where(fin, gl, 0.0) - np.where(fin, l, 0.0)
                lf = np.where(fin, l, 0.0)
                beta = float((d * lf).sum() / (lf * lf).sum())
                res = d - beta * lf
                r, v = np.unravel_index(np.argmax(err), err.shape)
                rep.bad.append(f"{tag}: logit abs err {err.max():.3g} (rms {np.sqrt((d ** 2).mean()):.3g}, "
                               f"fit d = {beta:.3g} l, residual rms {np.sqrt((res ** 2).mean()):.3g}; "
                               f"worst row {r} vocab {v} oracle {l[r, v]:.4f} gpu {gl[r, v]:.4f}; "
                               f"per-row rms {np.sqrt((d ** 2).mean(axis=1)).round(4).tolist()[:8]})")
        gap = top2_gap(l)
    else:
        gap = np.zeros(len(cand))      # without logits only selections are checked strictly
    o_sel = set(dec.choose(cand, c, k_in_block).tolist())
    g_sel = set(np.nonzero(after != before)[0].tolist())
    rep.decisions += len(cand)
    for pos in sorted(o_sel ^ g_sel):
        i = int(np.searchsorted(cand, pos))
        if i >= len(cand) or cand[i] != pos:
            rep.bad.append(f"{tag}: GPU changed non-candidate position {pos}")
        elif tol.fp32 or not _exempt_sel(i, c, dec.rule, dec.tau, dec.factor, tol):
            rep.bad.append(f"{tag}: selection differs at {pos} (oracle c={c[i]:.4f})")
        else:
            rep.exempt += 1
    for pos in sorted(o_sel & g_sel):
        i = int(np.searchsorted(cand, pos))
        if after[pos] != y[i]:
            if tol.fp32 or gap[i] > tol.top2_gap:
                rep.bad.append(f"{tag}: token differs at {pos}: gpu {after[pos]} oracle {y[i]}")
            else:
                rep.exempt += 1
    for i in np.nonzero(gt != y)[0]:
        if tol.fp32 or gap[i] > tol.top2_gap:
            rep.bad.append(f"{tag}: argmax differs at {cand[i]}")


def replay(engine, cv, cfg, model: OracleModel, prompt, target, alpha, cache, rule, tau=0.9,
           factor=1.0, k=1, tol: Tol = None, seq: int = 0, max_steps: int = 10 ** 9,
           check_logits: bool = True) -> Report:
    """Lock-step replay of sequence `seq` of a batch decode (all sequences
    advance on the GPU; the oracle follows sequence `seq`)."""
    P, Lg, B = cfg.prompt_len, cfg.gen_len, cfg.block_len
    dec = OracleDecoder(model, P, Lg, B, cache=cache, rule=rule, tau=tau, factor=factor, k=k)
    st = dec.new_state(prompt[seq], target[seq], alpha[seq])
    rep = Report()
    mask_id = model.shape.mask_id

    def sync_canvas():
        st.canvas[:] = cv.tokens[seq].cpu().numpy()

    engine.begin(cv, cfg)
    if cache == "block_causal":
        engine.refresh(cv, cfg, -1)
        dec.prefill(st)
    for j in range(Lg // B):
        k_in_block = 0
        if cache in ("prefix", "dual"):
            engine.refresh(cv, cfg, 0)
            sync_canvas()
            dec.refresh(st)
        s, e = dec.block_range(j)
        while (cv.tokens[:, s:e] == mask_id).any().item():
            if rep.steps >= max_steps:
                return rep
            sync_canvas()
            before = st.canvas.copy()
            has_mask = (before[s:e] == mask_id).any()
            if has_mask:
                cand, y, c, l = dec.evaluate(st, j)
            _, _, gconf, gtok, glog = engine.step(cv, cfg, j, debug=True, debug_logits=check_logits)
            after = cv.tokens[seq].cpu().numpy()
            if not has_mask:
                rep.steps += 1
                if not np.array_equal(before, after):
                    rep.bad.append(f"step {rep.steps}: finished sequence changed")
                continue
            rows = seq * B + (cand - s)
            gl = glog.cpu().numpy()[rows].astype(np.float64) if check_logits else None
            compare_step(rep, tol, dec, cand, y, c, l, gconf.cpu().numpy()[rows].astype(np.float64),
                         gtok.cpu().numpy()[rows], gl, before, after, k_in_block)
            k_in_block += 1
        if cache == "block_causal":
            engine.refresh(cv, cfg, j)
            sync_canvas()
            dec.commit_pass(st, j)
    return rep
