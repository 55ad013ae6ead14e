"""Helpers for GPU-vs-oracle parity: lock-step replay of a decode.

At every step the oracle evaluates the GPU's current canvas with its own
float64 cache (refreshed at the same boundaries), then the GPU step runs; the
two are compared on logits, confidences and decisions, and the replay
continues from the GPU's canvas."""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np
import torch

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


def _softmax_top2_gap(l: np.ndarray) -> np.ndarray:
    f = np.isfinite(l)
    z = np.where(f, l, -np.inf)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    s = np.sort(p, axis=1)
    return s[:, -1] - s[:, -2]


def _exempt_sel(i, cand, conf, rule, tau, factor, tol: Tol) -> bool:
    c = conf[i]
    if rule == "threshold" and abs(c - tau) <= tol.near_tau:
        return True
    others = np.delete(conf, i)
    if others.size and np.min(np.abs(others - c)) <= tol.near_rank:
        return True
    if rule == "factor":
        # any candidate whose factor condition sits near its boundary
        order = np.argsort(-conf, kind="stable")
        for r, j in enumerate(order):
            if abs((r + 2) * (1 - conf[j]) - factor) <= tol.near_rank * (r + 2):
                return True
    return False


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

    nb = Lg // B
    if cache == "block_causal":
        engine.refresh(cv, cfg, -1)
        dec.prefill(st)
    for j in range(nb):
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
            if (before[s:e] == mask_id).any():
                cand, y, c, l = dec.evaluate(st, j)
            else:
                cand = np.zeros(0, np.int64)
            nc, done, gconf, gtok, glog = engine.step(cv, cfg, j, debug=True, debug_logits=check_logits)
            after = cv.tokens[seq].cpu().numpy()
            rep.steps += 1
            if cand.size == 0:
                if not np.array_equal(before, after):
                    rep.bad.append(f"step {rep.steps}: finished sequence changed")
                continue
            rows = seq * B + (cand - s)
            gc = gconf.cpu().numpy()[rows].astype(np.float64)
            gt = gtok.cpu().numpy()[rows]
            rep.max_conf_err = max(rep.max_conf_err, float(np.abs(gc - c).max()))
            if not tol.fp32 and np.abs(gc - c).max() > tol.conf_abs:
                rep.bad.append(f"step {rep.steps}: conf err {np.abs(gc - c).max():.3g}")
            if check_logits:
                gl = glog.cpu().numpy()[rows].astype(np.float64)
                fin = np.isfinite(l)
                if not np.array_equal(fin, np.isfinite(gl)):
                    rep.bad.append(f"step {rep.steps}: -inf pattern differs")
                err = np.abs(np.where(fin, np.where(fin, gl, 0.0) - np.where(fin, l, 0.0), 0.0))
                if tol.fp32:
                    scale = np.abs(np.where(fin, l, 0.0)).max(axis=1, keepdims=True)
                    rel = float((err / scale).max())
                    rep.max_logit_err = max(rep.max_logit_err, rel)
                    if rel > tol.logit_rel:
                        rep.bad.append(f"step {rep.steps}: logit rel err {rel:.3g}")
                else:
                    rep.max_logit_err = max(rep.max_logit_err, float(err.max()))
                    if err.max() > tol.logit_abs:
                        rep.bad.append(f"step {rep.steps}: logit abs err {err.max():.3g}")
                gap = _softmax_top2_gap(l)
            else:
                gap = np.full(len(cand), 1.0)
            # decisions
            o_sel = set(dec.choose(cand, c).tolist())
            g_sel = set(np.nonzero(after != before)[0].tolist())
            rep.decisions += len(cand)
            for pos in sorted(o_sel ^ g_sel):
                i = int(np.searchsorted(cand, pos))
                if tol.fp32 or not _exempt_sel(i, cand, c, rule, tau, factor, tol):
                    rep.bad.append(f"step {rep.steps}: selection differs at {pos} (oracle c={c[i]:.4f})")
                else:
                    rep.exempt += 1
            for pos in sorted(o_sel & g_sel):
                i = int(np.searchsorted(cand, pos))
                if after[pos] != y[i]:
                    if tol.fp32 or gap[i] > tol.top2_gap:
                        rep.bad.append(f"step {rep.steps}: token differs at {pos}: gpu {after[pos]} oracle {y[i]}")
                    else:
                        rep.exempt += 1
            if (gt != y).any():
                for i in np.nonzero(gt != y)[0]:
                    if tol.fp32 or gap[i] > tol.top2_gap:
                        rep.bad.append(f"step {rep.steps}: argmax differs at {cand[i]}")
            # the oracle's cache rows follow its own evaluation; continue from the GPU canvas
        if cache == "block_causal":
            engine.refresh(cv, cfg, j)
            sync_canvas()
            dec.commit_pass(st, j)
    return rep
