"""Helpers for GPU-vs-oracle parity: lock-step replay of a decode.

At every step the oracle evaluates the GPU's current canvas with its own
float64 cache (refreshed at the same boundaries), then the GPU step runs; the
two are compared on logits, confidences and decisions, and the replay
continues from the GPU's canvas.

Every step is checked in two ways.

GPU self-consistency (fp32 and bf16, no exemption): the positions the GPU
committed are exactly the rule applied to the GPU's own reported
confidences; each committed token is the GPU's own argmax; with logits, that
argmax is the lowest index of the row's float32 maximum and the confidence
equals 1 / sum exp(l - max) of the GPU's logits.

GPU against the oracle: logits (fp32 1e-4 relative to the row's scale, bf16
5e-2 absolute), confidences (bf16 1e-2 absolute), then decisions.  In fp32
every decision must be identical.  In bf16 a selection difference is exempt
only at the rule's cut: for threshold membership when the oracle confidence
lies within 0.02 of tau; for the top-1 fallback, top-k, the factor rule and
the error budget when it lies within 0.02 of the oracle's confidence at the
cut (or the cut itself moved: the rule's criterion at the larger of the two
counts lies within 0.02 (n+1) of its bound).  A token difference is exempt
only when the oracle's top-2 probability gap is <= 0.05.  Exemptions are
counted per kind (selection; token of a committed position);
`Report.check_exemptions` bounds each at 1% of the decisions (at least one).
An argmax difference at a candidate that neither side commits this step
decides nothing; it is still allowed only at a top-2 gap <= 0.05, and is
counted apart (at random initialisation with a 126k vocabulary the top two
logits of a low-confidence row lie within the fp16 rounding of each other
for a few percent of rows)."""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List

import numpy as np

from oracle import OracleDecoder, OracleModel, order_by_confidence


@dataclass
class Tol:
    fp32: bool
    logit_abs: float = 5e-2        # bf16: absolute
    logit_rel: float = 1e-4        # fp32: relative to the row's max |logit|
    conf_abs: float = 1e-2
    near_cut: float = 0.02
    top2_gap: float = 0.05
    exempt_frac: float = 0.01


@dataclass
class Report:
    steps: int = 0
    max_logit_err: float = 0.0
    max_conf_err: float = 0.0
    decisions: int = 0
    exempt_sel: int = 0
    exempt_tok: int = 0
    argmax_flips: int = 0          # uncommitted candidates whose argmax differs (near-ties)
    bad: List[str] = field(default_factory=list)

    @property
    def exempt(self) -> int:
        return self.exempt_sel + self.exempt_tok

    def summary(self) -> str:
        return (f"steps={self.steps} max|dlogit|={self.max_logit_err:.3g} max|dconf|={self.max_conf_err:.3g} "
                f"decisions={self.decisions} exempt_selection={self.exempt_sel} exempt_token={self.exempt_tok} "
                f"argmax_flips_uncommitted={self.argmax_flips}")

    def check_exemptions(self, frac: float = 0.01) -> None:
        cap = max(1, math.floor(frac * self.decisions))
        for kind, n in (("selection", self.exempt_sel), ("token", self.exempt_tok)):
            if n > cap:
                self.bad.append(f"{n} {kind} exemptions over {self.decisions} decisions (cap {cap})")


def top2_gap(l: np.ndarray) -> np.ndarray:
    z = np.where(np.isfinite(l), l, -np.inf)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    s = np.sort(p, axis=1)
    return s[:, -1] - s[:, -2]


def _cut_exemptions(dec: OracleDecoder, cand, c, gc, o_sel, g_sel, near: float):
    """For each position where the oracle's and the GPU's selections differ:
    (position, exempt?, reason)."""
    diff = sorted(set(o_sel.tolist()) ^ set(g_sel.tolist()))
    if not diff:
        return []
    c32 = np.asarray(c, dtype=np.float32).astype(np.float64)
    order = order_by_confidence(c32, cand)
    cs = c32[order]                              # oracle confidences, descending
    rank = np.empty(len(cand), int)
    rank[order] = np.arange(len(cand))
    m = len(cand)
    out = []

    def near_cut_conf(i, n):
        """A cut after the top n (oracle ranking) separates c_i from a
        confidence within `near` of it: a near-tie across the cut."""
        if rank[i] < n:
            return n < m and abs(c32[i] - cs[n]) <= near
        return n >= 1 and abs(c32[i] - cs[n - 1]) <= near

    if dec.rule == "threshold":
        tau = float(np.float32(dec.tau))
        o_fb = not (c32 >= tau).any()
        g_fb = not (np.asarray(gc, np.float32) >= np.float32(dec.tau)).any()
        for pos in diff:
            i = int(np.searchsorted(cand, pos))
            if abs(c32[i] - tau) <= near:
                out.append((pos, True, "near tau"))
            elif (o_fb or g_fb) and near_cut_conf(i, 1):
                out.append((pos, True, "fallback near-tie at the top"))
            elif o_fb != g_fb and all(abs(c32[int(np.searchsorted(cand, q))] - tau) <= near
                                      for q in (g_sel if o_fb else o_sel)):
                out.append((pos, True, "fallback displaced by a near-tau threshold set"))
            else:
                out.append((pos, False, f"oracle c={c32[i]:.4f}, tau={tau}"))
        return out
    n_o, n_g = len(o_sel), len(g_sel)
    moved_ok = True
    if n_o != n_g and dec.rule in ("factor", "budget"):
        n = max(n_o, n_g)
        if dec.rule == "factor":
            crit, bound = (n + 1) * (1.0 - cs[n - 1]), dec.factor
        else:
            eps = 1.0 - cs[:n]
            crit, bound = eps.sum() + eps[-1], 1.0
        moved_ok = n >= 2 and abs(crit - bound) <= near * (n + 1)
    for pos in diff:
        i = int(np.searchsorted(cand, pos))
        if n_o != n_g and dec.rule in ("topk", "steps"):
            out.append((pos, False, f"GPU committed {n_g} positions, the rule {n_o}"))
        elif near_cut_conf(i, n_o) or near_cut_conf(i, n_g):
            out.append((pos, True, "near the confidence at the cut"))
        elif n_o != n_g and moved_ok and min(n_o, n_g) <= rank[i] < max(n_o, n_g):
            out.append((pos, True, "between the two cuts of a near-critical count"))
        else:
            out.append((pos, False, f"oracle c={c32[i]:.4f} rank {rank[i]}, counts {n_o}/{n_g}"))
    return out


def compare_step(rep: Report, tol: Tol, dec: OracleDecoder, cand, y, c, l, gc, gt, gl, before, after,
                 k_in_block: int = 0, tag: str = "") -> None:
    """Compare one step: oracle (cand, y, c, l) against the GPU's confidences
    gc, tokens gt, logits gl (rows of cand; gl may be None) and the canvas
    before/after the GPU step."""
    rep.steps += 1
    tag = tag or f"step {rep.steps}"
    cand = np.asarray(cand)
    gc = np.asarray(gc, dtype=np.float64)
    gt = np.asarray(gt)
    rep.max_conf_err = max(rep.max_conf_err, float(np.abs(gc - c).max()))
    if not tol.fp32 and np.abs(gc - c).max() > tol.conf_abs:
        rep.bad.append(f"{tag}: conf err {np.abs(gc - c).max():.3g}")
    # ---- GPU self-consistency -------------------------------------------
    changed = np.nonzero(after != before)[0]
    outside = np.setdiff1d(changed, cand)
    if outside.size:
        rep.bad.append(f"{tag}: GPU changed non-candidate positions {outside[:5].tolist()}")
    g_sel = np.intersect1d(changed, cand)
    g_rule = dec.choose(cand, gc, k_in_block)
    if not np.array_equal(g_sel, g_rule):
        rep.bad.append(f"{tag}: GPU committed {g_sel.tolist()}, its own confidences select {g_rule.tolist()}")
    gi = np.searchsorted(cand, g_sel)
    if not np.array_equal(after[g_sel], gt[gi]):
        rep.bad.append(f"{tag}: a committed token is not the GPU's own argmax")
    if gl is not None:
        g32 = gl.astype(np.float32)
        if not np.array_equal(np.argmax(g32, axis=1), gt):
            rep.bad.append(f"{tag}: GPU argmax differs from the lowest maximum of its own logits")
        fin = np.isfinite(gl)
        z = np.where(fin, gl, -np.inf)
        c_self = 1.0 / np.exp(z - z.max(axis=1, keepdims=True)).sum(axis=1)
        if np.abs(c_self - gc).max() > 1e-4 * max(1.0, float(np.abs(c_self).max())):
            rep.bad.append(f"{tag}: GPU confidence differs from its own logits' softmax maximum")
    # ---- against the oracle ---------------------------------------------
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
                r, v = np.unravel_index(np.argmax(err), err.shape)
                rep.bad.append(f"{tag}: logit abs err {err.max():.3g} (rms {np.sqrt((err ** 2).mean()):.3g}; "
                               f"worst row {r} vocab {v} oracle {l[r, v]:.4f} gpu {gl[r, v]:.4f})")
        gap = top2_gap(l)
    else:
        gap = np.zeros(len(cand))      # without logits no token difference is exempt
    o_sel = dec.choose(cand, c, k_in_block)
    rep.decisions += len(cand)
    for pos, ok, why in _cut_exemptions(dec, cand, c, gc, o_sel, g_sel, tol.near_cut):
        if ok and not tol.fp32:
            rep.exempt_sel += 1
        else:
            rep.bad.append(f"{tag}: selection differs at {pos} ({why})")
    committed = set(g_sel.tolist()) | set(o_sel.tolist())
    for i in np.nonzero(gt != y)[0]:
        if tol.fp32 or gap[i] > tol.top2_gap:
            rep.bad.append(f"{tag}: argmax differs at {cand[i]}: gpu {gt[i]} oracle {y[i]} (top-2 gap {gap[i]:.3g})")
        elif int(cand[i]) in committed:
            rep.exempt_tok += 1        # a committed token differs at a near-tie
        else:
            rep.argmax_flips += 1      # not committed this step: no decision taken on it


def replay(engine, cv, cfg, model: OracleModel, prompt, target, alpha, cache, rule, tau=0.9,
           factor=1.0, k=1, tol: Tol = None, seq: int = 0, max_steps: int = 10 ** 9,
           check_logits: bool = True, refresh_every: int = 0) -> Report:
    """Lock-step replay of sequence `seq` of a batch decode (all sequences
    advance on the GPU; the oracle follows sequence `seq`).  With
    refresh_every = r > 0 (PrefixCache / DualCache) both sides also refresh
    before in-block steps r, 2r, ..., as dllm_decode does.  Exemption counts
    are bounded at the end (`Report.check_exemptions`)."""
    P, Lg, B = cfg.prompt_len, cfg.gen_len, cfg.block_len
    dec = OracleDecoder(model, P, Lg, B, cache=cache, rule=rule, tau=tau, factor=factor, k=k,
                        refresh_every=refresh_every or None)
    st = dec.new_state(prompt[seq], target[seq], alpha[seq])
    rep = Report()
    mask_id = model.shape.mask_id
    cached = cache in ("prefix", "dual")

    def sync_canvas():
        st.canvas[:] = cv.tokens[seq].cpu().numpy()

    def both_refresh():
        engine.refresh(cv, cfg, 0)
        sync_canvas()
        dec.refresh(st)

    engine.begin(cv, cfg)
    if cache == "block_causal":
        engine.refresh(cv, cfg, -1)
        dec.prefill(st)
    for j in range(Lg // B):
        k_in_block = 0
        n_in_block = 0
        if cached:
            both_refresh()
        s, e = dec.block_range(j)
        while (cv.tokens[:, s:e] == mask_id).any().item():
            if rep.steps >= max_steps:
                rep.check_exemptions(tol.exempt_frac)
                return rep
            if cached and refresh_every and n_in_block > 0 and n_in_block % refresh_every == 0:
                both_refresh()
            n_in_block += 1
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
    rep.check_exemptions(tol.exempt_frac)
    return rep
