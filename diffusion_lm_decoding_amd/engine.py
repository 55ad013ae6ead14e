"""Thin Python front end of the HIP library: uploads weights, owns a context,
holds the canvas as torch device tensors and calls the C ABI.  PyTorch is used
for device memory and the stream only."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Dict, Optional

import ctypes as C
import numpy as np
import torch

from . import _lib as L


def to_device(a: np.ndarray, device) -> torch.Tensor:
    """numpy float32 -> float32 tensor; numpy uint16 (bf16 bits) -> bfloat16 tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclass
class CanvasState:
    tokens: torch.Tensor                 # int32 [batch, seq]
    target: Optional[torch.Tensor]       # int32 [batch, gen]
    alpha: Optional[torch.Tensor]        # float32 [batch, gen]
    commit_step: torch.Tensor            # int32 [batch, gen]

    def c_struct(self) -> L.Canvas:
        return L.Canvas(self.tokens.data_ptr(),
                        self.target.data_ptr() if self.target is not None else None,
                        self.alpha.data_ptr() if self.alpha is not None else None,
                        self.commit_step.data_ptr())


class Engine:
    """One library context for a model shape.

    tensors: name -> array for every name of workloads.tensor_names(shape), or a
    callable name -> array (lets an 8B model stream from the generator without
    holding 16 GB on the host)."""

    def __init__(self, shape, tensors, max_batch: int, max_seq: int, device: str = "cuda:0"):
        self.shape = shape
        self.device = torch.device(device)
        from workloads import tensor_names  # tensor order shared with the generator
        get: Callable[[str], np.ndarray] = tensors if callable(tensors) else tensors.__getitem__
        dev = []
        for name, _ in tensor_names(shape):
            dev.append(to_device(get(name), self.device))
        cfg = L.ModelCfg(shape.n_layers, shape.d_model, shape.n_heads, shape.head_dim, shape.d_ffn,
                         shape.vocab, shape.mask_id, shape.rms_eps, shape.rope_theta,
                         L.BF16 if shape.dtype == "bf16" else L.F32, max_batch, max_seq)
        self.stream = torch.cuda.current_stream(self.device)
        self.ctx = L.dllm_init_weights(cfg, [t.data_ptr() for t in dev], self.stream.cuda_stream)
        del dev
        torch.cuda.synchronize(self.device)
        self.max_batch, self.max_seq = max_batch, max_seq

    # -- configuration -------------------------------------------------------
    @staticmethod
    def decode_cfg(batch, prompt_len, gen_len, block_len, cache="dual", rule="threshold",
                   tau=0.9, factor=1.0, k=1, refresh_every=0) -> L.DecodeCfg:
        return L.DecodeCfg(batch, prompt_len, gen_len, block_len, L.CACHE[cache], L.RULE[rule],
                           tau, factor, k, refresh_every)

    @classmethod
    def cfg_from_workload(cls, w, **kw) -> L.DecodeCfg:
        args = dict(batch=w.batch, prompt_len=w.prompt_len, gen_len=w.gen_len, block_len=w.block_len,
                    cache=w.cache, rule=w.rule, tau=w.tau, factor=w.factor, k=w.k)
        args.update(kw)
        return cls.decode_cfg(**args)

    def canvas(self, prompt: np.ndarray, target: Optional[np.ndarray], alpha: Optional[np.ndarray],
               gen_len: int) -> CanvasState:
        b, p = prompt.shape
        toks = np.concatenate([prompt.astype(np.int32),
                               np.full((b, gen_len), self.shape.mask_id, np.int32)], axis=1)
        dev = self.device
        return CanvasState(
            torch.from_numpy(toks).to(dev),
            torch.from_numpy(np.ascontiguousarray(target, dtype=np.int32)).to(dev) if target is not None else None,
            torch.from_numpy(np.ascontiguousarray(alpha, dtype=np.float32)).to(dev) if alpha is not None else None,
            torch.full((b, gen_len), -1, dtype=torch.int32, device=dev))

    # -- calls -----------------------------------------------------------------
    def decode(self, cv: CanvasState, cfg: L.DecodeCfg) -> L.Stats:
        return L.dllm_decode(self.ctx, cv.c_struct(), cfg)

    def begin(self, cv: CanvasState, cfg: L.DecodeCfg) -> None:
        """Check the canvas and reset the step counters before driving
        refresh/step by hand."""
        L.dllm_begin_decode(self.ctx, cv.c_struct(), cfg)

    def refresh(self, cv: CanvasState, cfg: L.DecodeCfg, block_idx: int = 0) -> None:
        L.dllm_refresh_cache(self.ctx, cv.c_struct(), cfg, block_idx)

    def step(self, cv: CanvasState, cfg: L.DecodeCfg, block_idx: int, debug: bool = False,
             debug_logits: bool = False):
        """One block step; returns (n_committed, block_done) host arrays and,
        with debug, device tensors conf/tok [batch*B] (and logits)."""
        b, B = cfg.batch, cfg.block_len
        nc = (C.c_int32 * b)()
        dn = (C.c_int32 * b)()
        conf = tok = logits = None
        if debug:
            conf = torch.empty(b * B, dtype=torch.float32, device=self.device)
            tok = torch.empty(b * B, dtype=torch.int32, device=self.device)
        if debug_logits:
            logits = torch.empty(b * B, self.shape.vocab, dtype=torch.float32, device=self.device)
        L.dllm_block_step(self.ctx, cv.c_struct(), cfg, block_idx, nc, dn,
                          logits.data_ptr() if logits is not None else 0,
                          conf.data_ptr() if conf is not None else 0,
                          tok.data_ptr() if tok is not None else 0)
        return np.array(nc[:]), np.array(dn[:]), conf, tok, logits

    def staleness(self, cv: CanvasState, cfg: L.DecodeCfg, block_idx: int) -> dict:
        """Cached-vs-fresh evaluation of block block_idx at the current canvas
        and the per-layer, per-position K/V cosine of the cache against a fresh
        forward (device tensors); the cache is left unchanged."""
        b, B, N = cfg.batch, cfg.block_len, cfg.prompt_len + cfg.gen_len
        dev = self.device
        out = {"conf_cached": torch.empty(b * B, dtype=torch.float32, device=dev),
               "tok_cached": torch.empty(b * B, dtype=torch.int32, device=dev),
               "conf_fresh": torch.empty(b * B, dtype=torch.float32, device=dev),
               "tok_fresh": torch.empty(b * B, dtype=torch.int32, device=dev),
               "k_cos": torch.empty(self.shape.n_layers, b, N, dtype=torch.float32, device=dev),
               "v_cos": torch.empty(self.shape.n_layers, b, N, dtype=torch.float32, device=dev)}
        L.dllm_staleness(self.ctx, cv.c_struct(), cfg, block_idx, *(out[k].data_ptr() for k in
                         ("conf_cached", "tok_cached", "conf_fresh", "tok_fresh", "k_cos", "v_cos")))
        return out

    def close(self) -> None:
        if getattr(self, "ctx", None):
            L.dllm_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
