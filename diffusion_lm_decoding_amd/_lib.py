"""ctypes binding of libdllm.so (the C ABI declared in include/dllm.h).

Argument marshalling only: every step of the decode runs in the HIP library.
Loading fails loudly when the library has not been built; there is no
fallback.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdllm.so")

OK, ERR_ARG, ERR_OOM, ERR_DEVICE, ERR_STATE, ERR_NUMERIC = range(6)
STATUS_NAMES = {0: "OK", 1: "ERR_ARG", 2: "ERR_OOM", 3: "ERR_DEVICE", 4: "ERR_STATE", 5: "ERR_NUMERIC"}
F32, BF16 = 0, 1
CACHE = {"none": 0, "prefix": 1, "dual": 2, "block_causal": 3}
RULE = {"threshold": 0, "factor": 1, "topk": 2, "budget": 3, "steps": 4}

SYMBOLS = ("dllm_init_weights", "dllm_refresh_cache", "dllm_block_step", "dllm_block_step_noalloc",
           "dllm_staleness", "dllm_begin_decode",
           "dllm_decode", "dllm_set_timing", "dllm_get_timing", "dllm_probe_peaks", "dllm_probe_read",
           "dllm_probe_mfma_mix",
           "dllm_set_device_limit",
           "dllm_destroy", "dllm_last_error")
KERNEL_CLASSES = ("embed", "rmsnorm", "qkv", "attn", "oproj", "gateup", "down", "lmhead", "merge",
                  "select")


class KernelTime(C.Structure):
    _fields_ = [("launches", C.c_int64), ("ms", C.c_double), ("bytes", C.c_double),
                ("flops", C.c_double)]


class ModelCfg(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("head_dim", C.c_int32), ("d_ffn", C.c_int32), ("vocab", C.c_int32),
                ("mask_id", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_float),
                ("dtype", C.c_int32), ("max_batch", C.c_int32), ("max_seq", C.c_int32)]


class DecodeCfg(C.Structure):
    _fields_ = [("batch", C.c_int32), ("prompt_len", C.c_int32), ("gen_len", C.c_int32),
                ("block_len", C.c_int32), ("cache", C.c_int32), ("rule", C.c_int32),
                ("tau", C.c_float), ("factor", C.c_float), ("k", C.c_int32),
                ("refresh_every", C.c_int32)]


class Canvas(C.Structure):
    _fields_ = [("tokens", C.c_void_p), ("bias_target", C.c_void_p), ("bias_alpha", C.c_void_p),
                ("commit_step", C.c_void_p)]


class Stats(C.Structure):
    _fields_ = [("steps", C.c_int64), ("refreshes", C.c_int64), ("committed", C.c_int64),
                ("max_seq_steps", C.c_int64), ("ms_total", C.c_double), ("ms_refresh", C.c_double),
                ("ms_step", C.c_double), ("ms_select", C.c_double)]


class DllmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libdllm.so once; raise if it is missing (no CPU fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m diffusion_lm_decoding_amd.build`")
    lib = C.CDLL(path)
    P = C.c_void_p
    lib.dllm_init_weights.argtypes = [C.POINTER(P), C.POINTER(ModelCfg), C.POINTER(P), P]
    lib.dllm_init_weights.restype = C.c_int
    lib.dllm_refresh_cache.argtypes = [P, C.POINTER(Canvas), C.POINTER(DecodeCfg), C.c_int32]
    lib.dllm_refresh_cache.restype = C.c_int
    lib.dllm_block_step.argtypes = [P, C.POINTER(Canvas), C.POINTER(DecodeCfg), C.c_int32,
                                    C.POINTER(C.c_int32), C.POINTER(C.c_int32), P, P, P]
    lib.dllm_block_step.restype = C.c_int
    lib.dllm_block_step_noalloc.argtypes = lib.dllm_block_step.argtypes
    lib.dllm_block_step_noalloc.restype = C.c_int
    lib.dllm_staleness.argtypes = [P, C.POINTER(Canvas), C.POINTER(DecodeCfg), C.c_int32, P, P, P, P, P, P]
    lib.dllm_staleness.restype = C.c_int
    lib.dllm_begin_decode.argtypes = [P, C.POINTER(Canvas), C.POINTER(DecodeCfg)]
    lib.dllm_begin_decode.restype = C.c_int
    lib.dllm_probe_peaks.argtypes = [C.c_uint64, C.POINTER(C.c_double), C.POINTER(C.c_double)]
    lib.dllm_probe_peaks.restype = C.c_int
    lib.dllm_probe_read.argtypes = [C.c_uint64, C.POINTER(C.c_double)]
    lib.dllm_probe_read.restype = C.c_int
    lib.dllm_probe_mfma_mix.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_double)]
    lib.dllm_probe_mfma_mix.restype = C.c_int
    lib.dllm_decode.argtypes = [P, C.POINTER(Canvas), C.POINTER(DecodeCfg), C.POINTER(Stats)]
    lib.dllm_decode.restype = C.c_int
    lib.dllm_set_timing.argtypes = [P, C.c_uint32, C.c_uint32]
    lib.dllm_set_timing.restype = C.c_int
    lib.dllm_get_timing.argtypes = [P, C.POINTER(KernelTime), C.c_int32]
    lib.dllm_get_timing.restype = C.c_int
    lib.dllm_set_device_limit.argtypes = [C.c_uint64]
    lib.dllm_set_device_limit.restype = None
    lib.dllm_destroy.argtypes = [P]
    lib.dllm_destroy.restype = None
    lib.dllm_last_error.argtypes = []
    lib.dllm_last_error.restype = C.c_char_p
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != OK:
        raise DllmError(status, load().dllm_last_error().decode())


def dllm_init_weights(cfg: ModelCfg, tensor_ptrs, stream_ptr: int) -> int:
    lib = load()
    arr = (C.c_void_p * len(tensor_ptrs))(*tensor_ptrs)
    out = C.c_void_p()
    check(lib.dllm_init_weights(C.byref(out), C.byref(cfg), arr, C.c_void_p(stream_ptr)))
    return out.value


def dllm_refresh_cache(ctx: int, canvas: Canvas, cfg: DecodeCfg, block_idx: int) -> None:
    check(load().dllm_refresh_cache(C.c_void_p(ctx), C.byref(canvas), C.byref(cfg), block_idx))


def dllm_block_step(ctx: int, canvas: Canvas, cfg: DecodeCfg, block_idx: int, n_committed=None,
                    block_done=None, dbg_logits=0, dbg_conf=0, dbg_tok=0) -> None:
    check(load().dllm_block_step(C.c_void_p(ctx), C.byref(canvas), C.byref(cfg), block_idx,
                                 n_committed, block_done, C.c_void_p(dbg_logits),
                                 C.c_void_p(dbg_conf), C.c_void_p(dbg_tok)))


def dllm_block_step_noalloc(ctx: int, canvas: Canvas, cfg: DecodeCfg, block_idx: int, n_committed=None,
                            block_done=None, dbg_logits=0, dbg_conf=0, dbg_tok=0) -> None:
    check(load().dllm_block_step_noalloc(C.c_void_p(ctx), C.byref(canvas), C.byref(cfg), block_idx,
                                         n_committed, block_done, C.c_void_p(dbg_logits),
                                         C.c_void_p(dbg_conf), C.c_void_p(dbg_tok)))


def dllm_staleness(ctx: int, canvas: Canvas, cfg: DecodeCfg, block_idx: int, conf_cached=0, tok_cached=0,
                   conf_fresh=0, tok_fresh=0, k_cos=0, v_cos=0) -> None:
    check(load().dllm_staleness(C.c_void_p(ctx), C.byref(canvas), C.byref(cfg), block_idx,
                                C.c_void_p(conf_cached), C.c_void_p(tok_cached), C.c_void_p(conf_fresh),
                                C.c_void_p(tok_fresh), C.c_void_p(k_cos), C.c_void_p(v_cos)))


def dllm_begin_decode(ctx: int, canvas: Canvas, cfg: DecodeCfg) -> None:
    check(load().dllm_begin_decode(C.c_void_p(ctx), C.byref(canvas), C.byref(cfg)))


def dllm_decode(ctx: int, canvas: Canvas, cfg: DecodeCfg) -> Stats:
    st = Stats()
    check(load().dllm_decode(C.c_void_p(ctx), C.byref(canvas), C.byref(cfg), C.byref(st)))
    return st


def dllm_probe_peaks(nbytes: int = 8 << 30):
    """(achievable HBM read GB/s, achievable fp16 MFMA TFLOP/s) of device 0."""
    hbm, mfma = C.c_double(0.0), C.c_double(0.0)
    check(load().dllm_probe_peaks(C.c_uint64(nbytes), C.byref(hbm), C.byref(mfma)))
    return hbm.value, mfma.value


def dllm_probe_mfma_mix(waves_per_simd: int, lds_reads: int, dma_kib: int) -> float:
    """MFMA TFLOP/s of device 0 with LDS reads / DMA copies beside the MFMA stream."""
    t = C.c_double(0.0)
    check(load().dllm_probe_mfma_mix(C.c_int32(waves_per_simd), C.c_int32(lds_reads), C.c_int32(dma_kib),
                                     C.byref(t)))
    return t.value


def dllm_probe_read(nbytes: int) -> float:
    """Best streaming-read GB/s of device 0 for one read of `nbytes` bytes from HBM."""
    g = C.c_double(0.0)
    check(load().dllm_probe_read(C.c_uint64(nbytes), C.byref(g)))
    return g.value


def dllm_set_timing(ctx: int, classes, sample_every: int = 1) -> None:
    mask = 0
    for c in classes:
        mask |= 1 << KERNEL_CLASSES.index(c)
    check(load().dllm_set_timing(C.c_void_p(ctx), mask, sample_every))


def dllm_get_timing(ctx: int, reset: bool = True) -> dict:
    """{"step": {class: counters}, "cache": {class: counters}}"""
    n = len(KERNEL_CLASSES)
    arr = (KernelTime * (2 * n))()
    check(load().dllm_get_timing(C.c_void_p(ctx), arr, 1 if reset else 0))
    out = {}
    for part, off in (("step", 0), ("cache", n)):
        out[part] = {k: dict(launches=arr[off + i].launches, ms=arr[off + i].ms, bytes=arr[off + i].bytes,
                             flops=arr[off + i].flops) for i, k in enumerate(KERNEL_CLASSES)}
    return out


def dllm_set_device_limit(nbytes: int) -> None:
    load().dllm_set_device_limit(C.c_uint64(nbytes))


def dllm_destroy(ctx: int) -> None:
    load().dllm_destroy(C.c_void_p(ctx))
