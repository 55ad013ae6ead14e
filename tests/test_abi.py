"""The C ABI library loads, exports every function include/dllm.h declares,
and rejects bad arguments before touching the GPU (runs without a GPU)."""
import ctypes as C
import os
import re

import pytest

from diffusion_lm_decoding_amd import _lib as L

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dllm.h")


def _declared():
    txt = open(HDR).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dllm_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = L.load()
    names = _declared()
    assert set(names) == set(L.SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def _tiny_cfg(**kw):
    c = L.ModelCfg(2, 128, 4, 32, 384, 512, 511, 1e-5, 10000.0, L.F32, 1, 96)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value", [("head_dim", 48), ("d_model", 100), ("mask_id", 512),
                                         ("dtype", 7), ("max_batch", 0), ("vocab", 500),
                                         ("rms_eps", 0.0)])
def test_init_rejects_bad_model_cfg(field, value):
    lib = L.load()
    out = C.c_void_p(123)
    ptrs = (C.c_void_p * 20)()
    st = lib.dllm_init_weights(C.byref(out), C.byref(_tiny_cfg(**{field: value})), ptrs, None)
    assert st == L.ERR_ARG and out.value is None
    assert lib.dllm_last_error()


def test_null_arguments_rejected():
    lib = L.load()
    cfg = L.DecodeCfg(1, 32, 64, 16, 2, 0, 0.9, 1.0, 1, 0)
    cv = L.Canvas(None, None, None, None)
    assert lib.dllm_decode(None, C.byref(cv), C.byref(cfg), None) == L.ERR_ARG
    assert lib.dllm_refresh_cache(None, C.byref(cv), C.byref(cfg), 0) == L.ERR_ARG
    assert lib.dllm_block_step(None, C.byref(cv), C.byref(cfg), 0, None, None, None, None, None) == L.ERR_ARG
    assert lib.dllm_init_weights(None, C.byref(_tiny_cfg()), None, None) == L.ERR_ARG
    lib.dllm_destroy(None)


def test_header_compiles_as_plain_c(tmp_path):
    """include/dllm.h is a C header: a C99 translation unit that includes it
    and takes the address of every declared function compiles warning-free."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = _declared()
    src = tmp_path / "use_header.c"
    src.write_text('#include "dllm.h"\n#include <stddef.h>\n'
                   "typedef void (*fn_t)(void);\n"
                   "fn_t dllm_symbols[] = {\n" + ",\n".join(f"  (fn_t){n}" for n in names) + "\n};\n"
                   "int dllm_sizes_ok(void) {\n"
                   "  return sizeof(dllm_model_cfg) == 12 * 4 && sizeof(dllm_decode_cfg) == 10 * 4 &&\n"
                   "         sizeof(dllm_canvas) == 4 * sizeof(void*) && sizeof(dllm_stats) == 8 * 8;\n}\n")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.dirname(HDR),
                        "-c", str(src), "-o", str(tmp_path / "use_header.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_struct_layouts_match_the_binding():
    """The ctypes structures mirror the header's structs field for field."""
    assert C.sizeof(L.ModelCfg) == 12 * 4
    assert C.sizeof(L.DecodeCfg) == 10 * 4
    assert C.sizeof(L.Canvas) == 4 * C.sizeof(C.c_void_p)
    assert C.sizeof(L.Stats) == 8 * 8
    assert [f for f, _ in L.Stats._fields_] == ["steps", "refreshes", "committed", "max_seq_steps", "ms_total",
                                                "ms_refresh", "ms_step", "ms_select"]
