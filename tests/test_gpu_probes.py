"""The measurement probes the roofline fractions are read against: argument
checks and bounds that any correct measurement obeys (the MFMA stream alone
is at least as fast as with LDS traffic beside it and below the dense peak;
a read far larger than the memory-side cache stays below the HBM peak)."""
import pytest

pytestmark = pytest.mark.gpu


def test_probe_mfma_mix_orders_and_rejects():
    from diffusion_lm_decoding_amd import _lib as L
    for bad in ((3, 0, 0), (1, 4, 0), (2, 8, 3)):
        with pytest.raises(L.DllmError) as e:
            L.dllm_probe_mfma_mix(*bad)
        assert e.value.status == L.ERR_ARG
    for wps in (1, 2):
        alone = L.dllm_probe_mfma_mix(wps, 0, 0)
        both = L.dllm_probe_mfma_mix(wps, 8, 4)
        print(f"{wps} wave(s) per SIMD: MFMA alone {alone:.0f} TFLOP/s, beside reads and copies {both:.0f}", flush=True)
        assert 500.0 < alone < 2600.0          # below the 2.5 PFLOP/s dense peak (plus timing slack)
        assert 0.0 < both <= alone * 1.02


def test_probe_read_and_peaks():
    from diffusion_lm_decoding_amd import _lib as L
    with pytest.raises(L.DllmError) as e:
        L.dllm_probe_read(1024)
    assert e.value.status == L.ERR_ARG
    small = L.dllm_probe_read(32 << 20)
    big = L.dllm_probe_read(2 << 30)
    print(f"streaming read: 32 MiB {small:.0f} GB/s, 2 GiB {big:.0f} GB/s", flush=True)
    # a read of a few tens of MiB can be served partly by the 256 MB memory-side cache; a 2 GiB
    # read cannot, and stays below the 8 TB/s HBM peak
    assert small > 1000.0 and 3000.0 < big < 8100.0
