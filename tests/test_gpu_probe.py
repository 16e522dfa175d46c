"""The matrix-core rate probe of the library (a measurement aid that the bench
reports next to the nominal bf16 peak), called through the C ABI."""

import ctypes

import pytest

from helpers import say

pytestmark = pytest.mark.gpu

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import branch_attention_speculative_amd as ba
    ba.lib()
    return torch, ba


def test_probe_rates_and_sink(env):
    torch, ba = env
    L = ba.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.full((8192,), 7.0, device="cuda")
    rates = {}
    for random in (0, 1):
        out = ctypes.c_double(0.0)
        st = L.ba_probe_mfma(random, 2000, ctypes.c_void_p(sink.data_ptr()), sink.numel(), stream,
                             ctypes.byref(out))
        assert st == 0, L.ba_last_error()
        rates[random] = out.value
        s = sink.cpu()
        if random:
            assert bool(torch.isfinite(s).all()) and int((s != 0).sum()) > 8000
        else:
            assert bool((s == 0).all())
    say(f"  probe: zero operands {rates[0]:.0f} TFLOP/s, random {rates[1]:.0f} TFLOP/s")
    # a rate above the nominal peak would mean the probe lost work
    for r in rates.values():
        assert 0 < r <= 1.02 * PEAK_BF16_TFLOPS
    # the binding's wrapper gives the same kind of figure
    assert 0 < ba.probe_mfma(True, 2000) <= 1.02 * PEAK_BF16_TFLOPS


def test_probe_rejects_bad_arguments(env):
    torch, ba = env
    L = ba.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.zeros(8192, device="cuda")
    out = ctypes.c_double(0.0)
    assert L.ba_probe_mfma(1, 100, ctypes.c_void_p(sink.data_ptr()), 8191, stream, ctypes.byref(out)) == 1
    assert b"sink needs" in L.ba_last_error()
    assert L.ba_probe_mfma(1, 0, ctypes.c_void_p(sink.data_ptr()), 8192, stream, ctypes.byref(out)) == 1
    assert L.ba_probe_mfma(1, 100, None, 8192, stream, ctypes.byref(out)) == 1
