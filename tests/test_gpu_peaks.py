"""The microbenchmarks of libhta_peaks run on the GPU and give sane rates: each
call returns 0, the sinks are finite, and the rates fall between a floor no
working kernel misses and the published peaks (small launches, milliseconds)."""
import pytest
import torch

from hybrid_linear_temporal_hta_amd import peaks

pytestmark = pytest.mark.gpu


def _ms(fn, reps=3):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def test_mfma_loop_rate():
    sink = torch.empty(512 * 256, device="cuda")
    ms = _ms(lambda: peaks.mfma(512, 2000, sink))
    tflops = peaks.mfma_flop(512, 2000) / (ms / 1e3) / 1e12
    print(f"[peaks] mfma loop {tflops:.0f} TFLOP/s", flush=True)
    assert torch.isfinite(sink).all()
    assert 200.0 < tflops < 2500.0


def test_copy_rate_and_content():
    src = torch.arange(1 << 22, device="cuda", dtype=torch.float32)   # 16 MiB
    dst = torch.zeros_like(src)
    ms = _ms(lambda: peaks.copy(src, dst))
    assert torch.equal(src, dst)
    gbps = 2 * src.numel() * 4 / (ms / 1e3) / 1e9
    print(f"[peaks] copy {gbps:.0f} GB/s", flush=True)
    assert 100.0 < gbps < 40000.0   # a 16 MiB copy may run from the caches


@pytest.mark.parametrize("pattern", [0, 1])
def test_global_to_lds_rate(pattern):
    win = 1 << 21
    src = torch.ones(win // 4, device="cuda")
    ms = _ms(lambda: peaks.lds_dma(src, win, 512, 100, pattern))
    tbps = peaks.lds_dma_bytes(512, 100) / (ms / 1e3) / 1e12
    print(f"[peaks] global->LDS pattern {pattern}: {tbps:.2f} TB/s", flush=True)
    assert 0.5 < tbps < 60.0


@pytest.mark.parametrize("transposed", [False, True])
def test_lds_read_rate(transposed):
    sink = torch.empty(512 * 256, device="cuda")
    ms = _ms(lambda: peaks.lds_read(512, 500, transposed, sink))
    tbps = peaks.lds_read_bytes(512, 500, transposed) / (ms / 1e3) / 1e12
    print(f"[peaks] LDS read transposed={transposed}: {tbps:.1f} TB/s", flush=True)
    assert torch.isfinite(sink).all()
    assert 2.0 < tbps < 200.0
