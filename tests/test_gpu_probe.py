"""The peak micro-benchmarks of include/avey_probe.h on the GPU: the copy is exact, and the
matrix-core probe runs in both operand modes at a rate no higher than the datasheet peak allows
(a FLOP count that is wrong, or work removed by the compiler, would show as an impossible rate)."""
import pytest

import attention_free_long_amd as A

pytestmark = pytest.mark.gpu

PEAK_BF16_TFLOPS = 2500.0


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("nbytes", [16, 48, (1 << 20) + 16, 64 << 20])
def test_probe_copy_exact(torch_cuda, nbytes):
    torch = torch_cuda
    print(f"[probe copy] {nbytes} bytes", flush=True)
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    A.avey_probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("changing", [False, True])
def test_probe_mfma_rate_is_physical(torch_cuda, changing):
    torch = torch_cuda
    print(f"[probe mfma] changing={changing}", flush=True)
    iters = 400
    sink = A.avey_probe_mfma_bf16(iters, changing)     # warm-up, allocates the sink
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        A.avey_probe_mfma_bf16(iters, changing, sink)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 5 * 1e-3
    tflops = A.avey_probe_mfma_flops(iters) / t / 1e12
    print(f"[probe mfma] changing={changing}: {tflops:.0f} TFLOP/s", flush=True)
    assert 100.0 < tflops < PEAK_BF16_TFLOPS * 1.02
    assert not bool(torch.isnan(sink).any())
