"""The measurement probes (patch_probe_*) run to completion on the GPU and
report what they moved: they compute nothing of the method and are checked
for completion, byte and flop counts and plausible rates only."""
import pytest
import torch

from sparse_gemm_amd import patch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    patch.load()


def _timed(fn):
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    r = fn()
    b.record()
    torch.cuda.synchronize()
    return r, a.elapsed_time(b) * 1e-3


def test_probe_copy_rate_counts_and_rates():
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(4 * ncu, dtype=torch.uint8, device="cuda")
    src = torch.ones(64 << 20, dtype=torch.uint8, device="cuda")
    for nbytes, win in ((4 << 20, 256 << 10), (64 << 20, 256 << 10)):
        view = src[:nbytes]
        patch.probe_copy_rate(view, win, 5, ncu, sink)
        nb, t = _timed(lambda: patch.probe_copy_rate(view, win, 200, ncu, sink))
        assert nb == 7 * 8 * 1024 * 200 * ncu
        rate = nb / t / 1e12
        # between what one CU's copies could never drop below and far above
        # any L2 of this class of device
        assert 0.5 < rate < 200, (nbytes, rate)
    assert int(sink.sum()) == 0  # the guarded store never fires on these bytes


def test_probe_stream_read_and_matrix_rate():
    sink = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    buf = torch.ones(32 << 20, dtype=torch.uint8, device="cuda")
    patch.probe_stream_read(buf, sink)
    _, t = _timed(lambda: patch.probe_stream_read(buf, sink))
    assert 0.1 < buf.numel() / t / 1e12 < 100
    for kind in range(4):
        flops, t = _timed(lambda: patch.probe_matrix_rate(kind, 64, 256, sink))
        assert flops > 0 and t > 0
