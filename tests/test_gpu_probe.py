"""The library's streaming read probe (measurement helper): it runs, and rejects bad
sizes and alignment through the C-ABI."""
import pytest

from prefix_shared_kv_radix_amd import _lib

from conftest import gpu_available


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


@pytest.mark.gpu
def test_read_probe_runs_and_checks_arguments():
    import torch
    x = torch.ones(16 << 20, dtype=torch.int32, device="cuda")   # 64 MiB
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    _lib.probe_read(x, sink)
    torch.cuda.synchronize()
    assert int(sink.sum()) == 0   # XOR of the ones is 0, never the constant
    st = _lib.load().radix_probe_read(_lib._ptr(x), 24, _lib._ptr(sink), None)
    assert st != 0   # not a multiple of 16 bytes
    st = _lib.load().radix_probe_read(_lib._ptr(x[1:]), 16, _lib._ptr(sink), None)
    assert st != 0   # misaligned
