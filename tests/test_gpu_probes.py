"""The measurement probes run through the C ABI: each launch completes,
records positive clock counts and leaves the sink unwritten."""
import pytest
import torch

from paged_kv_cache_04_amd import binding

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _ops():
    g = torch.Generator().manual_seed(3)
    return torch.randn(2048, generator=g).to(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("vec", [False, True])
@pytest.mark.parametrize("probe", ["mfma", "prefill_loop"])
def test_matrix_probes_run(probe, vec):
    print(f"[probe] {probe} vector_work={vec}", flush=True)
    ops = _ops()
    clocks = torch.zeros(2, dtype=torch.int64, device=DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    fn = binding.probe_mfma if probe == "mfma" else binding.probe_prefill_loop
    fn(ops, 20, vec, 16, clocks, sink)
    torch.cuda.synchronize()
    c = clocks.tolist()
    assert c[0] > 0 and c[1] > 0
    assert int(sink[0]) == 0


def test_read_probe_runs():
    print("[probe] read, sequential and 4 KiB blocks", flush=True)
    nbytes = 4 << 20
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=DEV)
    order = torch.randperm(nbytes // 4096).to(torch.int32).to(DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    binding.probe_read(buf, None, 4096, grid=64, sink=sink)
    binding.probe_read(buf, order, 4096, grid=64, sink=sink)
    torch.cuda.synchronize()
    assert int(sink[0]) == 0
