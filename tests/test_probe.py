"""The memory-system probe library (liblaplex_probe.so, include/laplex_probe.h),
which the benchmark measures the operator's kernels against.  On the CPU: it
loads, exports what its header declares, and rejects bad arguments before any
launch.  On the GPU: each probe does what its header says, bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "laplex_probe.h")
LIB = os.path.join(ROOT, "laplace_prefix_scans_amd", "liblaplex_probe.so")
COPY_1, COPY_8, READ, WRITE, RUNS = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def P():
    if not os.path.exists(LIB):
        pytest.skip("liblaplex_probe.so not built")
    # torch first: the library's HIP symbols then bind to the runtime torch
    # loaded, which owns the device memory the GPU tests pass in
    import torch  # noqa: F401
    p = ctypes.CDLL(LIB)
    p.laplex_probe.restype = ctypes.c_int
    p.laplex_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    return p


def test_every_declared_symbol_is_exported(P):
    names = sorted(set(re.findall(r"\b(laplex_[a-z_]+)\s*\(", open(HEADER).read())))
    assert names == ["laplex_probe"]
    for name in names:
        assert hasattr(P, name), name


def test_host_argument_errors(P):
    src, dst = 0x100000, 0x200000  # never dereferenced: every call fails a check first
    assert P.laplex_probe(COPY_1, None, dst, 4096, None) == 1
    assert P.laplex_probe(COPY_1, src, None, 4096, None) == 1
    assert P.laplex_probe(COPY_1, src + 4, dst, 4096, None) == 3
    assert P.laplex_probe(WRITE, None, dst + 8, 4096, None) == 3
    assert P.laplex_probe(7, src, dst, 4096, None) == 9
    assert P.laplex_probe(-1, src, dst, 4096, None) == 9
    assert P.laplex_probe(COPY_8, src, dst, 4100, None) == 2
    assert P.laplex_probe(RUNS, src, dst, 4096, None) == 2  # not a whole 64 KiB tile
    assert P.laplex_probe(READ, src, dst, 0, None) == 0     # nothing to do


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 4096 * 3 + 48, 1 << 20, 5 << 20])
def test_probes_on_gpu(P, nbytes):
    import torch
    dev = torch.device("cuda:0")
    print("probe: %d bytes" % nbytes, flush=True)
    g = torch.Generator(device=dev).manual_seed(nbytes)
    x = torch.randn(nbytes // 4, device=dev, generator=g)
    s = torch.cuda.current_stream().cuda_stream
    for kind in (COPY_1, COPY_8):
        y = torch.full_like(x, float("nan"))
        assert P.laplex_probe(kind, x.data_ptr(), y.data_ptr(), nbytes, s) == 0
        torch.cuda.synchronize()
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), kind
    y = torch.zeros_like(x)
    assert P.laplex_probe(WRITE, None, y.data_ptr(), nbytes, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(y.view(-1, 4), torch.tensor([1.0, 2.0, 3.0, 4.0], device=dev).expand(nbytes // 16, 4))
    y = torch.zeros_like(x)
    assert P.laplex_probe(READ, x.data_ptr(), y.data_ptr(), nbytes, s) == 0
    torch.cuda.synchronize()
    chunks = (nbytes + 4095) // 4096
    xs = np.zeros(chunks * 1024, np.float64)
    xs[: nbytes // 4] = x.cpu().numpy()
    ref = xs.reshape(chunks, 1024).sum(axis=1)
    got = y[:chunks].cpu().numpy().astype(np.float64)
    scale = np.abs(xs).reshape(chunks, 1024).sum(axis=1)
    assert np.all(np.abs(got - ref) <= 1e-5 * scale + 1e-30)


@pytest.mark.gpu
@pytest.mark.parametrize("tiles", [1, 3, 40])
def test_runs_probe_on_gpu(P, tiles):
    import torch
    dev = torch.device("cuda:0")
    print("runs probe: %d tiles" % tiles, flush=True)
    nbytes = tiles * 8192 * 8
    x = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev)
    y = torch.zeros_like(x)
    assert P.laplex_probe(RUNS, x.data_ptr(), y.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    # pairs [tiles][256][32] -> [256][tiles][32]
    ref = x.view(tiles, 256, 32, 2).permute(1, 0, 2, 3).contiguous().view(-1)
    assert torch.equal(y, ref)
