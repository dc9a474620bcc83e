"""The benchmark's throughput probes (libsparge_probe.so): exports and
argument checks on the CPU, one small launch of each kind on the GPU."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_sparge_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparge_probe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.PROBE_LIB):
        pytest.fail(f"{build.PROBE_LIB} is missing: run the build first")
    lib = ctypes.CDLL(build.PROBE_LIB)
    lib.sparge_probe_launch.restype = ctypes.c_int
    lib.sparge_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.sparge_probe_flops.restype = ctypes.c_double
    lib.sparge_probe_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    return lib


def test_probe_library_exports_every_declared_function(lib):
    names = re.findall(r"^\w[\w\s\*]*?\b(sparge_\w+)\(", open(HEADER).read(), re.M)
    assert set(names) == {"sparge_probe_launch", "sparge_probe_flops"}
    for n in names:
        assert hasattr(lib, n), n


def test_probe_flops(lib):
    assert lib.sparge_probe_flops(768, 2000) == 768 * 4 * 2000 * 16 * 32768


@pytest.mark.parametrize("kind, wg, iters, out", [
    (2, 8, 10, 1), (-1, 8, 10, 1),          # unknown kind
    (0, 0, 10, 1), (1, 65537, 10, 1),       # workgroups out of range
    (0, 8, 0, 1), (1, 8, 1000001, 1),       # iterations out of range
    (0, 8, 10, 0),                          # no output buffer
])
def test_probe_rejects_bad_arguments(lib, kind, wg, iters, out):
    # hipErrorInvalidValue (1), returned before any HIP call.
    assert lib.sparge_probe_launch(kind, wg, iters, ctypes.c_void_p(out), None) == 1


@pytest.mark.gpu
@pytest.mark.parametrize("kind", [0, 1])
def test_probe_runs(lib, kind):
    import torch
    wg = 16
    out = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device="cuda")
    rc = lib.sparge_probe_launch(kind, wg, 50, ctypes.c_void_p(out.data_ptr()),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
