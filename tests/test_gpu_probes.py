"""The bandwidth probes behind the bench's peaks and the phase figures: each
reads exactly the bytes it is given. The read and phase probes leave one
uint32 per thread whose XOR over all threads is the XOR of every 32-bit word
read, whatever the split over threads; the copy probe copies."""

import ctypes
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def qg():
    import os

    import dequant_gemv_qgemv_amd as qg
    if not os.path.exists(qg.LIB_PATH):
        from dequant_gemv_qgemv_amd import build
        build.build()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qg.lib()
    yield qg


def xor_all(a):
    return int(np.bitwise_xor.reduce(np.ascontiguousarray(a).view(np.uint32).ravel()))


def words(n, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)


def test_read_and_copy_probes(qg):
    host = words(1 << 20, 1)  # 4 MiB
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    out = torch.empty(96 * 256, dtype=torch.int32, device=DEV)
    for cached in (False, True):
        qg.qg_probe_read(src, out, 96, cached=cached)
        torch.cuda.synchronize()
        assert xor_all(out.cpu().numpy()) == xor_all(host)
    dst = torch.empty_like(src)
    qg.qg_probe_copy(dst, src, 80)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


@pytest.mark.parametrize("barrier", [0, 1, 2])
def test_phase_probe_reads_every_range_once(qg, barrier):
    """Five ragged ranges (one clipped at the end of src), 48 workgroups:
    the XOR over the output is the XOR of the words in the ranges, without
    the barrier between them, with it, and with it and the next range's
    first loads issued before the wait; no barrier wait ran out."""
    print(f"phase probe barrier={barrier}", flush=True)
    sys.stdout.flush()
    n = 1 << 20
    host = words(n, 2)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    spans = [(0, 4096), (16384, 1 << 20), (8192, 16), (2 << 20, 123456 * 16), ((4 << 20) - 64, 4096)]
    ranges = torch.tensor([v for s in spans for v in s], dtype=torch.int64, device=DEV)
    blocks = 48
    out = torch.empty(blocks * 512, dtype=torch.int32, device=DEV)
    flags = torch.zeros(blocks, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    qg.qg_probe_phases(src, ranges, len(spans), barrier, out, blocks, flags, err)
    torch.cuda.synchronize()
    want = 0
    for off, nb in spans:
        nb = min(nb, 4 * n - off)  # clipped to src
        want ^= xor_all(host[off // 4:(off + nb) // 4])
    assert xor_all(out.cpu().numpy()) == want
    assert int(err.item()) == 0
    if barrier:
        assert np.all(flags.cpu().numpy() == len(spans) - 1)
