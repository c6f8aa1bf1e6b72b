"""The zero-allocation logits head: qlogits_topk_noalloc (scratch in a
library-held device array) against qlogits_topk (caller workspace), through
the C ABI, on two calls in a row, the second with a smaller input; also
inside a captured HIP graph replayed several times."""

import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-3


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


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def head(seed, V, K, norm):
    W = synth.qmat(seed, ("noalloc", V, K), V, K, 4)
    g = synth.norm_weight(seed, ("noalloc_g", K), K) if norm else None
    x = synth.activations(seed, ("noalloc_x", K), K, np.float32) * 4.0
    return W, g, x


def test_noalloc_matches_workspace_call_twice(qg):
    """Call 1: the Qwen-shaped head (151936 x 1024, top-40, final norm). Call 2:
    a smaller head (5000 x 256, top-8, no norm) on the same scratch. Each
    equals the workspace call bit for bit, its top-k equals the oracle's over
    the GPU logits, and its logits are within the bar of the oracle."""
    for (V, K, k, norm) in ((151936, 1024, 40, True), (5000, 256, 8, False)):
        say(f"noalloc logits V={V} K={K} k={k}")
        W, g, x = head(51, V, K, norm)
        Wd = qg.QMat.from_host(W, DEV)
        gd = None if g is None else to_dev(g)
        xd = to_dev(x)
        z1, i1, v1 = qg.qlogits_topk_noalloc(Wd, xd, k, gd, 1e-5)
        ws = qg.workspace(qg.QG_OP_LOGITS_TOPK, V, K, 1, 4, 0, k, DEV)
        z2, i2, v2 = qg.qlogits_topk(Wd, xd, k, gd, 1e-5, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(z1, z2) and torch.equal(i1, i2) and torch.equal(v1, v2)
        zc = z1.cpu().numpy()
        ridx, rvals = oracle.topk(zc, k)
        assert np.array_equal(i1.cpu().numpy(), ridx)
        assert np.array_equal(v1.cpu().numpy(), rvals.astype(np.float32))
        rows = np.unique(np.concatenate([[0, V - 1], np.random.default_rng(0).choice(V, 200)]))
        Wr = dict(W, N=len(rows), q=W["q"][rows], scales=W["scales"][rows], biases=W["biases"][rows])
        ref = oracle.gemv(Wr, oracle.rmsnorm(x, g, 1e-5) if norm else x)
        err = np.max(np.abs(zc[rows] - ref))
        assert err <= TOL * np.max(np.abs(ref)), err


def test_noalloc_in_a_replayed_graph(qg):
    """Captured (no allocation inside the capture) and replayed three times,
    with eager calls in between: every replay equals the eager result."""
    V, K, k = 20000, 512, 40
    W, g, x = head(52, V, K, True)
    Wd = qg.QMat.from_host(W, DEV)
    gd, xd = to_dev(g), to_dev(x)
    z = torch.empty(V, dtype=torch.float32, device=DEV)
    idx = torch.empty(k, dtype=torch.int32, device=DEV)
    vals = torch.empty(k, dtype=torch.float32, device=DEV)
    qg.qlogits_topk_noalloc(Wd, xd, k, gd, 1e-5, logits=z, idx=idx, vals=vals)
    torch.cuda.synchronize()
    e_idx, e_vals = idx.clone(), vals.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        qg.qlogits_topk_noalloc(Wd, xd, k, gd, 1e-5, logits=z, idx=idx, vals=vals)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qg.qlogits_topk_noalloc(Wd, xd, k, gd, 1e-5, logits=z, idx=idx, vals=vals)
    for rep in range(3):
        idx.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, e_idx) and torch.equal(vals, e_vals), f"replay {rep}"
        qg.qlogits_topk_noalloc(Wd, xd, k, gd, 1e-5, logits=z, idx=idx, vals=vals)
        torch.cuda.synchronize()
        assert torch.equal(idx, e_idx)


def test_noalloc_refuses_beyond_its_scratch(qg):
    """A vocabulary whose workspace need exceeds the 24 MiB array is refused
    by the host-side check before anything is enqueued."""
    V, K, k = 600000, 64, 40
    need = qg.qg_workspace_bytes(qg.QG_OP_LOGITS_TOPK, V, K, 1, 4, 0, k)
    assert need > 24 << 20
    q = torch.zeros((V, K // 8), dtype=torch.int32, device=DEV)
    s = torch.zeros((V, 1), dtype=torch.int16, device=DEV)
    Wd = qg.QMat(q, s, s, N=V, K=K, bits=4)
    x = torch.zeros(K, dtype=torch.float32, device=DEV)
    with pytest.raises(qg.QgError) as ei:
        qg.qlogits_topk_noalloc(Wd, x, k)
    assert ei.value.status == qg.QG_EUNSUPPORTED
